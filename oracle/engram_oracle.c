/*
 * CPU oracle for the Engram forward path -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct host implementation of what the path
 * computes, written from the DeepSeek V4.1 model pages
 * (open-model-atlas "stack-hashes" page and its duplicates on the
 * atlas.klimoza.dev "engram-first/lookup" and "engram-first/streams" pages):
 *
 *   hash         -- the engram hash module's forward (stack-hashes page)
 *   gather+dequant -- ParallelEngramEmbedding.forward
 *   wkv          -- the `wkv` Linear of Engram.forward
 *   gate dot     -- Engram.forward up to the gate pre-activation `dot`
 *   gate output  -- the rest of Engram.forward: signed-sqrt sigmoid gate,
 *                   masked positions shut, residual add of the gated value
 *
 * Only tests, the smoke entry point and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header, table or constant with the
 * HIP library: it includes nothing but the C standard library.
 *
 * Floating point: the dequant follows the pages' precision exactly (fp32
 * product, then bf16), everything else is accumulated in double.  Built with
 * -ffp-contract=off so no multiply-add is fused behind the source's back.
 *
 * Parity pins (tests/test_oracle_*.py): the hash against a Python big-int
 * brute force and against invariants the pages state; the decode against
 * torch's float8_e4m3fn for all 256 bytes; bf16 rounding against torch; the
 * projection against numpy's float64 matmul; the gate dot, gate and output on
 * hand-built vectors with closed-form results.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#include "engram_oracle.h"

/* ------------------------------------------------------------------------ */
/* step 1: hash                                                              */
/* ------------------------------------------------------------------------ */

/* torch's `%` on int64 takes the sign of the divisor (floor modulo). */
static int64_t floor_mod(int64_t a, int64_t p) {
    int64_t r = a % p; /* C truncates toward zero */
    if (r != 0 && ((r < 0) != (p < 0))) r += p;
    return r;
}

/* int64 product with two's-complement wrap, as torch's int64 `*` does. */
static int64_t wrap_mul(int64_t a, int64_t b) {
    return (int64_t)((uint64_t)a * (uint64_t)b);
}

int oracle_hash(const int64_t* input_ids, int64_t B, int64_t L, int64_t start_pos,
                const uint8_t* token_mask, const int64_t* token_map, int64_t vocab,
                int64_t* cache, int64_t cache_B, int64_t cache_L,
                const int64_t* multipliers, const int64_t* primes, const int64_t* offsets,
                int E, int N, int H, int64_t pad_id, int64_t dead, int64_t* hash_ids) {
    if (B < 0 || L < 0 || start_pos < 0 || E < 1 || N < 2 || H < 1) return ORACLE_EINVAL;
    if (B > cache_B || start_pos + L > cache_L) return ORACLE_ERANGE;
    const int C = (N - 1) * H;

    /* compressed = token_map[input_ids]; masked -> DEAD; write the cache.
     * (An id outside the vocabulary is treated like a masked token.) */
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t l = 0; l < L; ++l) {
            int64_t id = input_ids[b * L + l];
            int64_t c = (id >= 0 && id < vocab) ? token_map[id] : dead;
            if (token_mask && !token_mask[b * L + l]) c = dead;
            cache[b * cache_L + start_pos + l] = c;
        }
    }

    int64_t* tokens = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    int64_t* products = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    if (!tokens || !products) { free(tokens); free(products); return ORACLE_ENOMEM; }

    for (int64_t b = 0; b < B; ++b) {
        for (int64_t l = 0; l < L; ++l) {
            const int64_t p = start_pos + l;
            /* one lookback at a time; once a slot is blocked (before the start of
             * the sequence, or a masked source) every longer lookback is too */
            int blocked = 0;
            for (int s = 0; s < N; ++s) {
                int64_t q = p - s;
                if (q < 0) q = 0;
                int64_t source = cache[b * cache_L + q];
                if (p < s || source == dead) blocked = 1;
                tokens[s] = blocked ? pad_id : source;
            }
            int64_t* out = hash_ids + (b * L + l) * (int64_t)E * C;
            for (int e = 0; e < E; ++e) {
                for (int s = 0; s < N; ++s) products[s] = wrap_mul(tokens[s], multipliers[e * N + s]);
                /* after XOR-ing lookback i the running value is the (i+1)-gram hash */
                int64_t rolling = products[0];
                for (int i = 1; i < N; ++i) {
                    rolling ^= products[i];
                    for (int h = 0; h < H; ++h) {
                        const int col = (i - 1) * H + h;
                        const int64_t prime = primes[((int64_t)e * (N - 1) + (i - 1)) * H + h];
                        out[e * C + col] = floor_mod(rolling, prime) + offsets[e * C + col];
                    }
                }
            }
        }
    }
    free(tokens);
    free(products);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* step 2+3: gather and block dequant                                        */
/* ------------------------------------------------------------------------ */

/* float8_e4m3fn from the OCP 8-bit floating point definition: 1 sign bit,
 * 4 exponent bits (bias 7), 3 mantissa bits, no infinities, S.1111.111 = NaN. */
float oracle_e4m3fn_decode(uint8_t byte) {
    const int sign = byte >> 7;
    const int expo = (byte >> 3) & 0xF;
    const int mant = byte & 0x7;
    float v;
    if (expo == 0xF && mant == 0x7) return NAN;
    if (expo == 0)
        v = ldexpf((float)mant, -9);              /* subnormal: m * 2^-6 / 8 */
    else
        v = ldexpf((float)(8 + mant), expo - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* float -> bfloat16 bit pattern, round to nearest, ties to even. */
uint16_t oracle_bf16_rne(float f) {
    uint32_t u = f32_bits(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) /* NaN: keep sign, quiet it */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16, rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
    return (uint16_t)keep;
}

int oracle_gather_dequant(const int64_t* hash_ids, int64_t T, int64_t id_token_stride, int C,
                          const uint8_t* weight, const float* scale, int64_t R, int64_t row_start,
                          int D, int blk, uint16_t* out_bf16, uint8_t* out_fp8, float* out_scale) {
    if (T < 0 || C < 1 || D < 1 || blk < 1 || D % blk != 0 || R < 1) return ORACLE_EINVAL;
    const int S = D / blk;
    const int64_t vocab_end = row_start + R;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int c = 0; c < C; ++c) {
            const int64_t idx = hash_ids[t * id_token_stride + c];
            const int masked = idx < row_start || idx >= vocab_end;
            const int64_t local = masked ? 0 : idx - row_start;
            const uint8_t* w = weight + local * D;
            const float* sc = scale + local * S;
            const int64_t o = (t * C + c);
            for (int j = 0; j < D; ++j) {
                /* fp32 product (one rounding) then bf16 (a second rounding) */
                float prod = oracle_e4m3fn_decode(w[j]) * sc[j / blk];
                out_bf16[o * D + j] = masked ? 0 : oracle_bf16_rne(prod);
                if (out_fp8) out_fp8[o * D + j] = w[j];
            }
            if (out_scale)
                for (int s = 0; s < S; ++s) out_scale[o * S + s] = sc[s];
        }
    }
    return ORACLE_OK;
}

/* The same gather and dequant with the table's block scales in one of the formats `scale_dtype` may name
 * (the stack-hashes page leaves it open): 0 = float32, 1 = E8M0 (one byte, 2^(s-127), 0xFF NaN), 2 =
 * float8_e4m3fn (one byte); `scales.float()` is the decoded value, and the dequant is again the fp32
 * product, then bf16.  Ids are int64 (id_bytes 8) or int32 (id_bytes 4).  out_scale (optional) receives
 * the gathered scale elements as stored (4 or 1 bytes each). */
int oracle_gather_dequant_fmt(const void* hash_ids, int id_bytes, int64_t T, int64_t id_token_stride, int C,
                              const uint8_t* weight, const void* scale, int scale_format, int64_t R,
                              int64_t row_start, int D, int blk, uint16_t* out_bf16, uint8_t* out_fp8,
                              void* out_scale) {
    if (T < 0 || C < 1 || D < 1 || blk < 1 || D % blk != 0 || R < 1) return ORACLE_EINVAL;
    if ((id_bytes != 4 && id_bytes != 8) || scale_format < 0 || scale_format > 2) return ORACLE_EINVAL;
    const int S = D / blk;
    const int sbytes = scale_format == 0 ? 4 : 1;
    const int64_t vocab_end = row_start + R;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int c = 0; c < C; ++c) {
            const int64_t at = t * id_token_stride + c;
            const int64_t idx = id_bytes == 8 ? ((const int64_t*)hash_ids)[at] : (int64_t)((const int32_t*)hash_ids)[at];
            const int masked = idx < row_start || idx >= vocab_end;
            const int64_t local = masked ? 0 : idx - row_start;
            const uint8_t* w = weight + local * D;
            const int64_t o = (t * C + c);
            for (int j = 0; j < D; ++j) {
                const int64_t si = local * S + j / blk;
                float sv;
                if (scale_format == 0)
                    sv = ((const float*)scale)[si];
                else if (scale_format == 1)
                    sv = (float)oracle_e8m0_decode(((const uint8_t*)scale)[si]);
                else
                    sv = oracle_e4m3fn_decode(((const uint8_t*)scale)[si]);
                /* fp32 product (one rounding) then bf16 (a second rounding) */
                const float prod = oracle_e4m3fn_decode(w[j]) * sv;
                out_bf16[o * D + j] = masked ? (uint16_t)0 : oracle_bf16_rne(prod);
                if (out_fp8) out_fp8[o * D + j] = w[j];
            }
            if (out_scale)
                memcpy((uint8_t*)out_scale + o * S * sbytes, (const uint8_t*)scale + local * S * sbytes,
                       (size_t)(S * sbytes));
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* step 4: wkv projection                                                    */
/* ------------------------------------------------------------------------ */

double oracle_bf16_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

int oracle_wkv(const uint16_t* a, const uint16_t* w, double* kv, int64_t T, int K, int Nout) {
    if (T < 0 || K < 1 || Nout < 1) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int o = 0; o < Nout; ++o) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += oracle_bf16_to_double(a[t * K + k]) * oracle_bf16_to_double(w[(int64_t)o * K + k]);
            kv[t * Nout + o] = acc;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* step 4, fp8 block-scaled form: the `wkv` Linear under the released         */
/* config's "dtype": "fp8"                                                   */
/* ------------------------------------------------------------------------ */
/* Reading (the pages name the fp8 Linear but do not show it): weights and
 * inputs in the OCP microscaling (MX) fp8 format -- E4M3FN elements in blocks
 * of 32 consecutive input columns of a row, each block with one E8M0 scale,
 * the block-32/E8M0 format the pages name for the indexer's quantised
 * activations.  The input rows are quantised to it by the OCP MX rule; the
 * product accumulates scale_a * scale_w * sum(a * w) over the blocks. */

/* E8M0: eight exponent bits, bias 127, no sign and no mantissa; 0xFF is NaN. */
double oracle_e8m0_decode(uint8_t s) {
    if (s == 0xFF) return NAN;
    return ldexp(1.0, (int)s - 127);
}

/* Round half to even of a non-negative double (the quotient by the quantum is exact). */
static double round_half_even(double n) {
    const double fl = floor(n);
    const double frac = n - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) return fl + 1.0;
    return fl;
}

/* A finite double -> float8_e4m3fn byte: round to nearest, ties to even, on the E4M3 grid (subnormal
 * quantum 2^-9 below 2^-6, 3 mantissa bits above), magnitudes past the largest finite value 448
 * saturated to 448; the sign is kept (-0 -> 0x80); NaN -> 0x7F. */
uint8_t oracle_e4m3fn_encode_sat(double v) {
    if (isnan(v)) return 0x7F;
    const uint8_t sign = signbit(v) ? 0x80 : 0x00;
    const double m = fabs(v);
    if (m >= 448.0) return sign | 0x7E;
    if (m < ldexp(1.0, -6)) {                      /* subnormal: n * 2^-9, n in [0, 8] */
        const int n = (int)round_half_even(m / ldexp(1.0, -9));
        return sign | (uint8_t)n;                   /* n == 8 is the smallest normal, code 0x08 */
    }
    int e;
    frexp(m, &e);                                   /* m = f * 2^e, f in [0.5, 1): floor(log2 m) = e - 1 */
    e -= 1;
    double n = round_half_even(m / ldexp(1.0, e - 3));  /* in [8, 16] */
    if (n == 16.0) { n = 8.0; e += 1; }
    if (e > 8 || (e == 8 && n > 14.0)) return sign | 0x7E; /* rounds past 448 */
    return sign | (uint8_t)(((e + 7) << 3) | ((int)n - 8));
}

/* OCP MX quantisation of bf16 rows: for row r and block b of `blk` columns, with amax the largest
 * magnitude in the block, the shared exponent is floor(log2(amax)) - 8 (8 = the largest exponent of
 * E4M3), kept within the E8M0 range [-127, 127] (an all-zero block takes -127); scale[r, b] = that
 * exponent + 127, and q[r, k] = e4m3_sat(x[r, k] / 2^exponent).  Inputs must be finite. */
int oracle_mx_quant(const uint16_t* x, int64_t rows, int K, int blk, uint8_t* q, uint8_t* scale) {
    if (rows < 0 || K < 1 || blk < 1 || K % blk != 0) return ORACLE_EINVAL;
    const int nb = K / blk;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int b = 0; b < nb; ++b) {
            const uint16_t* xb = x + r * K + (int64_t)b * blk;
            double amax = 0.0;
            for (int k = 0; k < blk; ++k) amax = fmax(amax, fabs(oracle_bf16_to_double(xb[k])));
            int shared = -127;
            if (amax > 0.0) {
                int e;
                frexp(amax, &e);
                shared = (e - 1) - 8;
                if (shared < -127) shared = -127;
                if (shared > 127) shared = 127;
            }
            scale[r * nb + b] = (uint8_t)(shared + 127);
            for (int k = 0; k < blk; ++k)
                q[r * K + (int64_t)b * blk + k] = oracle_e4m3fn_encode_sat(ldexp(oracle_bf16_to_double(xb[k]), -shared));
        }
    }
    return ORACLE_OK;
}

/* The block-scaled projection: kv[t,o] = sum over blocks b of
 * e8m0(a_s[t,b]) * e8m0(w_s[o,b]) * sum_{k in b} e4m3(a_q[t,k]) * e4m3(w_q[o,k]), in double. */
int oracle_wkv_mx(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w_q, const uint8_t* w_s, double* kv,
                  int64_t T, int K, int Nout, int blk) {
    if (T < 0 || K < 1 || Nout < 1 || blk < 1 || K % blk != 0) return ORACLE_EINVAL;
    const int nb = K / blk;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int o = 0; o < Nout; ++o) {
            double acc = 0.0;
            for (int b = 0; b < nb; ++b) {
                double part = 0.0;
                for (int k = b * blk; k < (b + 1) * blk; ++k)
                    part += (double)oracle_e4m3fn_decode(a_q[t * K + k]) * (double)oracle_e4m3fn_decode(w_q[(int64_t)o * K + k]);
                acc += oracle_e8m0_decode(a_s[t * nb + b]) * oracle_e8m0_decode(w_s[(int64_t)o * nb + b]) * part;
            }
            kv[t * Nout + o] = acc;
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* step 5: gate pre-activation                                               */
/* ------------------------------------------------------------------------ */

int oracle_gate_dot(const uint16_t* x, const uint16_t* kv, int64_t ld_kv, const uint16_t* q_weight,
                    const uint16_t* k_weight, double eps, double* dot, int64_t T, int hc, int dim) {
    if (T < 0 || hc < 1 || dim < 1 || ld_kv < (int64_t)hc * dim) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int c = 0; c < hc; ++c) {
            const uint16_t* h = x + (t * hc + c) * (int64_t)dim;
            const uint16_t* key = kv + t * ld_kv + (int64_t)c * dim;
            double hh = 0.0, kk = 0.0, hwk = 0.0;
            for (int j = 0; j < dim; ++j) {
                const double hv = oracle_bf16_to_double(h[j]);
                const double kv_ = oracle_bf16_to_double(key[j]);
                /* the two weights are only ever used as their product */
                const double wv = oracle_bf16_to_double(q_weight[c * dim + j]) *
                                  oracle_bf16_to_double(k_weight[c * dim + j]);
                hh += hv * hv;
                kk += kv_ * kv_;
                hwk += hv * wv * kv_;
            }
            /* normalised per (token, copy) over dim, not jointly over the copies */
            const double rstd = (1.0 / sqrt(hh / dim + eps)) * (1.0 / sqrt(kk / dim + eps));
            dot[t * hc + c] = hwk * rstd / sqrt((double)dim);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* gate activation, mask and residual                                        */
/* ------------------------------------------------------------------------ */

/* The end of Engram.forward on the stack-hashes page: the gate is the sigmoid
 * of the signed square root of the dot, with |dot| clamped from below at 1e-6
 * first (so a zero dot still gives sigmoid(+-1e-3), its sign taken from the
 * dot, -0 included); a token whose mask entry is false gets gate 0; the output
 * adds the gated value, which all hc copies share, to each copy of the stream:
 *     out[t,c,j] = h[t,c,j] + gate[t,c] * value[t,j],  value = kv[t, hc*dim + j].
 * dot [T,hc] is an input (the oracle's own, or the device's for a unit check);
 * token_mask [T] (nonzero = takes part) or NULL; gate [T,hc] and out
 * [T,hc,dim] are double. */
int oracle_gate_output(const uint16_t* x, const uint16_t* kv, int64_t ld_kv, const double* dot,
                       const uint8_t* token_mask, double* gate, double* out, int64_t T, int hc, int dim) {
    if (T < 0 || hc < 1 || dim < 1 || ld_kv < (int64_t)(hc + 1) * dim) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t* value = kv + t * ld_kv + (int64_t)hc * dim;
        for (int c = 0; c < hc; ++c) {
            const double d = dot[t * hc + c];
            const double mag = sqrt(fmax(fabs(d), 1e-6));
            const double z = copysign(mag, d);
            double g = 1.0 / (1.0 + exp(-z));
            if (token_mask && !token_mask[t]) g = 0.0;
            gate[t * hc + c] = g;
            const uint16_t* h = x + (t * hc + c) * (int64_t)dim;
            double* o = out + (t * hc + c) * (int64_t)dim;
            for (int j = 0; j < dim; ++j)
                o[j] = oracle_bf16_to_double(h[j]) + g * oracle_bf16_to_double(value[j]);
        }
    }
    return ORACLE_OK;
}

/* Threads the parallel loops above use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the threads of the parallel loops above (a no-op without OpenMP). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
