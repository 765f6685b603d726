// engram_gate_dot: the gate pre-activation per (token, hc copy).
// engram_gate_output: the same dot, then the gate, the mask and the residual.
// engram_gate_residual: the gate, the mask and the residual from a given dot.
//
// Computes, from Engram.forward on the DeepSeek V4.1 "stack-hashes" page,
// the per-copy weight product q_weight * k_weight, the two RMS factors of
// the stream copy and of its key (each over `dim`, per copy, not jointly over
// the copies), and dot = sum(h * w * key) * rstd * dim^-1/2.
//
// Design (gfx950): HBM-bound streaming reduction.  Rows that cross HBM once (the stream copies, the keys,
// the output) use non-temporal loads and stores, leaving L2 to what is re-read (the value row, q and k).  One wave per 4 tokens of
// one copy: every lane streams 16-byte pieces (8 bf16) of the 4 stream rows
// and 4 key rows (8 loads in flight per lane and step), widens them to fp32,
// multiplies by the weight product (the copy's q and k pieces are loaded once
// for the 4 tokens; they stay in L2) and keeps three fp32 partial sums per
// token.  A wave-wide butterfly finishes the sums; lane 0 applies the two
// reciprocal square roots and writes one fp32 per token.  Launches with
// fewer such waves than four per CU (a decode call) instead give each
// (token, copy) a workgroup whose four waves split the row.
//
// engram_gate_output finishes the module (the end of Engram.forward): gate =
// sigmoid(signed sqrt of max(|dot|, 1e-6)), 0 for masked tokens, and out =
// bf16(h + gate * value) with the value row shared by the hc copies.  One wave
// per (2 tokens, copy); the wave's stream pieces and value pieces are loaded
// once into registers up front, the dot is reduced as above, and the output
// is written from the registers: x, key and value each cross HBM once, out is
// written once (the value row is re-read by the hc waves of a token from L2).
// Small launches split each row over a workgroup, as the dot does.
#include "common.h"

namespace engram {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTok = 4;  // tokens per wave: the copy's q/k chunks are loaded once for all of them
// below this many (4-token, copy) waves -- four per CU -- the dot splits each row over a workgroup
constexpr int64_t kSplitBelowWaves = 1024;

struct GateArgs {
    const uint16_t* x;
    const uint16_t* kv;
    int64_t ld_kv;
    const uint16_t* q;
    const uint16_t* k;
    float eps;
    float inv_dim;       // 1/dim
    float rsqrt_dim;     // dim^-1/2
    float* dot;
    int64_t T;
    int64_t groups;      // ceil(T / kTok) * hc
    int hc, dim;
};

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// One wave per (group of kTok tokens, copy c).
__global__ __launch_bounds__(kThreads) void gate_dot_kernel(GateArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t group = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (group >= a.groups) return;
    const int c = static_cast<int>(group % a.hc);
    const int64_t t0 = (group / a.hc) * kTok;
    const int ntok = static_cast<int>(min<int64_t>(kTok, a.T - t0));
    const u32x4* q = reinterpret_cast<const u32x4*>(a.q + static_cast<int64_t>(c) * a.dim);
    const u32x4* k = reinterpret_cast<const u32x4*>(a.k + static_cast<int64_t>(c) * a.dim);
    const u32x4* h[kTok];
    const u32x4* key[kTok];
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
        const int64_t t = t0 + min(u, ntok - 1);  // ragged tail: repeat the last token, never written
        h[u] = reinterpret_cast<const u32x4*>(a.x + (t * a.hc + c) * a.dim);
        key[u] = reinterpret_cast<const u32x4*>(a.kv + t * a.ld_kv + static_cast<int64_t>(c) * a.dim);
    }
    const int chunks = a.dim / 8;

    float hh[kTok], kk[kTok], hwk[kTok];
#pragma unroll
    for (int u = 0; u < kTok; ++u) hh[u] = kk[u] = hwk[u] = 0.f;
    for (int j = lane; j < chunks; j += 64) {
        const u32x4 qv = q[j], kw = k[j];
        u32x4 hv[kTok], kv[kTok];
#pragma unroll
        for (int u = 0; u < kTok; ++u) {
            hv[u] = __builtin_nontemporal_load(h[u] + j);  // stream and key rows are read once
            kv[u] = __builtin_nontemporal_load(key[u] + j);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float w0 = lo_bf16(qv[i]) * lo_bf16(kw[i]);  // exact: bf16 * bf16 fits fp32
            const float w1 = hi_bf16(qv[i]) * hi_bf16(kw[i]);
#pragma unroll
            for (int u = 0; u < kTok; ++u) {
                const float h0 = lo_bf16(hv[u][i]), h1 = hi_bf16(hv[u][i]);
                const float k0 = lo_bf16(kv[u][i]), k1 = hi_bf16(kv[u][i]);
                hh[u] += h0 * h0 + h1 * h1;
                kk[u] += k0 * k0 + k1 * k1;
                hwk[u] += h0 * w0 * k0 + h1 * w1 * k1;
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
        const float shh = wave_sum(hh[u]), skk = wave_sum(kk[u]), shwk = wave_sum(hwk[u]);
        if (lane == 0 && u < ntok) {
            const float rstd = rsqrtf(shh * a.inv_dim + a.eps) * rsqrtf(skk * a.inv_dim + a.eps);
            a.dot[(t0 + u) * a.hc + c] = shwk * rstd * a.rsqrt_dim;
        }
    }
}

// Small launches (a decode call: 256 tokens x 4 copies is 256 waves above, one per CU): one workgroup per
// (token, copy), its four waves taking every fourth 64-piece stretch of the row; each wave's three sums go
// through LDS and wave 0 adds the four in wave order.
__global__ __launch_bounds__(kThreads) void gate_dot_split_kernel(GateArgs a) {
    __shared__ float part[kWaves][3];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t tc = blockIdx.x;  // token * hc + copy
    const int c = static_cast<int>(tc % a.hc);
    const int64_t t = tc / a.hc;
    const u32x4* q = reinterpret_cast<const u32x4*>(a.q + static_cast<int64_t>(c) * a.dim);
    const u32x4* k = reinterpret_cast<const u32x4*>(a.k + static_cast<int64_t>(c) * a.dim);
    const u32x4* h = reinterpret_cast<const u32x4*>(a.x + tc * a.dim);
    const u32x4* key = reinterpret_cast<const u32x4*>(a.kv + t * a.ld_kv + static_cast<int64_t>(c) * a.dim);
    const int chunks = a.dim / 8;
    float hh = 0.f, kk = 0.f, hwk = 0.f;
    for (int j = w * 64 + lane; j < chunks; j += kThreads) {
        const u32x4 qv = q[j], kw = k[j], hv = h[j], kv = key[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float w0 = lo_bf16(qv[i]) * lo_bf16(kw[i]);  // exact: bf16 * bf16 fits fp32
            const float w1 = hi_bf16(qv[i]) * hi_bf16(kw[i]);
            const float h0 = lo_bf16(hv[i]), h1 = hi_bf16(hv[i]);
            const float k0 = lo_bf16(kv[i]), k1 = hi_bf16(kv[i]);
            hh += h0 * h0 + h1 * h1;
            kk += k0 * k0 + k1 * k1;
            hwk += h0 * w0 * k0 + h1 * w1 * k1;
        }
    }
    hh = wave_sum(hh);
    kk = wave_sum(kk);
    hwk = wave_sum(hwk);
    if (lane == 0) {
        part[w][0] = hh;
        part[w][1] = kk;
        part[w][2] = hwk;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float shh = 0.f, skk = 0.f, shwk = 0.f;
#pragma unroll
        for (int v = 0; v < kWaves; ++v) {
            shh += part[v][0];
            skk += part[v][1];
            shwk += part[v][2];
        }
        const float rstd = rsqrtf(shh * a.inv_dim + a.eps) * rsqrtf(skk * a.inv_dim + a.eps);
        a.dot[tc] = shwk * rstd * a.rsqrt_dim;
    }
}

// ---------------------------------------------------------------------------
// gate activation, mask and residual
// ---------------------------------------------------------------------------
struct OutArgs {
    const uint16_t* x;
    const uint16_t* kv;
    int64_t ld_kv;
    const uint16_t* q;
    const uint16_t* k;
    const uint8_t* mask;  // [T] or null
    float eps;
    float inv_dim;
    float rsqrt_dim;
    uint16_t* out;
    float* dot;           // [T, hc] or null
    int64_t T;
    int64_t groups;       // ceil(T / TOK) * hc
    int hc, dim;
};

__device__ inline uint32_t pack2_bf16(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

// h + gate * v as two fp32 roundings (the product, then the sum), then bf16: the pages form the
// gated value first and add it to the stream, so no fused multiply-add here
__device__ inline u32x4 residual(const u32x4 h, const u32x4 v, float gate) {
#pragma clang fp contract(off)
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float g0 = gate * lo_bf16(v[i]);
        const float g1 = gate * hi_bf16(v[i]);
        o[i] = pack2_bf16(lo_bf16(h[i]) + g0, hi_bf16(h[i]) + g1);
    }
    return o;
}

// sigmoid of the signed square root; |dot| is clamped from below at 1e-6 first
__device__ inline float gate_of(float d) {
    const float z = copysignf(sqrtf(fmaxf(fabsf(d), 1e-6f)), d);
    return 1.0f / (1.0f + expf(-z));
}

// One wave per (TOK tokens, copy c); lane l owns the 16-byte pieces l, l + 64, ... (P of them) of
// each row, which stay in registers from the first load to the output store.
template <int P, int TOK>
__global__ __launch_bounds__(kThreads) void gate_output_kernel(OutArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t group = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    if (group >= a.groups) return;
    const int c = static_cast<int>(group % a.hc);
    const int64_t t0 = (group / a.hc) * TOK;
    const int ntok = static_cast<int>(min<int64_t>(TOK, a.T - t0));
    const int chunks = a.dim / 8;
    const u32x4* q = reinterpret_cast<const u32x4*>(a.q + static_cast<int64_t>(c) * a.dim);
    const u32x4* k = reinterpret_cast<const u32x4*>(a.k + static_cast<int64_t>(c) * a.dim);
    const u32x4* h[TOK];
    const u32x4* key[TOK];
    const u32x4* val[TOK];
    u32x4* out[TOK];
    int64_t tok[TOK];
#pragma unroll
    for (int u = 0; u < TOK; ++u) {
        tok[u] = t0 + min(u, ntok - 1);  // ragged tail: repeat the last token, never written
        const uint16_t* row = a.kv + tok[u] * a.ld_kv;
        h[u] = reinterpret_cast<const u32x4*>(a.x + (tok[u] * a.hc + c) * a.dim);
        key[u] = reinterpret_cast<const u32x4*>(row + static_cast<int64_t>(c) * a.dim);
        val[u] = reinterpret_cast<const u32x4*>(row + static_cast<int64_t>(a.hc) * a.dim);
        out[u] = reinterpret_cast<u32x4*>(a.out + (tok[u] * a.hc + c) * a.dim);
    }

    u32x4 hr[TOK][P], vr[TOK][P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int j = lane + 64 * i;
        if (j < chunks) {
#pragma unroll
            for (int u = 0; u < TOK; ++u) {
                hr[u][i] = __builtin_nontemporal_load(h[u] + j);  // read once; the value row is shared by the copies
                vr[u][i] = val[u][j];
            }
        }
    }

    float hh[TOK], kk[TOK], hwk[TOK];
#pragma unroll
    for (int u = 0; u < TOK; ++u) hh[u] = kk[u] = hwk[u] = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int j = lane + 64 * i;
        if (j < chunks) {
            const u32x4 qv = q[j], kw = k[j];
            u32x4 kr[TOK];
#pragma unroll
            for (int u = 0; u < TOK; ++u) kr[u] = __builtin_nontemporal_load(key[u] + j);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float w0 = lo_bf16(qv[e]) * lo_bf16(kw[e]);  // exact: bf16 * bf16 fits fp32
                const float w1 = hi_bf16(qv[e]) * hi_bf16(kw[e]);
#pragma unroll
                for (int u = 0; u < TOK; ++u) {
                    const float h0 = lo_bf16(hr[u][i][e]), h1 = hi_bf16(hr[u][i][e]);
                    const float k0 = lo_bf16(kr[u][e]), k1 = hi_bf16(kr[u][e]);
                    hh[u] += h0 * h0 + h1 * h1;
                    kk[u] += k0 * k0 + k1 * k1;
                    hwk[u] += h0 * w0 * k0 + h1 * w1 * k1;
                }
            }
        }
    }

    float gate[TOK];
#pragma unroll
    for (int u = 0; u < TOK; ++u) {
        // butterfly sums: every lane ends with the totals, so every lane derives the same gate
        const float shh = wave_sum(hh[u]), skk = wave_sum(kk[u]), shwk = wave_sum(hwk[u]);
        const float rstd = rsqrtf(shh * a.inv_dim + a.eps) * rsqrtf(skk * a.inv_dim + a.eps);
        const float d = shwk * rstd * a.rsqrt_dim;
        if (a.dot && lane == 0 && u < ntok) a.dot[tok[u] * a.hc + c] = d;
        gate[u] = (a.mask && a.mask[tok[u]] == 0) ? 0.f : gate_of(d);
    }

#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int j = lane + 64 * i;
        if (j < chunks) {
#pragma unroll
            for (int u = 0; u < TOK; ++u)
                if (u < ntok) __builtin_nontemporal_store(residual(hr[u][i], vr[u][i], gate[u]), out[u] + j);
        }
    }
}

// Small launches: one workgroup per (token, copy); wave w keeps the 16-byte pieces w*64 + lane + 256 i
// (P of them) of the stream and value rows in registers, the four waves' sums go through LDS, and every
// thread adds them in wave order, so all derive the same dot and gate.
template <int P>
__global__ __launch_bounds__(kThreads) void gate_output_split_kernel(OutArgs a) {
    __shared__ float part[kWaves][3];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t tc = blockIdx.x;  // token * hc + copy
    const int c = static_cast<int>(tc % a.hc);
    const int64_t t = tc / a.hc;
    const int chunks = a.dim / 8;
    const u32x4* q = reinterpret_cast<const u32x4*>(a.q + static_cast<int64_t>(c) * a.dim);
    const u32x4* k = reinterpret_cast<const u32x4*>(a.k + static_cast<int64_t>(c) * a.dim);
    const uint16_t* row = a.kv + t * a.ld_kv;
    const u32x4* h = reinterpret_cast<const u32x4*>(a.x + tc * a.dim);
    const u32x4* key = reinterpret_cast<const u32x4*>(row + static_cast<int64_t>(c) * a.dim);
    const u32x4* val = reinterpret_cast<const u32x4*>(row + static_cast<int64_t>(a.hc) * a.dim);
    u32x4* out = reinterpret_cast<u32x4*>(a.out + tc * a.dim);

    u32x4 hr[P], vr[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int j = w * 64 + lane + kThreads * i;
        if (j < chunks) {
            hr[i] = h[j];
            vr[i] = val[j];
        }
    }
    float hh = 0.f, kk = 0.f, hwk = 0.f;
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int j = w * 64 + lane + kThreads * i;
        if (j < chunks) {
            const u32x4 qv = q[j], kw = k[j], kr = key[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float w0 = lo_bf16(qv[e]) * lo_bf16(kw[e]);  // exact: bf16 * bf16 fits fp32
                const float w1 = hi_bf16(qv[e]) * hi_bf16(kw[e]);
                const float h0 = lo_bf16(hr[i][e]), h1 = hi_bf16(hr[i][e]);
                const float k0 = lo_bf16(kr[e]), k1 = hi_bf16(kr[e]);
                hh += h0 * h0 + h1 * h1;
                kk += k0 * k0 + k1 * k1;
                hwk += h0 * w0 * k0 + h1 * w1 * k1;
            }
        }
    }
    hh = wave_sum(hh);
    kk = wave_sum(kk);
    hwk = wave_sum(hwk);
    if (lane == 0) {
        part[w][0] = hh;
        part[w][1] = kk;
        part[w][2] = hwk;
    }
    __syncthreads();
    float shh = 0.f, skk = 0.f, shwk = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
        shh += part[v][0];
        skk += part[v][1];
        shwk += part[v][2];
    }
    const float rstd = rsqrtf(shh * a.inv_dim + a.eps) * rsqrtf(skk * a.inv_dim + a.eps);
    const float d = shwk * rstd * a.rsqrt_dim;
    if (a.dot && threadIdx.x == 0) a.dot[tc] = d;
    const float gate = (a.mask && a.mask[t] == 0) ? 0.f : gate_of(d);
#pragma unroll
    for (int i = 0; i < P; ++i) {
        const int j = w * 64 + lane + kThreads * i;
        if (j < chunks) out[j] = residual(hr[i], vr[i], gate);
    }
}

template <int P, int TOK>
int launch_gate_output(const OutArgs& a, hipStream_t stream) {
    OutArgs b = a;
    b.groups = (a.T + TOK - 1) / TOK * a.hc;
    const int64_t blocks = (b.groups + kWaves - 1) / kWaves;
    if (blocks > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "engram_gate_output: too many tokens");
    if (b.groups < kSplitBelowWaves && a.dim >= 512 * kWaves && a.dim <= 3 * 8 * kThreads) {
        // fewer waves than the CUs need: a workgroup per (token, copy), the row split over its waves
        hipLaunchKernelGGL(gate_output_split_kernel<3>, dim3(static_cast<unsigned>(a.T * a.hc)), dim3(kThreads), 0,
                           stream, b);
    } else {
        hipLaunchKernelGGL((gate_output_kernel<P, TOK>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, stream,
                           b);
    }
    return check_launch("engram_gate_output");
}

// ---------------------------------------------------------------------------
// gate and residual from a given dot (the fused projection's output)
// ---------------------------------------------------------------------------
struct ResArgs {
    const uint16_t* x;
    const uint16_t* value;
    int64_t ld_value;
    const float* dot;
    const uint8_t* mask;  // [T] or null
    uint16_t* out;
    int64_t T;
    int64_t pieces;       // T * hc * dim / 8
    int hc, chunks;       // chunks = dim / 8
};

constexpr int kResPieces = 4;  // 16-byte pieces per thread

// Streaming: thread-block b covers kResPieces * 256 consecutive 16-byte pieces of out (= of x);
// the gate of a piece's (token, copy) is recomputed from its dot (one fp32 sqrt, exp and divide per
// 8 outputs), the value piece of its token is re-read from L2 by the hc copies.
__global__ __launch_bounds__(kThreads) void gate_residual_kernel(ResArgs a) {
    const int64_t base = static_cast<int64_t>(blockIdx.x) * (kResPieces * kThreads) + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kResPieces; ++u) {
        const int64_t i = base + u * kThreads;
        if (i >= a.pieces) return;
        const int64_t tc = i / a.chunks;
        const int j = static_cast<int>(i - tc * a.chunks);
        const int64_t t = tc / a.hc;
        const float g = (a.mask && a.mask[t] == 0) ? 0.f : gate_of(a.dot[tc]);
        const u32x4 h = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.x) + i);  // read once
        const u32x4 v = *reinterpret_cast<const u32x4*>(a.value + t * a.ld_value + 8 * j);    // shared by the copies
        __builtin_nontemporal_store(residual(h, v, g), reinterpret_cast<u32x4*>(a.out) + i);
    }
}

}  // namespace
}  // namespace engram

using namespace engram;

extern "C" int engram_gate_dot(const uint16_t* x, const uint16_t* kv, int64_t ld_kv, const uint16_t* q_weight,
                               const uint16_t* k_weight, float eps, float* dot, int64_t T, int32_t hc, int32_t dim,
                               void* stream) {
    if (T < 0) return fail(ENGRAM_EINVAL, "engram_gate_dot: T < 0");
    if (hc < 1 || hc > 64) return fail(ENGRAM_EINVAL, "engram_gate_dot: hc=%d outside [1, 64]", hc);
    if (dim < 8 || dim % 8 != 0) return fail(ENGRAM_EINVAL, "engram_gate_dot: dim=%d must be a positive multiple of 8", dim);
    if (ld_kv < static_cast<int64_t>(hc) * dim || ld_kv % 8 != 0)
        return fail(ENGRAM_EINVAL, "engram_gate_dot: ld_kv=%lld must be >= hc*dim and a multiple of 8", (long long)ld_kv);
    if (T == 0) return ENGRAM_OK;
    if (!x || !kv || !q_weight || !k_weight || !dot) return fail(ENGRAM_EINVAL, "engram_gate_dot: null pointer");
    if (!aligned(x, 16) || !aligned(kv, 16) || !aligned(q_weight, 16) || !aligned(k_weight, 16) || !aligned(dot, 4))
        return fail(ENGRAM_EINVAL, "engram_gate_dot: misaligned pointer");
    GateArgs a;
    a.x = x;
    a.kv = kv;
    a.ld_kv = ld_kv;
    a.q = q_weight;
    a.k = k_weight;
    a.eps = eps;
    a.inv_dim = 1.0f / static_cast<float>(dim);
    a.rsqrt_dim = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(dim)));
    a.dot = dot;
    a.T = T;
    a.groups = (T + kTok - 1) / kTok * hc;
    a.hc = hc;
    a.dim = dim;
    const int64_t blocks = (a.groups + kWaves - 1) / kWaves;
    if (blocks > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "engram_gate_dot: too many tokens");
    if (a.groups < kSplitBelowWaves && dim >= 512 * kWaves) {
        // fewer waves than the CUs need: a workgroup per (token, copy) instead, the row split over its waves
        hipLaunchKernelGGL(gate_dot_split_kernel, dim3(static_cast<unsigned>(T * hc)), dim3(kThreads), 0,
                           as_stream(stream), a);
    } else {
        hipLaunchKernelGGL(gate_dot_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, as_stream(stream), a);
    }
    return check_launch("engram_gate_dot");
}

extern "C" int engram_gate_output(const uint16_t* x, const uint16_t* kv, int64_t ld_kv, const uint16_t* q_weight,
                                  const uint16_t* k_weight, float eps, const uint8_t* token_mask, uint16_t* out,
                                  float* dot, int64_t T, int32_t hc, int32_t dim, void* stream) {
    if (T < 0) return fail(ENGRAM_EINVAL, "engram_gate_output: T < 0");
    if (hc < 1 || hc > 64) return fail(ENGRAM_EINVAL, "engram_gate_output: hc=%d outside [1, 64]", hc);
    if (dim < 8 || dim % 8 != 0 || dim > 8192)
        return fail(ENGRAM_EINVAL, "engram_gate_output: dim=%d must be a multiple of 8 in [8, 8192]", dim);
    if (ld_kv < static_cast<int64_t>(hc + 1) * dim || ld_kv % 8 != 0)
        return fail(ENGRAM_EINVAL, "engram_gate_output: ld_kv=%lld must be >= (hc+1)*dim and a multiple of 8",
                    (long long)ld_kv);
    if (T == 0) return ENGRAM_OK;
    if (!x || !kv || !q_weight || !k_weight || !out) return fail(ENGRAM_EINVAL, "engram_gate_output: null pointer");
    if (!aligned(x, 16) || !aligned(kv, 16) || !aligned(q_weight, 16) || !aligned(k_weight, 16) ||
        !aligned(out, 16) || !aligned(dot, 4))
        return fail(ENGRAM_EINVAL, "engram_gate_output: misaligned pointer");
    OutArgs a;
    a.x = x;
    a.kv = kv;
    a.ld_kv = ld_kv;
    a.q = q_weight;
    a.k = k_weight;
    a.mask = token_mask;
    a.eps = eps;
    a.inv_dim = 1.0f / static_cast<float>(dim);
    a.rsqrt_dim = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(dim)));
    a.out = out;
    a.dot = dot;
    a.T = T;
    a.groups = 0;
    a.hc = hc;
    a.dim = dim;
    hipStream_t s = as_stream(stream);
    const int pieces = (dim / 8 + 63) / 64;  // 16-byte pieces per lane and row
    if (pieces <= 1) return launch_gate_output<1, 2>(a, s);
    if (pieces <= 2) return launch_gate_output<2, 2>(a, s);
    if (pieces <= 4) return launch_gate_output<4, 2>(a, s);
    if (pieces <= 6) return launch_gate_output<6, 2>(a, s);
    if (pieces <= 8) return launch_gate_output<8, 2>(a, s);
    if (pieces <= 10) return launch_gate_output<10, 2>(a, s);
    if (pieces <= 12) return launch_gate_output<12, 1>(a, s);
    return launch_gate_output<16, 1>(a, s);
}

extern "C" int engram_gate_residual(const uint16_t* x, const uint16_t* value, int64_t ld_value, const float* dot,
                                    const uint8_t* token_mask, uint16_t* out, int64_t T, int32_t hc, int32_t dim,
                                    void* stream) {
    if (T < 0) return fail(ENGRAM_EINVAL, "engram_gate_residual: T < 0");
    if (hc < 1 || hc > 64) return fail(ENGRAM_EINVAL, "engram_gate_residual: hc=%d outside [1, 64]", hc);
    if (dim < 8 || dim % 8 != 0) return fail(ENGRAM_EINVAL, "engram_gate_residual: dim=%d must be a positive multiple of 8", dim);
    if (ld_value < dim || ld_value % 8 != 0)
        return fail(ENGRAM_EINVAL, "engram_gate_residual: ld_value=%lld must be >= dim and a multiple of 8",
                    (long long)ld_value);
    if (T == 0) return ENGRAM_OK;
    if (!x || !value || !dot || !out) return fail(ENGRAM_EINVAL, "engram_gate_residual: null pointer");
    if (!aligned(x, 16) || !aligned(value, 16) || !aligned(out, 16) || !aligned(dot, 4))
        return fail(ENGRAM_EINVAL, "engram_gate_residual: misaligned pointer");
    ResArgs a;
    a.x = x;
    a.value = value;
    a.ld_value = ld_value;
    a.dot = dot;
    a.mask = token_mask;
    a.out = out;
    a.T = T;
    a.chunks = dim / 8;
    a.hc = hc;
    a.pieces = T * hc * a.chunks;
    const int64_t blocks = (a.pieces + kResPieces * kThreads - 1) / (kResPieces * kThreads);
    if (blocks > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "engram_gate_residual: too many tokens");
    hipLaunchKernelGGL(gate_residual_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0,
                       as_stream(stream), a);
    return check_launch("engram_gate_residual");
}
