/*
 * CPU oracle for the Engram forward path -- TEST INFRASTRUCTURE ONLY.
 * Host C, no GPU headers; nothing here is shared with the HIP library.
 * Layouts are row-major and match the HIP library's arguments so that the
 * same synthetic inputs can be handed to both.
 */
#ifndef ENGRAM_ORACLE_H
#define ENGRAM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_OK = 0, ORACLE_EINVAL = 1, ORACLE_ERANGE = 2, ORACLE_ENOMEM = 4 };

/* Hash (the stack-hashes page, the hash module's forward).
 * input_ids [B,L]; token_mask [B,L] (1 = takes part) or NULL; token_map [vocab];
 * cache [cache_B, cache_L] in/out (positions start_pos..start_pos+L-1 of rows
 * 0..B-1 are written, earlier positions are read); multipliers [E,N];
 * primes [E,N-1,H]; offsets [E,(N-1)H]; hash_ids out [B,L,E,(N-1)H]. */
int oracle_hash(const int64_t* input_ids, int64_t B, int64_t L, int64_t start_pos,
                const uint8_t* token_mask, const int64_t* token_map, int64_t vocab,
                int64_t* cache, int64_t cache_B, int64_t cache_L,
                const int64_t* multipliers, const int64_t* primes, const int64_t* offsets,
                int E, int N, int H, int64_t pad_id, int64_t dead, int64_t* hash_ids);

/* ParallelEngramEmbedding.forward: ids [T, stride] (first C used per token);
 * weight fp8 e4m3fn [R,D]; scale fp32 [R,D/blk] -> out_bf16 [T,C,D] and,
 * optionally, the gathered bytes [T,C,D] and scales [T,C,D/blk]. */
int oracle_gather_dequant(const int64_t* hash_ids, int64_t T, int64_t id_token_stride, int C,
                          const uint8_t* weight, const float* scale, int64_t R, int64_t row_start,
                          int D, int blk, uint16_t* out_bf16, uint8_t* out_fp8, float* out_scale);

/* The same with the block scales as float32 (scale_format 0), E8M0 (1) or
 * float8_e4m3fn (2) bytes, and int64 (id_bytes 8) or int32 (4) ids; out_scale
 * receives the gathered scale elements as stored. */
int oracle_gather_dequant_fmt(const void* hash_ids, int id_bytes, int64_t T, int64_t id_token_stride, int C,
                              const uint8_t* weight, const void* scale, int scale_format, int64_t R,
                              int64_t row_start, int D, int blk, uint16_t* out_bf16, uint8_t* out_fp8,
                              void* out_scale);

/* wkv: kv[t,o] = sum_k a[t,k] w[o,k] in double (a [T,K], w [Nout,K] bf16 bits). */
int oracle_wkv(const uint16_t* a, const uint16_t* w, double* kv, int64_t T, int K, int Nout);

/* fp8 block-scaled projection (OCP MX: E4M3FN elements, one E8M0 scale per
 * `blk` consecutive columns of a row).  mx_quant: bf16 x [rows,K] -> q
 * [rows,K] e4m3fn bytes and scale [rows,K/blk] E8M0 bytes; wkv_mx: kv[t,o] in
 * double from a (q, scale) [T,K] and w (q, scale) [Nout,K]. */
double oracle_e8m0_decode(uint8_t s);
uint8_t oracle_e4m3fn_encode_sat(double v);
int oracle_mx_quant(const uint16_t* x, int64_t rows, int K, int blk, uint8_t* q, uint8_t* scale);
int oracle_wkv_mx(const uint8_t* a_q, const uint8_t* a_s, const uint8_t* w_q, const uint8_t* w_s, double* kv,
                  int64_t T, int K, int Nout, int blk);

/* gate pre-activation: x [T,hc,dim] bf16; key = kv[t, c*dim + j] with row stride
 * ld_kv (bf16); q_weight, k_weight [hc,dim] bf16 -> dot [T,hc] double. */
int oracle_gate_dot(const uint16_t* x, const uint16_t* kv, int64_t ld_kv, const uint16_t* q_weight,
                    const uint16_t* k_weight, double eps, double* dot, int64_t T, int hc, int dim);

/* gate activation, mask and residual: gate = sigmoid(copysign(sqrt(max(|dot|,
 * 1e-6)), dot)), 0 where token_mask [T] (or NULL = all true) is 0; out[t,c,j] =
 * h[t,c,j] + gate[t,c] * kv[t, hc*dim + j].  dot [T,hc] in; gate [T,hc] and
 * out [T,hc,dim] double out. */
int oracle_gate_output(const uint16_t* x, const uint16_t* kv, int64_t ld_kv, const double* dot,
                       const uint8_t* token_mask, double* gate, double* out, int64_t T, int hc, int dim);

float oracle_e4m3fn_decode(uint8_t byte);
uint16_t oracle_bf16_rne(float f);
double oracle_bf16_to_double(uint16_t h);
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
