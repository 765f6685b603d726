// engram_gate_dot: the gate pre-activation per (token, hc copy).
//
// Computes, from Engram.forward on the DeepSeek V4.1 "stack-hashes" page,
// the per-copy weight product q_weight * k_weight, the two RMS factors of
// the stream copy and of its key (each over `dim`, per copy, not jointly over
// the copies), and dot = sum(h * w * key) * rstd * dim^-1/2.
//
// Design (gfx950): HBM-bound streaming reduction.  One wave per 4 tokens of
// one copy: every lane streams 16-byte pieces (8 bf16) of the 4 stream rows
// and 4 key rows (8 loads in flight per lane and step), widens them to fp32,
// multiplies by the weight product (the copy's q and k pieces are loaded once
// for the 4 tokens; they stay in L2) and keeps three fp32 partial sums per
// token.  A wave-wide butterfly finishes the sums; lane 0 applies the two
// reciprocal square roots and writes one fp32 per token.
#include "common.h"

namespace engram {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTok = 4;  // tokens per wave: the copy's q/k chunks are loaded once for all of them

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
            hv[u] = h[u][j];
            kv[u] = key[u][j];
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
    hipLaunchKernelGGL(gate_dot_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, as_stream(stream), a);
    return check_launch("engram_gate_dot");
}
