// Internal helpers shared by the HIP sources of libengram.so (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/engram.h"

namespace engram {

// Record a one-line failure description for engram_last_error() and return `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// ENGRAM_EHIP with the runtime's message if the last launch failed, else ENGRAM_OK.
int check_launch(const char* what);

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// 16-byte vector of 32-bit words: the unit of every wide global access.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The bf16 projection on v_mfma_f32_16x16x32_bf16 (wkv16.hip) for one layer: whether it takes a launch of T
// tokens (K a multiple of 64 with at least three slabs, and enough tiles of all N = (hc + 1) dim columns for two
// waves over the CUs, so that a fused launch takes it exactly when the plain one of the same weights does; for
// the gate, 128 rows of x under 2^31 bytes), and the launch.  Plain (gate false): kv [T, ld_out] = a [T, K] x
// w [N, K]^T.  Gate: w holds (hc + 1) dim rows; the key rows are reduced against x into `part`
// ([hc][dim/128][3][T] fp32, what launch_gate_finalize reads) and the dim value rows stored into kv [T, ld_out].
// Arguments are checked by the caller.
bool wkv16_takes(int64_t T, int K, int N, int hc, int dim, bool gate);
int launch_wkv16(const uint16_t* a, const uint16_t* w, uint16_t* kv, int64_t ld_out, int64_t T, int K, int N,
                 const uint16_t* x, const uint16_t* q, const uint16_t* k, float* part, int hc, int dim, bool gate,
                 hipStream_t stream, const char* what);

// One layer's tensors in a several-layer launch of the fused projection: a [T, K], w [(hc + 1) dim, K], the value
// rows out kv [T, ld_out], x [T, hc, dim], q and k [hc, dim], part [hc][dim/128][3][T] fp32.
struct W16Layer {
    const uint16_t* a;
    const uint16_t* w;
    uint16_t* kv;
    const uint16_t* x;
    const uint16_t* q;
    const uint16_t* k;
    float* part;
};
constexpr int kW16MaxLayers = 8;
// The fused projection of `layers` layers (at most kW16MaxLayers) as one launch of the 16 x 16 x 32 kernels, key
// and value tiles of every layer sharing the CUs: whether it takes such a launch (K a multiple of 64 with at least
// three slabs, dim a multiple of 256, 128 rows of x under 2^31 bytes), and the launch.  Each layer's results are
// those of launch_wkv16 with gate true on that layer, bit for bit.  Arguments are checked by the caller.
bool wkv16_layers_takes(int64_t T, int K, int hc, int dim, int layers);
int launch_wkv16_layers(const W16Layer* lay, int layers, int64_t ld_out, int64_t T, int K, int hc, int dim,
                        hipStream_t stream, const char* what);

// The second launch of a fused projection + gate (wkv.hip): per (token, copy), the per-128-column partial sums
// [hc][dim/128][3][T] of each of `layers` layers (layer e's at part + e * part_stride floats) added in slice
// order, then dot = sum(h w key) * rsqrt(mean h^2 + eps) * rsqrt(mean key^2 + eps) * dim^-1/2.
int launch_gate_finalize(const float* part, int64_t part_stride, float* const* dot, int layers, int64_t T, int hc,
                         int dim, float eps, hipStream_t stream, const char* what);

}  // namespace engram
