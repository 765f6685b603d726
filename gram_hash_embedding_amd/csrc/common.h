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

// The second launch of a fused projection + gate (wkv.hip): per (token, copy), the per-128-column partial sums
// [hc][dim/128][3][T] of each of `layers` layers (layer e's at part + e * part_stride floats) added in slice
// order, then dot = sum(h w key) * rsqrt(mean h^2 + eps) * rsqrt(mean key^2 + eps) * dim^-1/2.
int launch_gate_finalize(const float* part, int64_t part_stride, float* const* dot, int layers, int64_t T, int hc,
                         int dim, float eps, hipStream_t stream, const char* what);

}  // namespace engram
