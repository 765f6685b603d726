// The dequant of 16 gathered fp8 bytes, shared by the gather and the fused hash + gather kernels.
#pragma once

#include "common.h"

namespace engram {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t pack_bf16_rne(float lo, float hi) {
    bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

// 16 fp8 E4M3FN bytes times their block scale -> 16 bf16 (two 16-byte vectors): v_cvt_pk_f32_fp8 (exact),
// an fp32 product rounded to nearest even, then bf16 rounded to nearest even -- the page's two roundings.
__device__ inline void dequant16(const u32x4& v, float s, u32x4& o0, u32x4& o1) {
    uint32_t r[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v[i]), false);  // bytes 0, 1
        const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v[i]), true);   // bytes 2, 3
        r[2 * i] = pack_bf16_rne(a.x * s, a.y * s);
        r[2 * i + 1] = pack_bf16_rne(b.x * s, b.y * s);
    }
    o0 = u32x4{r[0], r[1], r[2], r[3]};
    o1 = u32x4{r[4], r[5], r[6], r[7]};
}

}  // namespace engram
