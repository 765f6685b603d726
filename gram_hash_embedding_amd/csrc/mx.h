// OCP MX fp8 block encoding (E4M3 elements, one E8M0 scale per 32 elements), shared by the quantiser of bf16
// rows (engram_mx_quant) and the gather that writes MX fp8 rows directly (engram_gather_mx): both encode the
// same bf16 values, so their bytes agree.
#pragma once

#include "common.h"

namespace engram {

// The block's shared exponent from its amax (a bf16 value held in fp32, normal or subnormal, so fp32 holds it
// exactly): floor(log2 amax) - 8 (8 is E4M3's largest exponent), clamped to E8M0's [-127, 127], read off the
// exponent field (or, for a subnormal, the leading one of the fraction); -127 for an all-zero block.  Its E8M0
// code is shared + 127.
__device__ inline int mx_shared_exp(float amax) {
    if (!(amax > 0.f)) return -127;
    const uint32_t au = __float_as_uint(amax);
    const int ef = static_cast<int>(au >> 23);
    const int fl = ef != 0 ? ef - 127 : 31 - __builtin_clz(au & 0x7FFFFFu) - 149;  // floor(log2 amax)
    return max(-127, min(127, fl - 8));
}

// Four elements times 2^-shared (exact: a power of two; results below fp32's normal range round to 0 in E4M3
// either way), clamped to +-448 so that the conversion cannot overflow, rounded to E4M3 (nearest even,
// subnormals included) by v_cvt_pk_fp8_f32 -- OCP E4M3 on gfx950: the saturating conversion.  Bytes in
// element order.
__device__ inline uint32_t mx_encode4(float f0, float f1, float f2, float f3, int shared) {
    auto g = [shared](float f) { return __builtin_amdgcn_fmed3f(__builtin_ldexpf(f, -shared), -448.0f, 448.0f); };
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(g(f0), g(f1), 0, false);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(g(f2), g(f3), lo, true));
}

// Byte offset of the E8M0 scale of (row r, 32-column block b) in the scale layout [K/128][rows4][4].
__device__ inline int64_t mx_scale_offset(int64_t r, int b, int64_t rows4) {
    return (static_cast<int64_t>(b >> 2) * rows4 + r) * 4 + (b & 3);
}

}  // namespace engram
