// Microbenchmarks of the ceilings the Engram kernels are measured against (include/engram_probe.h):
// matrix-core throughput on register-resident operands, and streaming HBM reads and copies.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/engram_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// independent accumulators: back-to-back MFMAs never wait on each other (32 x 32 blocks: 4, 16 x 16 blocks: 8)
constexpr int kChains = 4;

// kKind: 0 bf16 32x32x16, 1 fp8 32x32x64 with zero scale operands (the compiler issues the unscaled
// instruction), 2 bf16 16x16x32, 3 fp8 32x32x64 scaled, 4 fp8 16x16x128 scaled (scales from registers)
template <int kKind>
__global__ __launch_bounds__(512) void mfma_probe(const u32x4* ops, float* out, int iters) {
    constexpr bool kBf16 = kKind == 0 || kKind == 2;
    constexpr bool kSmall = kKind == 2 || kKind == 4;  // 16 x 16 result blocks
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    // each chain its own A and B fragments (32 bytes each), from a 64 KiB window of random bytes
    i32x8 a[kChains], b[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        const int base = ((wave * 7 + c * 64 + lane) * 4) & 4095;
        const u32x4 a0 = ops[base], a1 = ops[base + 1], b0 = ops[base + 2], b1 = ops[base + 3];
        a[c] = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        b[c] = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
        if (kBf16) {  // bf16: keep the patterns finite (clear the exponent's top bit of every element)
            for (int i = 0; i < 8; ++i) {
                a[c][i] &= 0xBFFFBFFF;
                b[c][i] &= 0xBFFFBFFF;
            }
        } else {  // E4M3: clear the NaN codes (S.1111.111) by clearing each byte's exponent top bit
            for (int i = 0; i < 8; ++i) {
                a[c][i] &= 0xBFBFBFBF;
                b[c][i] &= 0xBFBFBFBF;
            }
        }
    }
    // E8M0 scale operands held in a register (2^0 .. 2^3 by lane): a literal would let the compiler drop them
    int sc = 127 + (lane & 3);
    asm volatile("" : "+v"(sc));
    float s = 0.f;
    if constexpr (!kSmall) {
        f32x16 acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                if constexpr (kKind == 0) {
                    // the first 16 bytes of a chain's operands
                    const bf16x8 a_lo = __builtin_bit_cast(bf16x8, i32x8{a[c][0], a[c][1], a[c][2], a[c][3], 0, 0, 0, 0}.lo);
                    const bf16x8 b_lo = __builtin_bit_cast(bf16x8, i32x8{b[c][0], b[c][1], b[c][2], b[c][3], 0, 0, 0, 0}.lo);
                    acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo, b_lo, acc[c], 0, 0, 0);
                } else if constexpr (kKind == 1) {
                    acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[c], b[c], acc[c], 0, 0, 0, 0, 0, 0);
                } else {
                    acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[c], b[c], acc[c], 0, 0, 0, sc, 0, sc);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < kChains; ++c)
#pragma unroll
            for (int r = 0; r < 16; ++r) s += acc[c][r];
    } else {
        f32x4 acc[2 * kChains];  // chain c: A fragment c / 2, B fragment c % 2 of the pair c / 2
#pragma unroll
        for (int c = 0; c < 2 * kChains; ++c) acc[c] = f32x4{};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < 2 * kChains; ++c) {
                if constexpr (kKind == 2) {
                    const bf16x8 av = __builtin_bit_cast(bf16x8, i32x8{a[c >> 1][0], a[c >> 1][1], a[c >> 1][2], a[c >> 1][3], 0, 0, 0, 0}.lo);
                    const bf16x8 bv = __builtin_bit_cast(
                        bf16x8, i32x8{b[c >> 1][4 * (c & 1)], b[c >> 1][4 * (c & 1) + 1], b[c >> 1][4 * (c & 1) + 2],
                                      b[c >> 1][4 * (c & 1) + 3], 0, 0, 0, 0}.lo);
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[c], 0, 0, 0);
                } else {
                    acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[c >> 1], (c & 1) ? b[c >> 1] : a[(c >> 1) ^ 1],
                                                                               acc[c], 0, 0, 0, sc, 0, sc);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < 2 * kChains; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) s += acc[c][r];
    }
    if (lane == 0) out[wave] = s;
}

constexpr int kReadGrid = 256 * 8;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(256) void read_probe(const u32x4* src, int64_t n, float* out) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t x = 0;
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n; i += stride) {
        const u32x4 v = src[i];
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    __shared__ uint32_t red[256];
    red[threadIdx.x] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int t = 0; t < 256; ++t) r ^= red[t];
        out[blockIdx.x] = static_cast<float>(r & 0xFFFF);
    }
}

__global__ __launch_bounds__(256) void copy_probe(const u32x4* src, u32x4* dst, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

int launch_status() { return hipGetLastError() == hipSuccess ? 0 : 3; }

}  // namespace

extern "C" int engram_probe_mfma(int32_t kind, const void* operands, float* out, int32_t workgroups, int32_t waves,
                                 int32_t iters, void* stream) {
    if (kind < 0 || kind > 4 || !operands || !out || workgroups < 1 || waves < 1 || waves > 8 || iters < 1 ||
        (reinterpret_cast<uintptr_t>(operands) & 15))
        return 1;
    const dim3 grid(workgroups), block(64 * waves);
    auto s = reinterpret_cast<hipStream_t>(stream);
    const u32x4* ops = static_cast<const u32x4*>(operands);
    switch (kind) {
        case 0: hipLaunchKernelGGL(mfma_probe<0>, grid, block, 0, s, ops, out, iters); break;
        case 1: hipLaunchKernelGGL(mfma_probe<1>, grid, block, 0, s, ops, out, iters); break;
        case 2: hipLaunchKernelGGL(mfma_probe<2>, grid, block, 0, s, ops, out, iters); break;
        case 3: hipLaunchKernelGGL(mfma_probe<3>, grid, block, 0, s, ops, out, iters); break;
        default: hipLaunchKernelGGL(mfma_probe<4>, grid, block, 0, s, ops, out, iters); break;
    }
    return launch_status();
}

extern "C" int32_t engram_probe_read_grid(void) { return kReadGrid; }

extern "C" int engram_probe_read(const void* src, int64_t bytes, float* out, void* stream) {
    if (!src || !out || bytes < 16 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15)) return 1;
    hipLaunchKernelGGL(read_probe, dim3(kReadGrid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), bytes / 16, out);
    return launch_status();
}

extern "C" int engram_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (!src || !dst || bytes < 16 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) & 15) ||
        (reinterpret_cast<uintptr_t>(dst) & 15))
        return 1;
    hipLaunchKernelGGL(copy_probe, dim3(kReadGrid), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
    return launch_status();
}
