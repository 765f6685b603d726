// Device side of the seeded input generator (see synth/__init__.py): fills an
// fp8 table and its fp32 block scales from the counter-based SplitMix64
// definition, so tables of hundreds of millions of rows never pass through
// the host.  Holds none of the Engram method's arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ inline uint64_t splitmix64_at(uint64_t seed, uint64_t n) {
    uint64_t z = seed + (n + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// one lane = 16 table bytes (4 words of the row's stream)
__global__ __launch_bounds__(256) void fill_weight(uint8_t* weight, int64_t rows, int D, int W, uint64_t seed,
                                                   const uint8_t* lut) {
    const int pieces = D / 16;
    const int64_t total = rows * pieces;
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
        const int64_t r = q / pieces;
        const int piece = (int)(q - r * pieces);
        u32x4 out;
        for (int i = 0; i < 4; ++i) {
            const uint64_t u = splitmix64_at(seed, (uint64_t)r * W + piece * 4 + i);
            uint32_t word = 0;
            for (int b = 0; b < 4; ++b) word |= (uint32_t)lut[(u >> (16 * b)) & 0xFFFF] << (8 * b);
            out[i] = word;
        }
        *reinterpret_cast<u32x4*>(weight + r * D + piece * 16) = out;
    }
}

__global__ __launch_bounds__(256) void fill_scale(float* scale, int64_t rows, int D, int S, int W, uint64_t seed) {
    const int64_t total = rows * S;
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
        const int64_t r = q / S;
        const int j = (int)(q - r * S);
        const uint64_t u = splitmix64_at(seed, (uint64_t)r * W + D / 4 + j);
        const uint32_t mant = (uint32_t)(u & 0x7FFFFF);
        const uint32_t ex = (uint32_t)((u >> 32) % 6);
        scale[q] = __uint_as_float(((127u - 8u + ex) << 23) | mant);
    }
}

}  // namespace

// weight uint8 [rows, D] (16-byte aligned), scale float [rows, D/blk], lut uint8 [65536]; all device pointers.
extern "C" int synth_fill_table(uint8_t* weight, float* scale, int64_t rows, int D, int blk, uint64_t seed,
                                const uint8_t* lut, void* stream) {
    if (rows < 0 || D < 16 || D % 16 != 0 || blk < 1 || D % blk != 0) return 1;
    if (rows == 0) return 0;
    if (((uintptr_t)weight & 15) || ((uintptr_t)scale & 3)) return 1;
    const int S = D / blk, W = D / 4 + S;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(fill_weight, dim3(8192), dim3(256), 0, s, weight, rows, D, W, seed, lut);
    hipLaunchKernelGGL(fill_scale, dim3(4096), dim3(256), 0, s, scale, rows, D, S, W, seed);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}
