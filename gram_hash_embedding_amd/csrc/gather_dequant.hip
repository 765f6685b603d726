// engram_gather_dequant: fused fp8 row gather + block-scale dequant to bf16.
//
// Computes ParallelEngramEmbedding.forward of the DeepSeek V4.1
// "stack-hashes" page for one rank's rows [row_start, row_start + R): the
// range mask, the two embedding lookups (fp8 row and its fp32 block scales),
// the dequant (fp32 product, then bf16) and the zero fill of out-of-range
// ids.  The table stays fp8 in HBM; only gathered rows are ever widened.
//
// Design (gfx950): HBM-bound random gather.
// - A table row is D bytes (64 at the released shape): D/16 lanes each move
//   one 16-byte piece with a single dwordx4 load, and the same lanes fetch
//   the row's fp32 scale (lanes of one 32-wide block read the same word).
// - The ids are read with non-temporal loads (they stream through once, and
//   keeping them out of L2 leaves it to the table lines and their
//   translations); one row per lane (the many resident waves cover the
//   random-read latency) measured best: 69 us against 85 us for ordinary
//   accesses and 8 rows per lane on the long-prefill ids, 152 against 170 us
//   on uniform ids.  The rows are written with ordinary stores, which leave
//   them in the Infinity Cache for the projection that reads them next: 74-75
//   against 70-71 us for the long prefill's gather in the step, and a 6 %
//   shorter decode step when its gathers are separate launches.
// - Decode: v_cvt_pk_f32_fp8 (OCP E4M3FN on gfx950) two bytes at a time,
//   v_mul_f32 by the scale (round to nearest even), v_cvt_pk_bf16_f32 (round
//   to nearest even): the same two roundings as the page.
// - Output rows (t, c) are laid out consecutively, so a wave's stores for
//   one u cover 64/(D/16) whole rows: 2 KB contiguous at D = 64.
// - Packed tables (engram_pack_table): the pages keep a row's D fp8 bytes and
//   its D/blk fp32 scales in two tensors, so a random lookup of a 64-byte row
//   costs two 128-byte lines (the row's and the scale's) -- 256 bytes fetched
//   for 72 used.  A packed record of 2*D bytes holds the row and then its
//   scales (zero padded), aligned to its size: at D <= 64 a lookup touches one
//   line.  The dequant is the same code, so the outputs are bit-identical.
// - MX output (engram_gather_mx): the dequantised bf16 values are encoded
//   as OCP MX fp8 in the kernel (mx.h, the quantiser's code) and written as
//   the fp8 projection's A operand -- D bytes per row and one E8M0 byte per
//   32 columns in the [K/128][rows4][4] scale layout -- instead of 2 D bytes
//   of bf16 that a second pass would read back and quantise.  The two lanes
//   of a 32-column block combine their amax with one lane swap.
#include "dequant.h"
#include "mx.h"

namespace engram {
namespace {

constexpr int kThreads = 256;

struct GatherArgs {
    const void* ids;        // int64 (or, with IdT = int32_t, int32) [T, stride]
    int64_t stride;
    int64_t W;  // rows to produce = T * C
    int C;
    const uint8_t* weight;  // [R, D] fp8, or the packed table [R, 2D]
    const void* scale;      // [R, D/blk]: fp32, or one-byte E8M0 / E4M3 (unused for a packed table)
    int64_t R, row_start;
    int blk;
    uint16_t* out;
    uint8_t* out_fp8;
    void* out_scale;        // the gathered scale elements as stored, or null
    uint8_t* mx_q;          // MX output: fp8 [T, C*D] and E8M0 [C*D/128][rows4][4]
    uint8_t* mx_scale;
    int64_t rows4;
};

// Block scale formats of the table: 32-bit float, E8M0 (2^(s-127); 0xFF NaN) and float8_e4m3fn.
constexpr int kScaleF32 = 0, kScaleE8M0 = 1, kScaleE4M3 = 2;

// One-byte scale -> fp32 (exact): E8M0 as the exponent field (0 is the fp32 subnormal 2^-127), E4M3 through
// the fp8 convert (OCP E4M3FN on gfx950).
template <int SF>
__device__ inline float decode_scale(uint32_t s) {
    if constexpr (SF == kScaleE8M0)
        return __uint_as_float(s == 0 ? 0x00400000u : (s == 0xFFu ? 0x7FC00000u : s << 23));
    else
        return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(s), 0);
}

template <int D, int U, bool kPacked, int SF = kScaleF32, typename IdT = int64_t, bool kMx = false>
__global__ __launch_bounds__(kThreads) void gather_dequant_kernel(GatherArgs a) {
    constexpr int LPR = D / 16;              // lanes per row
    constexpr int RPS = kThreads / LPR;      // rows per step of the block
    const int lane_in_row = threadIdx.x % LPR;
    const int64_t base = static_cast<int64_t>(blockIdx.x) * (RPS * U) + threadIdx.x / LPR;
    const int S = D / a.blk;
    const int sidx = (lane_in_row * 16) / a.blk;  // this lane's scale block

    int64_t row[U];
    bool ok[U];
    bool live[U];
    int64_t tok[U];
    int col[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t w = base + static_cast<int64_t>(u) * RPS;
        live[u] = w < a.W;
        int64_t id = 0;
        tok[u] = 0;
        col[u] = 0;
        if (live[u]) {
            int64_t t, c;
            if (a.W <= 0xFFFFFFFFll) {
                const uint32_t w32 = static_cast<uint32_t>(w);
                const uint32_t t32 = w32 / static_cast<uint32_t>(a.C);
                t = t32;
                c = w32 - t32 * static_cast<uint32_t>(a.C);
            } else {
                t = w / a.C;
                c = w - t * a.C;
            }
            id = __builtin_nontemporal_load(static_cast<const IdT*>(a.ids) + t * a.stride + c);
            tok[u] = t;
            col[u] = static_cast<int>(c);
        }
        const int64_t local = id - a.row_start;
        ok[u] = live[u] && local >= 0 && local < a.R;
        row[u] = ok[u] ? local : 0;
    }

    u32x4 v[U];
    float sc[U];
    uint32_t sraw[U];  // the stored scale element
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (kPacked) {
            const uint8_t* rec = a.weight + row[u] * (2 * D);
            v[u] = *reinterpret_cast<const u32x4*>(rec + lane_in_row * 16);
            sc[u] = reinterpret_cast<const float*>(rec + D)[sidx];
        } else {
            v[u] = *reinterpret_cast<const u32x4*>(a.weight + row[u] * D + lane_in_row * 16);
            if constexpr (SF == kScaleF32) {
                sc[u] = static_cast<const float*>(a.scale)[row[u] * S + sidx];
            } else {
                sraw[u] = static_cast<const uint8_t*>(a.scale)[row[u] * S + sidx];
                sc[u] = decode_scale<SF>(sraw[u]);
            }
        }
    }

    if constexpr (kMx) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // every lane runs the block's amax exchange (its partner lane has the same row, hence the same
            // `live`); only live rows store
            u32x4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
            if (ok[u]) dequant16(v[u], sc[u], o0, o1);
            float f[16];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                f[2 * i] = __uint_as_float(o0[i] << 16);
                f[2 * i + 1] = __uint_as_float(o0[i] & 0xFFFF0000u);
                f[8 + 2 * i] = __uint_as_float(o1[i] << 16);
                f[8 + 2 * i + 1] = __uint_as_float(o1[i] & 0xFFFF0000u);
            }
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(f[i]));
            amax = fmaxf(amax, __shfl_xor(amax, 1, 64));  // lanes 2j, 2j + 1 of a row: its 32-column block j
            const int shared = mx_shared_exp(amax);
            const u32x4 qv = {mx_encode4(f[0], f[1], f[2], f[3], shared), mx_encode4(f[4], f[5], f[6], f[7], shared),
                              mx_encode4(f[8], f[9], f[10], f[11], shared),
                              mx_encode4(f[12], f[13], f[14], f[15], shared)};
            if (!live[u]) continue;
            const int64_t w = base + static_cast<int64_t>(u) * RPS;
            *reinterpret_cast<u32x4*>(a.mx_q + w * D + lane_in_row * 16) = qv;
            if ((lane_in_row & 1) == 0)
                a.mx_scale[mx_scale_offset(tok[u], (col[u] * D + lane_in_row * 16) / 32, a.rows4)] =
                    static_cast<uint8_t>(shared + 127);
        }
        return;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (!live[u]) continue;
        const int64_t w = base + static_cast<int64_t>(u) * RPS;
        u32x4 o0, o1;
        if (ok[u]) {
            dequant16(v[u], sc[u], o0, o1);
        } else {
            o0 = u32x4{0, 0, 0, 0};
            o1 = o0;
        }
        u32x4* dst = reinterpret_cast<u32x4*>(a.out + w * D + lane_in_row * 16);
        dst[0] = o0;
        dst[1] = o1;
        if (a.out_fp8) *reinterpret_cast<u32x4*>(a.out_fp8 + w * D + lane_in_row * 16) = v[u];
        if (a.out_scale && (lane_in_row * 16) % a.blk == 0) {
            if constexpr (SF == kScaleF32)
                static_cast<float*>(a.out_scale)[w * S + sidx] = sc[u];
            else
                static_cast<uint8_t*>(a.out_scale)[w * S + sidx] = static_cast<uint8_t>(sraw[u]);
        }
    }
}

template <int D, bool kPacked, int SF = kScaleF32, typename IdT = int64_t, bool kMx = false>
int launch(const GatherArgs& a, hipStream_t stream, const char* name) {
    constexpr int U = 1;
    constexpr int rows_per_block = (kThreads / (D / 16)) * U;
    const int64_t blocks = (a.W + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "%s: too many rows", name);
    hipLaunchKernelGGL((gather_dequant_kernel<D, U, kPacked, SF, IdT, kMx>), dim3(static_cast<unsigned>(blocks)),
                       dim3(kThreads), 0, stream, a);
    return check_launch(name);
}

// the MX-output gather (fp32 scales, int64 ids), D dispatched here
template <bool kPacked>
int launch_mx(const GatherArgs& a, int D, hipStream_t s, const char* name) {
    switch (D) {
        case 32: return launch<32, kPacked, kScaleF32, int64_t, true>(a, s, name);
        case 64: return launch<64, kPacked, kScaleF32, int64_t, true>(a, s, name);
        case 128: return launch<128, kPacked, kScaleF32, int64_t, true>(a, s, name);
        default: return launch<256, kPacked, kScaleF32, int64_t, true>(a, s, name);
    }
}

// the two-tensor gather for a scale format and id type (D dispatched here)
template <int SF, typename IdT>
int launch_fmt(const GatherArgs& a, int D, hipStream_t s, const char* name) {
    switch (D) {
        case 32: return launch<32, false, SF, IdT>(a, s, name);
        case 64: return launch<64, false, SF, IdT>(a, s, name);
        case 128: return launch<128, false, SF, IdT>(a, s, name);
        default: return launch<256, false, SF, IdT>(a, s, name);
    }
}

// One thread per 16-byte piece of the packed table: pieces [0, D/16) of a record are the row, the rest its
// scales followed by zeros.
__global__ __launch_bounds__(kThreads) void pack_table_kernel(const uint8_t* weight, const float* scale, int64_t R,
                                                              int D, int S, uint8_t* packed) {
    const int64_t pieces = R * (2 * D / 16);
    const int per_rec = 2 * D / 16;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < pieces;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
        const int64_t r = i / per_rec;
        const int pc = static_cast<int>(i - r * per_rec);
        u32x4 v = {0, 0, 0, 0};
        if (pc < D / 16) {
            v = *reinterpret_cast<const u32x4*>(weight + r * D + pc * 16);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int sidx = (pc - D / 16) * 4 + k;
                if (sidx < S) v[k] = __float_as_uint(scale[r * S + sidx]);
            }
        }
        *reinterpret_cast<u32x4*>(packed + i * 16) = v;
    }
}

}  // namespace
}  // namespace engram

using namespace engram;

namespace {
// scale_format: 0 fp32, 1 E8M0, 2 E4M3 (two-tensor tables only); id_bytes 8 or 4
int gather_entry(const char* name, bool packed, const void* hash_ids, int64_t T, int64_t id_token_stride, int32_t C,
                 const uint8_t* weight, const void* scale, int64_t R, int64_t row_start, int32_t D, int32_t blk,
                 uint16_t* out_bf16, uint8_t* out_fp8, void* out_scale, void* stream, int scale_format = 0,
                 int id_bytes = 8, uint8_t* mx_q = nullptr, uint8_t* mx_scale = nullptr) {
    const bool mx = mx_q != nullptr || mx_scale != nullptr;
    if (T < 0) return fail(ENGRAM_EINVAL, "%s: T < 0", name);
    if (C < 1 || C > 1024) return fail(ENGRAM_EINVAL, "%s: C=%d outside [1, 1024]", name, C);
    if (id_token_stride < C) return fail(ENGRAM_EINVAL, "%s: id_token_stride < C", name);
    if (D != 32 && D != 64 && D != 128 && D != 256)
        return fail(ENGRAM_EINVAL, "%s: D=%d not in {32, 64, 128, 256}", name, D);
    if (blk < 16 || blk % 16 != 0 || D % blk != 0)
        return fail(ENGRAM_EINVAL, "%s: blk=%d must be a multiple of 16 dividing D=%d", name, blk, D);
    if (R < 1) return fail(ENGRAM_EINVAL, "%s: R < 1", name);
    if (mx && (static_cast<int64_t>(C) * D) % 128 != 0)
        return fail(ENGRAM_EINVAL, "%s: C*D=%lld must be a multiple of 128", name, static_cast<long long>(C) * D);
    if (T == 0) return ENGRAM_OK;
    if (!hash_ids || !weight || (!packed && !scale) || (mx ? (!mx_q || !mx_scale) : !out_bf16))
        return fail(ENGRAM_EINVAL, "%s: null pointer", name);
    const int sbytes = scale_format == 0 ? 4 : 1;
    if (!aligned(hash_ids, id_bytes) || !aligned(weight, packed ? 2 * D : 16) || (!packed && !aligned(scale, sbytes)) ||
        (out_bf16 && !aligned(out_bf16, 16)) || (out_fp8 && !aligned(out_fp8, 16)) ||
        (out_scale && !aligned(out_scale, sbytes)) || (mx_q && !aligned(mx_q, 16)))
        return fail(ENGRAM_EINVAL, "%s: misaligned pointer", name);

    GatherArgs a;
    a.ids = hash_ids;
    a.stride = id_token_stride;
    a.W = T * C;
    a.C = C;
    a.weight = weight;
    a.scale = scale;
    a.R = R;
    a.row_start = row_start;
    a.blk = blk;
    a.out = out_bf16;
    a.out_fp8 = out_fp8;
    a.out_scale = out_scale;
    a.mx_q = mx_q;
    a.mx_scale = mx_scale;
    a.rows4 = (T + 3) / 4 * 4;
    hipStream_t s = as_stream(stream);
    if (mx) return packed ? launch_mx<true>(a, D, s, name) : launch_mx<false>(a, D, s, name);
    if (packed) {
        switch (D) {
            case 32: return launch<32, true>(a, s, name);
            case 64: return launch<64, true>(a, s, name);
            case 128: return launch<128, true>(a, s, name);
            default: return launch<256, true>(a, s, name);
        }
    }
    if (id_bytes == 4) {
        if (scale_format == kScaleE8M0) return launch_fmt<kScaleE8M0, int32_t>(a, D, s, name);
        if (scale_format == kScaleE4M3) return launch_fmt<kScaleE4M3, int32_t>(a, D, s, name);
        return launch_fmt<kScaleF32, int32_t>(a, D, s, name);
    }
    if (scale_format == kScaleE8M0) return launch_fmt<kScaleE8M0, int64_t>(a, D, s, name);
    if (scale_format == kScaleE4M3) return launch_fmt<kScaleE4M3, int64_t>(a, D, s, name);
    return launch_fmt<kScaleF32, int64_t>(a, D, s, name);
}
}  // namespace

extern "C" int engram_gather_dequant(const int64_t* hash_ids, int64_t T, int64_t id_token_stride, int32_t C,
                                     const uint8_t* weight, const float* scale, int64_t R, int64_t row_start,
                                     int32_t D, int32_t blk, uint16_t* out_bf16, uint8_t* out_fp8,
                                     float* out_scale, void* stream) {
    return gather_entry("engram_gather_dequant", false, hash_ids, T, id_token_stride, C, weight, scale, R, row_start,
                        D, blk, out_bf16, out_fp8, out_scale, stream);
}

extern "C" int engram_gather_dequant_fmt(const void* hash_ids, int32_t id_bytes, int64_t T, int64_t id_token_stride,
                                         int32_t C, const uint8_t* weight, const void* scale, int32_t scale_format,
                                         int64_t R, int64_t row_start, int32_t D, int32_t blk, uint16_t* out_bf16,
                                         uint8_t* out_fp8, void* out_scale, void* stream) {
    const char* name = "engram_gather_dequant_fmt";
    if (id_bytes != 4 && id_bytes != 8) return fail(ENGRAM_EINVAL, "%s: id_bytes=%d not 4 or 8", name, id_bytes);
    if (scale_format < kScaleF32 || scale_format > kScaleE4M3)
        return fail(ENGRAM_EINVAL, "%s: scale_format=%d not 0 (fp32), 1 (E8M0) or 2 (E4M3)", name, scale_format);
    return gather_entry(name, false, hash_ids, T, id_token_stride, C, weight, scale, R, row_start, D, blk, out_bf16,
                        out_fp8, out_scale, stream, scale_format, id_bytes);
}

extern "C" int engram_gather_dequant_packed(const int64_t* hash_ids, int64_t T, int64_t id_token_stride, int32_t C,
                                            const uint8_t* table, int64_t R, int64_t row_start, int32_t D,
                                            int32_t blk, uint16_t* out_bf16, uint8_t* out_fp8, float* out_scale,
                                            void* stream) {
    return gather_entry("engram_gather_dequant_packed", true, hash_ids, T, id_token_stride, C, table, nullptr, R,
                        row_start, D, blk, out_bf16, out_fp8, out_scale, stream);
}

extern "C" int engram_gather_mx(const int64_t* hash_ids, int64_t T, int64_t id_token_stride, int32_t C,
                                const uint8_t* weight, const float* scale, int64_t R, int64_t row_start, int32_t D,
                                int32_t blk, uint8_t* q, uint8_t* q_scale, void* stream) {
    return gather_entry("engram_gather_mx", false, hash_ids, T, id_token_stride, C, weight, scale, R, row_start, D,
                        blk, nullptr, nullptr, nullptr, stream, 0, 8, q, q_scale);
}

extern "C" int engram_gather_mx_packed(const int64_t* hash_ids, int64_t T, int64_t id_token_stride, int32_t C,
                                       const uint8_t* table, int64_t R, int64_t row_start, int32_t D, int32_t blk,
                                       uint8_t* q, uint8_t* q_scale, void* stream) {
    return gather_entry("engram_gather_mx_packed", true, hash_ids, T, id_token_stride, C, table, nullptr, R, row_start,
                        D, blk, nullptr, nullptr, nullptr, stream, 0, 8, q, q_scale);
}

extern "C" int engram_pack_table(const uint8_t* weight, const float* scale, int64_t R, int32_t D, int32_t blk,
                                 uint8_t* packed, void* stream) {
    if (D != 32 && D != 64 && D != 128 && D != 256)
        return fail(ENGRAM_EINVAL, "engram_pack_table: D=%d not in {32, 64, 128, 256}", D);
    if (blk < 16 || blk % 16 != 0 || D % blk != 0)
        return fail(ENGRAM_EINVAL, "engram_pack_table: blk=%d must be a multiple of 16 dividing D=%d", blk, D);
    if (R < 0) return fail(ENGRAM_EINVAL, "engram_pack_table: R < 0");
    if (R == 0) return ENGRAM_OK;
    if (!weight || !scale || !packed) return fail(ENGRAM_EINVAL, "engram_pack_table: null pointer");
    if (!aligned(weight, 16) || !aligned(scale, 4) || !aligned(packed, 2 * D))
        return fail(ENGRAM_EINVAL, "engram_pack_table: misaligned pointer");
    const int64_t pieces = R * (2 * D / 16);
    const int64_t need = (pieces + kThreads - 1) / kThreads;
    const int64_t blocks = need < (1 << 20) ? need : (1 << 20);
    hipLaunchKernelGGL(pack_table_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, as_stream(stream),
                       weight, scale, R, D, D / blk, packed);
    return check_launch("engram_pack_table");
}
