// engram_wkv: kv = A * W^T on bf16 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// Computes the `wkv` Linear of Engram.forward on the DeepSeek V4.1
// "stack-hashes" page: [T, C*D] gathered rows -> [T, dim*(hc_mult+1)] (the hc
// keys followed by the shared value), fp32 accumulation, one bf16 rounding.
//
// Design (gfx950, dense contraction -> MFMA):
// - Both operands are K-contiguous (A [T,K], W [Nout,K]), so one loader
//   serves both: 16-byte global loads, 8 lanes per 128-byte row segment.
// - Workgroup tile 256 x 256 x 64, four waves in a 2 x 2 grid, each wave a
//   128 x 128 sub-tile = 4 x 4 MFMA 32x32x16 blocks held in 256 fp32
//   accumulators (AGPRs).
// - LDS double buffer (2 x 72 KB of the CU's 160 KB); rows padded to 144 bytes
//   so the 16-byte fragment reads of 8 consecutive rows hit distinct banks.
//   The next K slab is fetched from HBM into registers while the current one
//   is multiplied, then written to the other buffer: one barrier per slab.
// - Epilogue: accumulators -> bf16 -> LDS (reusing the buffers) -> 16-byte
//   row-contiguous global stores.
// - Tile order: workgroups are dispatched round-robin over the 8 XCDs; the
//   block index is remapped so each XCD walks a contiguous run of tiles, and
//   runs are grouped 8 M-tiles deep so concurrently resident tiles share A and
//   W panels in that XCD's L2.
#include "common.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int LDA = BK + 8;               // padded LDS row (elements): 144 bytes
constexpr int kTileElems = BM * LDA;      // one operand tile in LDS
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
constexpr int EPI_LD = 128 + 8;           // epilogue LDS row (elements) of a wave's 128x128 tile

struct WkvArgs {
    const uint16_t* a;
    const uint16_t* w;
    uint16_t* kv;
    int64_t M;
    int N, K;
    int tiles_m, tiles_n;
};

__device__ inline void tile_coords(const WkvArgs& p, int& tm, int& tn) {
    const int n = p.tiles_m * p.tiles_n;
    const int pid = blockIdx.x;
    // contiguous run of tiles per XCD
    const int xcd = pid % kXcds, idx = pid / kXcds;
    const int per = n / kXcds, rem = n % kXcds;
    const int logical = xcd * per + min(xcd, rem) + idx;
    // grouped ordering: kGroupM M-tiles share each sweep over N
    const int in_group = kGroupM * p.tiles_n;
    const int group = logical / in_group;
    const int first_m = group * kGroupM;
    const int gsize = min(p.tiles_m - first_m, kGroupM);
    const int r = logical - group * in_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

__global__ __launch_bounds__(kThreads, 1) void wkv_kernel(WkvArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * kTileElems];  // [buf][A|B][BM][LDA]

    int tm, tn;
    tile_coords(p, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // ---- global -> register loader: 8 x 16 B of A and of W per lane ----
    const int ld_row = tid >> 3;        // + 32 * i
    const int ld_col = (tid & 7) * 8;   // element offset inside the K slab
    const uint16_t* a_src[8];
    const uint16_t* w_src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int64_t m = m0 + ld_row + 32 * i;
        if (m >= p.M) m = p.M - 1;  // ragged M: duplicate the last row, never stored
        int n = n0 + ld_row + 32 * i;
        if (n >= p.N) n = p.N - 1;
        a_src[i] = p.a + m * p.K + ld_col;
        w_src[i] = p.w + static_cast<int64_t>(n) * p.K + ld_col;
    }
    u32x4 ra[8], rw[8];
    auto load_slab = [&](int k0) {
        const bool in_k = k0 + ld_col < p.K;  // K % 8 == 0: a 16-byte piece is wholly in or out
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            ra[i] = in_k ? *reinterpret_cast<const u32x4*>(a_src[i] + k0) : u32x4{0, 0, 0, 0};
            rw[i] = in_k ? *reinterpret_cast<const u32x4*>(w_src[i] + k0) : u32x4{0, 0, 0, 0};
        }
    };
    auto store_slab = [&](int buf) {
        uint16_t* la = lds + buf * 2 * kTileElems;
        uint16_t* lb = la + kTileElems;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            *reinterpret_cast<u32x4*>(la + (ld_row + 32 * i) * LDA + ld_col) = ra[i];
            *reinterpret_cast<u32x4*>(lb + (ld_row + 32 * i) * LDA + ld_col) = rw[i];
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // fragment addressing: lane holds row (lane % 32), k pieces 8*(lane/32) .. +8
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;

    const int KT = (p.K + BK - 1) / BK;
    load_slab(0);
    store_slab(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) load_slab((kt + 1) * BK);
        const uint16_t* la = lds + cur * 2 * kTileElems + (wm * 128 + frag_row) * LDA + frag_k;
        const uint16_t* lb = lds + cur * 2 * kTileElems + kTileElems + (wn * 128 + frag_row) * LDA + frag_k;
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(la + i * 32 * LDA + kk);
#pragma unroll
            for (int j = 0; j < 4; ++j) fb[j] = *reinterpret_cast<const bf16x8*>(lb + j * 32 * LDA + kk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) store_slab(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: bf16 through LDS, then row-contiguous 16-byte stores ----
    uint16_t* ep = lds + wave * 128 * EPI_LD;
    // accumulator element r of block (i, j): row 32i + 8(r/4) + 4(lane/32) + r%4, column 32j + lane%32
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int col = 32 * j + (lane & 31);
                ep[row * EPI_LD + col] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[i][j][r]));
            }
    __syncthreads();
    const int64_t row0 = m0 + wm * 128;
    const int col0 = n0 + wn * 128;
#pragma unroll 4
    for (int q = lane; q < 128 * 16; q += 64) {
        const int row = q >> 4, c16 = (q & 15) * 8;
        const int64_t m = row0 + row;
        const int n = col0 + c16;
        if (m < p.M && n < p.N)
            *reinterpret_cast<u32x4*>(p.kv + m * p.N + n) = *reinterpret_cast<const u32x4*>(ep + row * EPI_LD + c16);
    }
}

}  // namespace
}  // namespace engram

using namespace engram;

extern "C" int engram_wkv(const uint16_t* a, const uint16_t* w, uint16_t* kv, int64_t T, int32_t K, int32_t Nout,
                          void* stream) {
    if (T < 0) return fail(ENGRAM_EINVAL, "engram_wkv: T < 0");
    if (K < 8 || K % 8 != 0) return fail(ENGRAM_EINVAL, "engram_wkv: K=%d must be a positive multiple of 8", K);
    if (Nout < 8 || Nout % 8 != 0) return fail(ENGRAM_EINVAL, "engram_wkv: Nout=%d must be a positive multiple of 8", Nout);
    if (T == 0) return ENGRAM_OK;
    if (!a || !w || !kv) return fail(ENGRAM_EINVAL, "engram_wkv: null pointer");
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(kv, 16)) return fail(ENGRAM_EINVAL, "engram_wkv: misaligned pointer");
    WkvArgs p;
    p.a = a;
    p.w = w;
    p.kv = kv;
    p.M = T;
    p.N = Nout;
    p.K = K;
    const int64_t tiles_m = (T + BM - 1) / BM;
    p.tiles_n = (Nout + BN - 1) / BN;
    if (tiles_m * p.tiles_n > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "engram_wkv: too many tiles");
    p.tiles_m = static_cast<int>(tiles_m);
    hipLaunchKernelGGL(wkv_kernel, dim3(static_cast<unsigned>(tiles_m * p.tiles_n)), dim3(kThreads), 0,
                       as_stream(stream), p);
    return check_launch("engram_wkv");
}
