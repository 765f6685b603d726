// engram_wkv: kv = A * W^T on bf16 matrix cores (v_mfma_f32_32x32x16_bf16).
// Launches long enough for two waves of 256 x 256 tiles over the CUs per layer
// (K a multiple of 64, at least three slabs) run wkv16.hip's
// v_mfma_f32_16x16x32_bf16 kernels instead, layer by layer, and so does a
// fused launch of several shorter layers on 256-token tiles, in one launch; the
// kernels here serve launches small enough for one pass of 128-token tiles
// over the CUs, K below three 64-column slabs and K not a multiple of 64.
//
// Computes the `wkv` Linear of Engram.forward on the DeepSeek V4.1
// "stack-hashes" page: [T, C*D] gathered rows -> [T, dim*(hc_mult+1)] (the hc
// keys followed by the shared value), fp32 accumulation, one bf16 rounding.
//
// Design (gfx950, dense contraction -> MFMA):
// - Workgroup tile 256 x 256 and eight waves, two per SIMD: wave (wm, wn) owns
//   128 tokens x 64 outputs = 4 x 2 MFMA 32x32x16 blocks in 128 fp32
//   accumulators (VGPRs; the first k-step of a tile takes a zero C operand,
//   so they are never cleared separately).  One workgroup per CU.  With one wave per SIMD,
//   a wave stalled on issuing its direct-to-LDS loads (the CU's address FIFO
//   fills) left the matrix core idle; with two, the SIMD partner keeps it busy
//   (main loop 4.17 -> 3.73 ms on the long-prefill shape).  Fragment reads grow
//   to 96 B/clk/CU at full MFMA rate, under half of the 256 B/clk the LDS
//   delivers (measured).
// - Main kernel (K a multiple of 64): persistent, one workgroup per CU walks
//   its tiles; A and W slabs of 64 along K go HBM/L2 -> LDS with the gfx950
//   direct-to-LDS loads (buffer_load_dwordx4 ... lds: no VGPR staging, no
//   ds_write instructions), two 64 KB stages, issued by the four loader waves
//   (one per SIMD).  Rows are 128 B with the 16-byte pieces XOR-swizzled by
//   (row/2) mod 8, so the fragment reads of 16 consecutive rows hit 16
//   distinct bank groups.
// - One barrier per slab, placed before the last of its four k-steps: it
//   publishes the next slab (already landed) and frees the current stage for
//   the slab after next, whose loads are issued right away; the first
//   fragments of the next slab are then read while the last 8 MFMAs of this
//   one run.  The load stream runs across tile boundaries, so the next tile's
//   first slabs arrive during the current tile's last ones and its epilogue.
// - Fragment reads of k-step s+1 are interleaved with the 8 MFMAs of step s.
// - The MFMA is issued as W-fragment x A-fragment, so each lane ends up with
//   4 consecutive output columns of one token.  The epilogue turns them into
//   full 128-byte-line, non-temporal 16-byte stores through a 32 KB LDS
//   exchange region (the rest of the CU's LDS), written by the four storer
//   waves; scattered 8-byte stores measured 15% slower.
// - Tile order: workgroups are dispatched round-robin over the 8 XCDs; tiles
//   are renumbered so each XCD walks a contiguous run, grouped 8 M-tiles deep,
//   so the 32 tiles resident on an XCD share A and W panels in its L2.
// - Launches whose 256-token tiles would leave CUs idle (a decode step of a
//   few hundred tokens: 100 tiles for 256 CUs) use 128 x 256 tiles instead
//   (NI = 2 token blocks per wave, 64 x 64 per wave, 48 KB stages), as long
//   as those still fit the CUs in one pass: twice the CUs at work.  Such a
//   workgroup holds one tile, so it runs a three-stage ring (the slab loads,
//   mostly from beyond L2 there, get two slab periods instead of one) and
//   puts the stream rows and the epilogue exchange into the stages its last
//   slabs free.
// - Several engram layers in one launch (engram_wkv_gate_layers): their M tiles
//   are stacked and numbered layer by layer, each tile reading its layer's
//   operand pointers with a wave-uniform index into the kernel arguments; the
//   tile height is chosen for all layers together.
// - K not a multiple of 64: a register-staged four-wave variant with a
//   zero-filled K tail.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "common.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
constexpr int kCUs = 256;

// scheduling-group masks of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedVmem = 0x010;

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
constexpr int wait_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kWaitLgkmcnt0 = 0xC07F;  // lgkmcnt == 0 only (vmcnt 63, expcnt 7 left at their maxima)
// cache-policy operand of a global load: non-temporal (the line is streamed through L2 instead of
// displacing the operand panels that the other tiles of the XCD are re-reading)
constexpr int kNonTemporal = 2;
// word 3 of a raw buffer resource on gfx9-family targets (32-bit data format, no swizzle)
constexpr int kBufferWord3 = 0x00020000;

constexpr int kMaxLayers = 8;  // engram layers one launch may take (their tiles share the CUs)
static_assert(kMaxLayers <= kW16MaxLayers, "the 16 x 16 x 32 several-layer launch holds every layer");

// One layer's operands (every layer of a launch has the same M, N, K, hc and dim).
struct LayerPtrs {
    const uint16_t* a;
    const uint16_t* w;
    uint16_t* kv;       // stored output rows: columns [out_col0, N) of the product, row stride ld_out
    // fused gate partial sums (key columns [0, hc*dim) are reduced, not stored)
    const uint16_t* x;  // [M, hc, dim] bf16
    const uint16_t* q;  // [hc, dim] bf16
    const uint16_t* k;  // [hc, dim] bf16
    float* part;        // [hc][dim/128][3][M] fp32: per 128-column slice pair sum(h w key), sum(key^2), sum(h^2)
};

struct WkvArgs {
    LayerPtrs lay[kMaxLayers];  // indexed with a wave-uniform layer: one scalar load from the kernel arguments
    int64_t M;
    int N, K;
    int tiles_m, tiles_n;  // tiles_m = layers * tiles_ml: the layers' M tiles stacked, layer by layer
    int tiles_ml;          // M tiles of one layer
    int64_t ld_out;
    int out_col0;
    int hc, dim;
};

// pid -> (tm, tn).  Layer by layer (a persistent workgroup finishes its tiles of one layer before it starts
// the next, so the CUs share one layer's W panels at a time); inside a layer, contiguous runs per XCD (pid % 8
// is the XCD a workgroup lands on), grouped kGroupM deep.
__device__ inline void tile_coords(const WkvArgs& p, int pid, int& tm, int& tn) {
    const int n = p.tiles_ml * p.tiles_n;
    const int layer = pid / n;
    pid -= layer * n;
    const int xcd = pid % kXcds, idx = pid / kXcds;
    const int per = n / kXcds, rem = n % kXcds;
    const int logical = xcd * per + min(xcd, rem) + idx;
    const int in_group = kGroupM * p.tiles_n;
    const int group = logical / in_group;
    const int first_m = group * kGroupM;
    const int gsize = min(p.tiles_ml - first_m, kGroupM);
    const int r = logical - group * in_group;
    tm = layer * p.tiles_ml + first_m + r % gsize;
    tn = r / gsize;
}

// lane id recomputed from the exec mask (two VALU ops) rather than kept live in a VGPR
__device__ inline int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two fp32 -> packed bf16 (RNE) in one instruction, opaque to the compiler so that it keeps the pair
__device__ inline uint32_t cvt_pk_bf16(float lo, float hi) {
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
    return r;
}

// c + a.lo * b.lo + a.hi * b.hi over packed bf16 pairs, fp32 accumulation
__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ inline uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// acc[i][j] = W-block j (32 outputs) x A-block i (32 tokens): element r of a lane is output
// 32j + 8(r/4) + 4(lane/32) + r%4 of token 32i + lane%32.
__device__ inline void mfma_step(f32x16 (&acc)[4][4], const bf16x8* fa, const bf16x8* fw) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[j], fa[i], acc[i][j], 0, 0, 0);
}

// the 8 fragment reads of the next k-step spread among the 16 MFMAs of this one
__device__ inline void interleave_reads() {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    }
}

__device__ inline void zero(f32x16 (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

// 4 consecutive outputs per lane and block row -> one 8-byte bf16 store
__device__ inline void store_tile(const WkvArgs& p, const f32x16 (&acc)[4][4], int64_t m0, int n0, int wm, int wn,
                                  int lane) {
    const int64_t tok0 = m0 + wm * 128 + (lane & 31);
    const int col0 = n0 + wn * 128 + 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = tok0 + 32 * i;
        if (m >= p.M) continue;
        uint16_t* row = p.lay[0].kv + m * p.N;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = col0 + 32 * j + 8 * g;
                if (n < p.N) {
                    const u32x2 v = {pack_bf16(acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]),
                                     pack_bf16(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
                    *reinterpret_cast<u32x2*>(row + n) = v;
                }
            }
    }
}

// ============================================================================
// main kernel: persistent, eight waves, direct-to-LDS loads (K % 64 == 0)
// ============================================================================
constexpr int kWaves = 8;                      // two per SIMD
constexpr int kMainThreads = 64 * kWaves;
constexpr int kOpBytes = BN * BK * 2;          // the W slab: 256 rows x 128 B = 32 KB
constexpr int kExBytes = 64 * 512;             // epilogue exchange: 64 token rows x 256 outputs (bf16)
constexpr int kXArea = 32 * 128;               // a wave's stream rows for one round: 32 tokens x 64 bf16

// the eight-wave tile: wave (wm, wn) owns tokens [32 NI wm, +32 NI) x outputs [64 wn, +64), as NI x 2 MFMA
// blocks (NI = 4: a 256 x 256 workgroup tile; NI = 2: 128 x 256, for launches too small to fill the CUs)
template <int NI>
__device__ inline void mfma_step8(f32x16 (&acc)[NI][2], const bf16x8* fa, const bf16x8* fw) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[j], fa[i], acc[i][j], 0, 0, 0);
}

// the first k-step of a tile: C = 0 (no separate zeroing of the accumulators)
template <int NI>
__device__ inline void mfma_step8_zero(f32x16 (&acc)[NI][2], const bf16x8* fa, const bf16x8* fw) {
    const f32x16 z = {};
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[j], fa[i], z, 0, 0, 0);
}

// The NI + 2 fragment reads of the next k-step spread among the 2 NI MFMAs of this one, and with them
// V global loads (V / (2 NI) per MFMA).
template <int NI, int V>
__device__ inline void interleave8() {
    constexpr int kReads = NI + 2, kMfmas = 2 * NI;
    if constexpr (V == 0) {
#pragma unroll
        for (int s = 0; s < kReads; ++s) {
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        }
    } else {
        static_assert(V % kMfmas == 0, "loads spread evenly over the MFMAs");
#pragma unroll
        for (int s = 0; s < kMfmas; ++s) {
            if (s < kReads) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVmem, V / kMfmas, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        }
    }
}

struct SlabCursor {
    int pid;  // tile being loaded
    int kt;   // slab inside that tile
    // that tile's A and W panels (first row, bytes of valid rows), and the next tile's: computed once per
    // tile, off the slab loop, so a slab's issue does no index arithmetic and no argument load
    const uint16_t* a;
    const uint16_t* w;
    int a_bytes, w_bytes;
    const uint16_t* nxt_a;
    const uint16_t* nxt_w;
    int nxt_a_bytes, nxt_w_bytes;
};

// Eight waves, two per SIMD: wave w runs on SIMD w % 4, so each SIMD hosts one loader wave (0-3) and one
// storer wave (4-7).  A wave that issues its slab's 16 direct-to-LDS loads stalls while the CU's address
// FIFO drains; its SIMD partner keeps the matrix core busy meanwhile (with one wave per SIMD that stall
// was a matrix-core bubble, measured at ~20 % of the main loop).  A wave's vmcnt counts its loads and
// stores together and the slab barrier must wait for the loads, so the roles stay split: loaders never
// have stores outstanding, storers never wait for slab loads.
// kOneSlab: K is a single slab (K = 64; fused launches only), a tile loop of its own so that the other
// instances do not carry its registers.
template <bool kGate, int NI, bool kOneSlab = false>
__global__ __launch_bounds__(kMainThreads, 1) void wkv_kernel(WkvArgs p) {
    constexpr int kBM = 64 * NI;               // tokens per tile
    constexpr int kABytes = kBM * BK * 2;      // the A slab: kBM rows x 128 B
    constexpr int kStageBytes = kABytes + kOpBytes;
    constexpr int kSlabLoads = 2 * NI + 8;     // direct-to-LDS loads per loader wave and slab
    // NI = 2 is launched only when every workgroup holds a single tile: its three-stage ring (144 KB) needs
    // no exchange region, since the stream rows and the epilogue use the stages the last slabs free.
    constexpr bool kOneTile = NI == 2;
    constexpr int kStages = kOneTile ? 3 : 2;
    // [stage][A (kBM rows) | W (256 rows)][128 B] (+ exchange region): 160 KB at NI = 4, the whole LDS of a CU
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * kStageBytes + (kOneTile ? 0 : kExBytes)];

    const int tiles = p.tiles_m * p.tiles_n;
    const int G = gridDim.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
    const int wm = wave & 1, wn = wave >> 1;
    const bool loader = wave < 4;
    const int KT = p.K / BK;
    // tile pid -> its layer, first token inside the layer and first output column
    auto tile_of = [&](int pid, int& e, int64_t& m0, int& n0) {
        int tm, tn;
        tile_coords(p, pid, tm, tn);
        e = tm / p.tiles_ml;
        m0 = static_cast<int64_t>(tm - e * p.tiles_ml) * kBM;
        n0 = tn * BN;
    };
    int cur = 0;  // the layer of the tile in the epilogue (the tile loops set it)

    // A barrier that publishes LDS: every wave's LDS accesses are done (lgkmcnt); the loaders wait for
    // their slab loads (vmcnt) right before it.  The empty asm statements keep the compiler from moving
    // memory accesses across the barrier.
    auto sync = [&]() {
        __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // epilogue barrier: also a scheduling fence, so each round's accumulator conversions stay in
    // that round instead of being clustered (and spilled) ahead of the first barrier
    auto sync_epi = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        sync();
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- loader waves: wave w fills rows [16 NI w, +16 NI) of the A slab and [64w, 64w+64) of the W
    // slab, 8 rows per instruction; lane l lands at slot (l & 7) of row base + 8q + (l >> 3) and fetches
    // the 16-byte piece the swizzle puts there.  Buffer loads: the tile's rows are a buffer resource
    // (SGPRs) whose size stops at the last valid row, so rows past M or N read as zero instead of
    // faulting; a lane's offset is one of two 32-bit bases (every base is a multiple of 16 rows, so the
    // swizzle key of row base + 8q + r is ((r >> 1) | 4(q & 1))) plus the instruction's row offset.
    const int ld_r = lane >> 3, ld_slot = lane & 7;
    const int row_bytes = p.K * 2;
    const uint32_t vo_piece = static_cast<uint32_t>(ld_r * row_bytes + ((ld_slot ^ (ld_r >> 1)) << 4));
    const uint32_t vo_a = vo_piece + static_cast<uint32_t>(wave * 16 * NI * row_bytes);
    const uint32_t vo_w = vo_piece + static_cast<uint32_t>(wave * 64 * row_bytes);
    // `live` false (past this workgroup's last slab) still issues the instructions, against an empty
    // resource: they touch no memory, and keeping them unconditional lets them sit in the same basic
    // block as the MFMAs they are interleaved with.  An empty resource zero-fills a free stage.
    auto issue_slab = [&](const SlabCursor& c, int stage, bool live) {
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(c.a), 0, live ? c.a_bytes : 0, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(c.w), 0, live ? c.w_bytes : 0, kBufferWord3);
        const uint32_t k0b = static_cast<uint32_t>(c.kt * BK * 2);
        uint8_t* sa = lds + stage * kStageBytes + wave * 16 * NI * 128;
        uint8_t* sw = lds + stage * kStageBytes + kABytes + wave * 64 * 128;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            // the row offset goes into the VGPR offset: a raw buffer's range check covers the VGPR and
            // immediate offsets but not the SGPR offset, which carries only the slab's column
            // (row bases are multiples of 128 bytes: the XOR flips the piece's swizzle bit only)
            const uint32_t flip = (q & 1) ? (4u << 4) : 0u;
            const uint32_t qrows = static_cast<uint32_t>(q * 8 * row_bytes);
            if (q < 2 * NI)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, sa + q * 8 * 128, 16, (vo_a ^ flip) + qrows, k0b, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, sw + q * 8 * 128, 16, (vo_w ^ flip) + qrows, k0b, 0, 0);
        }
    };
    auto advance = [&](SlabCursor& c) {  // branch-free: it sits inside the interleaved block
        const bool wrap = c.kt + 1 == KT;
        c.kt = wrap ? 0 : c.kt + 1;
        c.pid += wrap ? G : 0;
        c.a = wrap ? c.nxt_a : c.a;
        c.w = wrap ? c.nxt_w : c.w;
        c.a_bytes = wrap ? c.nxt_a_bytes : c.a_bytes;
        c.w_bytes = wrap ? c.nxt_w_bytes : c.w_bytes;
    };
    // the panels of tile pid (rows past M or N left out of the resource: they read as zero)
    auto panels = [&](int pid, const uint16_t*& a, const uint16_t*& w, int& a_bytes, int& w_bytes) {
        int e, n0;
        int64_t m0;
        tile_of(pid, e, m0, n0);
        a = p.lay[e].a + m0 * p.K;
        w = p.lay[e].w + static_cast<int64_t>(n0) * p.K;
        a_bytes = static_cast<int>(min<int64_t>(kBM, p.M - m0)) * row_bytes;
        w_bytes = min(BN, p.N - n0) * row_bytes;
    };
    // the tile after tile pid, for the cursor's next wrap (past the last one: any valid tile; its loads are
    // issued against an empty resource)
    auto prepare_next = [&](SlabCursor& c, int pid) {
        const int np = pid + G < p.tiles_m * p.tiles_n ? pid + G : static_cast<int>(blockIdx.x);
        panels(np, c.nxt_a, c.nxt_w, c.nxt_a_bytes, c.nxt_w_bytes);
    };

    // ---- fragments: lane reads row (lane % 32) of a 32-row block, pieces 2kk + lane/32 ----
    const int g = (lane >> 1) & 7;  // swizzle key of the lane's rows (every block starts at a multiple of 16)
    const int a_row = (wm * 32 * NI + (lane & 31)) * 128;
    const int w_row = kABytes + (wn * 64 + (lane & 31)) * 128;
    auto read_frags = [&](int stage, int kk, bf16x8* fa, bf16x8* fw) {
        const uint8_t* base = lds + stage * kStageBytes;
        const int off = (((2 * kk + (lane >> 5)) ^ g) << 4);
#pragma unroll
        for (int i = 0; i < NI; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(base + a_row + i * 32 * 128 + off);
#pragma unroll
        for (int j = 0; j < 2; ++j) fw[j] = *reinterpret_cast<const bf16x8*>(base + w_row + j * 32 * 128 + off);
    };

    // ---- epilogue: NI rounds; in round i every wave puts its tokens 32i..32i+31 (64 outputs each) into
    // the exchange region (64 rows of 512 B: row 32 wm + t, 16-byte pieces XOR-swizzled by row), then the
    // four storer waves write 16 whole rows each with full-line, non-temporal 16-byte stores (kv is not
    // read again here)
    uint8_t* ex = lds + 2 * kStageBytes;  // (NI = 4 only)
    auto epilogue = [&](const f32x16 (&acc)[NI][2], int64_t m0, int n0, uint8_t* xch) {
        // Every lane-derived address below is rebuilt from a freshly computed lane id, so the compiler
        // cannot hoist the epilogue addresses out of the tile loop (where they would pin VGPRs for the
        // whole kernel).
        const int l = lane_id();
        const int key = l & 31;
        const uint32_t wbase = static_cast<uint32_t>((wm * 32 + (l & 31)) * 512 + (l >> 5) * 8);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int chunk = wn * 8 + 4 * j + gq;  // 16-byte piece of the 512-byte row
                    const u32x2 v = {pack_bf16(acc[i][j][4 * gq + 0], acc[i][j][4 * gq + 1]),
                                     pack_bf16(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3])};
                    *reinterpret_cast<u32x2*>(xch + wbase + ((chunk ^ key) << 4)) = v;
                }
            sync_epi();
            if (!loader) {
                const int s = wave - 4;  // exchange rows [16s, 16s + 16)
                const int ls = lane_id();
                const int chunk = ls & 31, hi = ls >> 5;
                const bool col_ok = n0 + chunk * 8 < p.N;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int rr = 16 * s + 2 * q + hi;  // exchange row: token half rr / 32, token rr % 32
                    const u32x4 v = *reinterpret_cast<const u32x4*>(xch + rr * 512 + ((chunk ^ (rr & 31)) << 4));
                    const int64_t m = m0 + (rr >> 5) * 32 * NI + 32 * i + (rr & 31);
                    if (m < p.M && col_ok)
                        __builtin_nontemporal_store(
                            v, reinterpret_cast<u32x4*>(p.lay[cur].kv + m * p.ld_out + (n0 - p.out_col0) + chunk * 8));
                }
            }
            sync_epi();
        }
    };

    // ---- fused gate epilogue of a key tile: no stores of the product.  The tile's 256 columns lie in
    // one copy c; wave (wm, wn) owns the 64-column slice s = (n0 - c dim) / 64 + wn of that copy and
    // tokens [32 NI wm, 32 NI (wm + 1)).  Lane l holds, per round i < NI, token 32i + l%32 and 32 of the
    // slice's columns (4 consecutive columns per (j, gq), as the MFMA leaves them).  Each accumulator is
    // rounded to bf16 (the product is a bf16 tensor before it is used) and reduced against the stream's
    // matching element: sum(h w key), sum(key^2), sum(h^2) over the lane's columns, then over the two
    // lane halves; per (copy, pair of slices, token) the three sums go to the workspace.
    // Stream rows come in with full-line, non-temporal direct-to-LDS loads into a 4 KB area per wave and
    // round (row t of an area is token t's 128 bytes, 16-byte piece p at slot p ^ ((t >> 1) & 7), so the
    // lane-layout reads below are conflict-free).  Round 0 goes into the exchange region while the
    // tile's main loop runs, loaded by the storer waves (which have no slab loads to wait for) for
    // their own area and for their SIMD partner's (loader wave w - 4: same tokens, the slice 128
    // columns to the left).  Rounds 1 and 2 go into the stage the tile's last slab frees (the next
    // tile's second slab is loaded into it only after the epilogue) and round 3 into the exchange
    // region once round 0 is reduced (NI = 2: rounds 0 and 1 only); each wave loads these for its own area and waits only for its
    // own loads, so the rounds need no workgroup barrier.  Loader waves hand their sums to their
    // partner, which stores both, so loaders never have stores outstanding at a slab barrier.
    // NI = 4: rounds 0 and 3 in the exchange region, 1 and 2 in stage sa.  One tile (NI = 2): round 0 in
    // stage sa, round 1 in stage sb.
    auto round_region = [&](int i, int sa, int sb) -> uint8_t* {
        if constexpr (kOneTile) return lds + (i == 0 ? sa : sb) * kStageBytes;
        return (i == 1 || i == 2) ? lds + sa * kStageBytes + (i - 1) * kExBytes : ex;
    };
    // storer wave: round i's 32 rows of its own area (v = 0) and its partner's (v = 1) into `region`,
    // 8 rows of 8 pieces per instruction (8 loads)
    auto dma_x = [&](int64_t m0, int n0, int i, uint8_t* region, auto both_tag) {
        constexpr int kAreas = decltype(both_tag)::value ? 2 : 1;
        const int ll = lane_id();
        const int c = n0 / p.dim;
        const int colw = n0 - c * p.dim;
        const int64_t xstride = static_cast<int64_t>(p.hc) * p.dim;  // elements per token of x
#pragma unroll
        for (int v = 0; v < kAreas; ++v) {
            const int ow = wave - 4 * v;  // owner wave of the area
            const uint16_t* xs = p.lay[cur].x + static_cast<int64_t>(c) * p.dim + colw + (ow >> 1) * 64;
#pragma unroll
            for (int ins = 0; ins < 4; ++ins) {
                const int r = 8 * ins + (ll >> 3);
                const int piece = (ll & 7) ^ ((r >> 1) & 7);
                const int64_t t = min<int64_t>(m0 + (ow & 1) * 32 * NI + 32 * i + r, p.M - 1);  // past M: unused
                __builtin_amdgcn_global_load_lds(xs + t * xstride + 8 * piece, region + ow * kXArea + ins * 1024, 16,
                                                 0, kNonTemporal);
            }
        }
    };
    // wait for this wave's own loads down to n outstanding, and keep LDS accesses after the wait
    auto own_wait = [&](auto n_tag) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(decltype(n_tag)::value));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto lds_fence = [&]() {  // this wave's LDS reads are done (before a load or write into the same area)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    // On entry the storers have round 0 of both their areas (8 loads) and rounds 1 and 2 (NI = 2: round 1)
    // of their own area (4 loads each) in flight, the loaders rounds 1 and 2 of their own area.  Round 0 reaches the loaders
    // through the one barrier; every later round is the wave's own loads, so it only waits for them.
    auto gate_epilogue = [&](const f32x16 (&acc)[NI][2], int64_t m0, int n0, int sa, int sb) {
        const int l = lane_id();
        const int c = n0 / p.dim;
        const int col0 = n0 - c * p.dim + wn * 64;  // this wave's slice
        const uint16_t* qrow = p.lay[cur].q + static_cast<int64_t>(c) * p.dim + col0 + 4 * (l >> 5);
        const uint16_t* krow = p.lay[cur].k + static_cast<int64_t>(c) * p.dim + col0 + 4 * (l >> 5);
        float wgt[2][4][4];  // q * k (exact in fp32) for the lane's 32 columns
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const u32x2 qv = *reinterpret_cast<const u32x2*>(qrow + 32 * j + 8 * gq);
                const u32x2 kv = *reinterpret_cast<const u32x2*>(krow + 32 * j + 8 * gq);
                wgt[j][gq][0] = lo_bf16(qv[0]) * lo_bf16(kv[0]);
                wgt[j][gq][1] = hi_bf16(qv[0]) * hi_bf16(kv[0]);
                wgt[j][gq][2] = lo_bf16(qv[1]) * lo_bf16(kv[1]);
                wgt[j][gq][3] = hi_bf16(qv[1]) * hi_bf16(kv[1]);
            }
        if constexpr (kOneTile) {
            own_wait(std::integral_constant<int, 4>{});  // round 0 (own loads; round 1's 4 may still fly)
        } else {
            // own loads in flight after round 0 has landed: rounds 1 and 2, 4 loads each
            if (!loader) own_wait(std::integral_constant<int, 8>{});
            sync_epi();  // round 0's stream rows are in, for every wave
        }
        float res[NI][3];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            if (i == 1) own_wait(std::integral_constant<int, 4 * (NI - 2)>{});  // rounds 2 .. NI-1 may still be in flight
            if (i == 2) own_wait(std::integral_constant<int, 4 * (NI > 3 ? NI - 3 : 0)>{});
            if (i == 3) own_wait(std::integral_constant<int, 0>{});
            const uint8_t* xl = round_region(i, sa, sb) + wave * kXArea;
            u32x2 xr[2][4];
            {
                const int rr = l & 31, h = l >> 5;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq)
                        xr[j][gq] = *reinterpret_cast<const u32x2*>(
                            xl + rr * 128 + (((4 * j + gq) ^ ((rr >> 1) & 7)) << 4) + h * 8);
            }
            if (i == 0 && NI == 4) {
                lds_fence();  // round 0 is read out of this wave's area: round 3 goes there
                dma_x(m0, n0, 3, ex, std::false_type{});
            }
            float hwk = 0.f, kk = 0.f, hh = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const uint32_t k01 = cvt_pk_bf16(acc[i][j][4 * gq + 0], acc[i][j][4 * gq + 1]);
                    const uint32_t k23 = cvt_pk_bf16(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3]);
                    const float key[4] = {lo_bf16(k01), hi_bf16(k01), lo_bf16(k23), hi_bf16(k23)};
                    const float h[4] = {lo_bf16(xr[j][gq][0]), hi_bf16(xr[j][gq][0]), lo_bf16(xr[j][gq][1]),
                                        hi_bf16(xr[j][gq][1])};
#pragma unroll
                    for (int r = 0; r < 4; ++r) hwk += h[r] * wgt[j][gq][r] * key[r];
                    kk = dot2_bf16(k01, k01, kk);
                    kk = dot2_bf16(k23, k23, kk);
                    hh = dot2_bf16(xr[j][gq][0], xr[j][gq][0], hh);
                    hh = dot2_bf16(xr[j][gq][1], xr[j][gq][1], hh);
                }
            res[i][0] = hwk + __shfl_xor(hwk, 32, 64);
            res[i][1] = kk + __shfl_xor(kk, 32, 64);
            res[i][2] = hh + __shfl_xor(hh, 32, 64);
        }
        // hand-over: a loader wave leaves its sums in its own area of the last round's region (it has read
        // that round there); its SIMD partner adds them to its own and stores both
        uint8_t* const hand = round_region(NI - 1, sa, sb);
        uint8_t* xl = hand + wave * kXArea;
        if (loader) {
            lds_fence();
            if (l < 32) {
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int q = 0; q < 3; ++q) reinterpret_cast<float*>(xl)[(i * 3 + q) * 32 + l] = res[i][q];
            }
        }
        sync_epi();
        if (!loader) {
            // the storer adds its partner's sums (slice 64 (wn - 2) of the tile) to its own (slice 64 wn):
            // one value per (copy, 128-column slice pair, token), always summed in this order
            const int ls = lane_id();
            if (ls < 32) {
                const float* partner = reinterpret_cast<const float*>(hand + (wave - 4) * kXArea);
                const int64_t tbase = m0 + wm * 32 * NI + ls;
                const int pair = (n0 - c * p.dim) / 128 + (wn - 2);
                float* out = p.lay[cur].part + (static_cast<int64_t>(c) * (p.dim / 128) + pair) * 3 * p.M;
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int64_t t = tbase + 32 * i;
#pragma unroll
                    for (int q = 0; q < 3; ++q) {
                        const float v = res[i][q] + partner[(i * 3 + q) * 32 + ls];
                        // ordinary stores: the finalize launch that follows reads them from L2 (the launches
                        // this kernel serves are decode-sized, a few hundred KB of sums; the long ones take
                        // wkv16.hip, which streams them)
                        if (t < p.M) out[q * p.M + t] = v;
                    }
                }
            }
        }
        sync_epi();  // the partner's sums and the stream rows in the freed stage are read before reuse
    };

    if (static_cast<int>(blockIdx.x) >= tiles) return;
    const int total_slabs_mine = ((tiles - 1 - static_cast<int>(blockIdx.x)) / G + 1) * KT;

    // The tile loop, instantiated separately for loader and storer waves (the branch is per wave, the
    // barrier count per tile is the same in both).  In the loader instance the 16 loads of the slab
    // after next are spread among the last 8 MFMAs of the current slab.
    auto run = [&](auto loader_tag) {
        constexpr bool kLoader = decltype(loader_tag)::value;
        int pid = blockIdx.x;
        SlabCursor ld{};
        ld.pid = pid;
        panels(pid, ld.a, ld.w, ld.a_bytes, ld.w_bytes);
        prepare_next(ld, pid);
        int issued = 0;
        if (kLoader) {
            if constexpr (kOneTile) {
                // prologue: three slabs in flight (the one tile has at least four), wait for the first
#pragma unroll
                for (int s0 = 0; s0 < kStages; ++s0) {
                    issue_slab(ld, s0, true);
                    advance(ld);
                    prepare_next(ld, ld.pid);
                    ++issued;
                }
                __builtin_amdgcn_s_waitcnt(wait_vmcnt((kStages - 1) * kSlabLoads));
            } else {
                // prologue: two slabs in flight
                issue_slab(ld, 0, true);
                advance(ld);
                prepare_next(ld, ld.pid);
                ++issued;
                issue_slab(ld, 1, issued < total_slabs_mine);
                advance(ld);
                prepare_next(ld, ld.pid);
                ++issued;
                __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
            }
        }
        sync();

        f32x16 acc[NI][2];
        bf16x8 fa0[NI], fw0[2], fa1[NI], fw1[2];
        read_frags(0, 0, fa0, fw0);
        int stage = 0;
        // One slab: four k-steps of 8 MFMAs, one barrier before the last.  kDefer (the last slab of a
        // fused key tile): the freed stage is kept for the epilogue's stream rows -- the loaders skip the
        // slab after next (issued after the epilogue) and every wave fetches its rounds 1 and 2 into it.
        auto slab = [&](auto defer_tag, auto first_tag, int64_t m0, int n0) {
            constexpr bool kDefer = decltype(defer_tag)::value;
            constexpr bool kFirst = decltype(first_tag)::value;
            read_frags(stage, 1, fa1, fw1);
            if (kFirst)
                mfma_step8_zero(acc, fa0, fw0);
            else
                mfma_step8(acc, fa0, fw0);
            interleave8<NI, 0>();
            read_frags(stage, 2, fa0, fw0);
            mfma_step8(acc, fa1, fw1);
            interleave8<NI, 0>();
            read_frags(stage, 3, fa1, fw1);
            mfma_step8(acc, fa0, fw0);
            interleave8<NI, 0>();
            // the next slab has landed and this stage is no longer read: publish one, refill the other
            if (kLoader) __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
            sync();
            // The next slab's first fragments (the next tile's, at the end of a tile; harmless stale
            // reads after the last one) are read under the last 2 NI MFMAs of this slab.
            read_frags(stage ^ 1, 0, fa0, fw0);
            if (kLoader && !kDefer) {
                issue_slab(ld, stage, issued < total_slabs_mine);  // slab after next into the freed stage
                advance(ld);
                ++issued;
                mfma_step8(acc, fa1, fw1);
                interleave8<NI, kSlabLoads>();
            } else if (kDefer) {
                // rounds 1 and 2 (NI = 4) or round 1 (NI = 2) of this wave's stream rows: 4 loads a round
                dma_x(m0, n0, 1, round_region(1, stage, 0), std::false_type{});
                if (NI == 4) dma_x(m0, n0, 2, round_region(2, stage, 0), std::false_type{});
                mfma_step8(acc, fa1, fw1);
                interleave8<NI, 4 * (NI == 4 ? 2 : 1)>();
            } else {
                mfma_step8(acc, fa1, fw1);
                interleave8<NI, 0>();
            }
            stage ^= 1;
        };
        // One-tile launches (NI = 2): a three-stage ring.  Phase 0: the slab three ahead goes into the freed
        // stage; phases 1 and 2 (the third- and second-to-last slab): the freed stage takes this wave's
        // stream rows of round 0 and round 1 (key tiles); phase 3: the last slab.  A loader's wait before a
        // barrier leaves in flight only what it issued after the slab being published.
        auto slab3 = [&](auto phase_tag, auto first_tag, auto key_tag, int64_t m0, int n0) {
            constexpr int kPhase = decltype(phase_tag)::value;
            constexpr bool kFirst = decltype(first_tag)::value;
            constexpr bool kKey = decltype(key_tag)::value;
            const int next = stage + 1 == kStages ? 0 : stage + 1;
            read_frags(stage, 1, fa1, fw1);
            if (kFirst)
                mfma_step8_zero(acc, fa0, fw0);
            else
                mfma_step8(acc, fa0, fw0);
            interleave8<NI, 0>();
            read_frags(stage, 2, fa0, fw0);
            mfma_step8(acc, fa1, fw1);
            interleave8<NI, 0>();
            read_frags(stage, 3, fa1, fw1);
            mfma_step8(acc, fa0, fw0);
            interleave8<NI, 0>();
            if (kLoader) {
                if constexpr (kPhase <= 1)
                    __builtin_amdgcn_s_waitcnt(wait_vmcnt(kSlabLoads));  // the next slab; the one after may fly
                else if constexpr (kPhase == 2)
                    __builtin_amdgcn_s_waitcnt(wait_vmcnt(kKey ? 4 : 0));  // the last slab; round 0 may fly
            }
            sync();
            read_frags(next, 0, fa0, fw0);  // (phase 3: stale, unused)
            if constexpr (kPhase == 0) {
                if (kLoader) {
                    issue_slab(ld, stage, true);
                    advance(ld);
                    ++issued;
                    mfma_step8(acc, fa1, fw1);
                    interleave8<NI, kSlabLoads>();
                } else {
                    mfma_step8(acc, fa1, fw1);
                    interleave8<NI, 0>();
                }
            } else if constexpr ((kPhase == 1 || kPhase == 2) && kKey) {
                dma_x(m0, n0, kPhase - 1, lds + stage * kStageBytes, std::false_type{});
                mfma_step8(acc, fa1, fw1);
                interleave8<NI, 4>();
            } else {
                mfma_step8(acc, fa1, fw1);
                interleave8<NI, 0>();
            }
            stage = next;
        };
        if constexpr (kOneTile) {
            for (; pid < tiles; pid += G) {  // one tile per workgroup
                int64_t m0;
                int n0;
                tile_of(pid, cur, m0, n0);
                auto body = [&](auto key_tag) {
                    constexpr bool kKey = decltype(key_tag)::value;
                    using Ph0 = std::integral_constant<int, 0>;
                    slab3(Ph0{}, std::true_type{}, key_tag, m0, n0);
                    for (int kt = 1; kt < KT - 3; ++kt) slab3(Ph0{}, std::false_type{}, key_tag, m0, n0);
                    const int sa = stage;
                    slab3(std::integral_constant<int, 1>{}, std::false_type{}, key_tag, m0, n0);
                    const int sb = stage;
                    slab3(std::integral_constant<int, 2>{}, std::false_type{}, key_tag, m0, n0);
                    const int sc = stage;
                    slab3(std::integral_constant<int, 3>{}, std::false_type{}, key_tag, m0, n0);
                    if constexpr (kKey)
                        gate_epilogue(acc, m0, n0, sa, sb);
                    else
                        epilogue(acc, m0, n0, lds + sc * kStageBytes);
                };
                if (kGate && n0 < p.out_col0)
                    body(std::true_type{});
                else
                    body(std::false_type{});
            }
            __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
            return;
        }
        for (; pid < tiles; pid += G) {
            int64_t m0;
            int n0;
            tile_of(pid, cur, m0, n0);
            // the loader wraps to its next tile exactly once during this tile's slabs: have that tile ready
            if (kLoader) prepare_next(ld, ld.pid);
            const bool key_tile = kGate && n0 < p.out_col0;
            if (key_tile) {
                // the exchange region is free until the epilogue: fetch the stream rows of round 0 now
                if (!kLoader) dma_x(m0, n0, 0, ex, std::true_type{});
                int free_stage = stage;
                if constexpr (kOneSlab) {
                    slab(std::true_type{}, std::true_type{}, m0, n0);
                } else {
                    slab(std::false_type{}, std::true_type{}, m0, n0);
                    for (int kt = 1; kt < KT - 1; ++kt) slab(std::false_type{}, std::false_type{}, m0, n0);
                    free_stage = stage;
                    slab(std::true_type{}, std::false_type{}, m0, n0);
                }
                gate_epilogue(acc, m0, n0, free_stage, 0);
                if (kLoader) {  // the slab after next, held back while the epilogue used its stage
                    issue_slab(ld, free_stage, issued < total_slabs_mine);
                    advance(ld);
                    ++issued;
                }
            } else {
                slab(std::false_type{}, std::true_type{}, m0, n0);
                for (int kt = 1; kt < KT; ++kt) slab(std::false_type{}, std::false_type{}, m0, n0);
                epilogue(acc, m0, n0, ex);
            }
        }
        // the slabs issued past this workgroup's last one (empty resources) still write LDS: let them land
        // before the workgroup ends
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    };
    if (loader)
        run(std::true_type{});
    else
        run(std::false_type{});
}

// ============================================================================
// register-staged kernel for any K % 8 == 0 (zero-filled K tail)
// ============================================================================
constexpr int LDA = BK + 8;               // padded LDS row (elements): 144 bytes
constexpr int kTileElems = BM * LDA;      // one operand tile in LDS

__global__ __launch_bounds__(kThreads, 1) void wkv_kernel_staged(WkvArgs p) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * 2 * kTileElems];  // [buf][A|W][256][LDA]

    int tm, tn;
    tile_coords(p, blockIdx.x, tm, tn);
    const int64_t m0 = static_cast<int64_t>(tm) * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    const int ld_row = tid >> 3;        // + 32 * i
    const int ld_col = (tid & 7) * 8;   // element offset inside the K slab
    const uint16_t* a_src[8];
    const uint16_t* w_src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int64_t m = m0 + ld_row + 32 * i;
        if (m >= p.M) m = p.M - 1;
        int n = n0 + ld_row + 32 * i;
        if (n >= p.N) n = p.N - 1;
        a_src[i] = p.lay[0].a + m * p.K + ld_col;
        w_src[i] = p.lay[0].w + static_cast<int64_t>(n) * p.K + ld_col;
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
    const int frag_off_a = (wm * 128 + (lane & 31)) * LDA + (lane >> 5) * 8;
    const int frag_off_w = kTileElems + (wn * 128 + (lane & 31)) * LDA + (lane >> 5) * 8;
    auto read_frags = [&](int buf, int kk, bf16x8* fa, bf16x8* fw) {
        const uint16_t* base = lds + buf * 2 * kTileElems + kk;
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(base + frag_off_a + i * 32 * LDA);
#pragma unroll
        for (int j = 0; j < 4; ++j) fw[j] = *reinterpret_cast<const bf16x8*>(base + frag_off_w + j * 32 * LDA);
    };

    f32x16 acc[4][4];
    zero(acc);
    bf16x8 fa0[4], fw0[4], fa1[4], fw1[4];
    const int KT = (p.K + BK - 1) / BK;
    load_slab(0);
    store_slab(0);
    __syncthreads();
    read_frags(0, 0, fa0, fw0);
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KT;
        if (more) load_slab((kt + 1) * BK);
        read_frags(cur, 16, fa1, fw1);
        mfma_step(acc, fa0, fw0);
        interleave_reads();
        read_frags(cur, 32, fa0, fw0);
        mfma_step(acc, fa1, fw1);
        interleave_reads();
        read_frags(cur, 48, fa1, fw1);
        mfma_step(acc, fa0, fw0);
        interleave_reads();
        if (more) store_slab(cur ^ 1);
        __syncthreads();
        if (more) read_frags(cur ^ 1, 0, fa0, fw0);
        mfma_step(acc, fa1, fw1);
        if (more) interleave_reads();
    }
    store_tile(p, acc, m0, n0, wm, wn, lane);
}

// ============================================================================
// gate finalize: the fused kernel's per-slice partial sums -> dot (fixed summation order)
// ============================================================================
// The finalize of every layer of a launch: blockIdx.y is the layer.
struct FinArgs {
    const float* part;    // layer 0's workspace; layer e's follows at e * part_stride floats
    int64_t part_stride;
    float* dot[kMaxLayers];
    int64_t M;
    int hc, slices;
    float eps, inv_dim, rsqrt_dim;
};

__global__ __launch_bounds__(256) void gate_finalize_kernel(FinArgs f) {
    const float* part = f.part + blockIdx.y * f.part_stride;
    float* dot = f.dot[blockIdx.y];
    const int64_t M = f.M;
    const int hc = f.hc, slices = f.slices;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= M * hc) return;
    const int c = static_cast<int>(idx / M);  // consecutive threads: consecutive tokens of one copy
    const int64_t t = idx - static_cast<int64_t>(c) * M;
    const float* src = part + static_cast<int64_t>(c) * slices * 3 * M + t;
    // The slices' loads go out in batches of kBatch (3 kBatch independent loads in flight per thread), so a
    // small launch pays a few memory latencies rather than one per slice; the sums still run in slice order.
    constexpr int kBatch = 20;
    float hwk = 0.f, kk = 0.f, hh = 0.f;
    int s0 = 0;
    for (; s0 + kBatch <= slices; s0 += kBatch) {
        float v[kBatch][3];
#pragma unroll
        for (int b = 0; b < kBatch; ++b)
#pragma unroll
            for (int q = 0; q < 3; ++q) v[b][q] = src[(3 * (s0 + b) + q) * M];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            hwk += v[b][0];
            kk += v[b][1];
            hh += v[b][2];
        }
    }
    for (; s0 < slices; ++s0) {
        hwk += src[(3 * s0 + 0) * M];
        kk += src[(3 * s0 + 1) * M];
        hh += src[(3 * s0 + 2) * M];
    }
    const float rstd = rsqrtf(hh * f.inv_dim + f.eps) * rsqrtf(kk * f.inv_dim + f.eps);
    dot[t * hc + c] = hwk * rstd * f.rsqrt_dim;
}

// The same for a launch with few (token, copy) pairs (a decode step: 1,024 pairs, 4 workgroups above): the
// slices of a pair are split over kGroups threads, kPer slices each, all their loads in flight at once
// (one memory latency), and the group sums are added through LDS in group order.  Workgroup: kGroups x 32
// consecutive tokens of one copy.
constexpr int kFinGroups = 8;
constexpr int kFinPer = 8;  // slices per thread at most: dim <= kFinGroups * kFinPer * 128
__global__ __launch_bounds__(256) void gate_finalize_split_kernel(FinArgs f) {
    __shared__ float red[kFinGroups][32][3];
    const float* part = f.part + blockIdx.y * f.part_stride;
    float* dot = f.dot[blockIdx.y];
    const int64_t M = f.M;
    const int hc = f.hc, slices = f.slices;
    const int g = threadIdx.x / 32, tl = threadIdx.x % 32;
    const int64_t nb = (M + 31) / 32;
    const int c = static_cast<int>(blockIdx.x / nb);
    const int64_t t = (blockIdx.x - static_cast<int64_t>(c) * nb) * 32 + tl;
    const int per = (slices + kFinGroups - 1) / kFinGroups;
    const int s0 = g * per;
    const float* src = part + static_cast<int64_t>(c) * slices * 3 * M + t;
    float v[kFinPer][3];
#pragma unroll
    for (int i = 0; i < kFinPer; ++i)
#pragma unroll
        for (int q = 0; q < 3; ++q)
            v[i][q] = (t < M && i < per && s0 + i < slices) ? src[(3 * (s0 + i) + q) * M] : 0.f;
    float sum[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kFinPer; ++i)
#pragma unroll
        for (int q = 0; q < 3; ++q) sum[q] += v[i][q];  // slice order inside the group (zeros past its end)
#pragma unroll
    for (int q = 0; q < 3; ++q) red[g][tl][q] = sum[q];
    __syncthreads();
    if (g != 0 || t >= M) return;
    float hwk = 0.f, kk = 0.f, hh = 0.f;
#pragma unroll
    for (int j = 0; j < kFinGroups; ++j) {  // group order
        hwk += red[j][tl][0];
        kk += red[j][tl][1];
        hh += red[j][tl][2];
    }
    const float rstd = rsqrtf(hh * f.inv_dim + f.eps) * rsqrtf(kk * f.inv_dim + f.eps);
    dot[t * hc + c] = hwk * rstd * f.rsqrt_dim;
}

}  // namespace

int launch_gate_finalize(const float* part, int64_t part_stride, float* const* dot, int layers, int64_t T, int hc,
                         int dim, float eps, hipStream_t stream, const char* what) {
    const int64_t blocks = (T * hc + 255) / 256;
    if (blocks > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "%s: too many tokens", what);
    FinArgs f = {};
    f.part = part;
    f.part_stride = part_stride;
    for (int e = 0; e < layers; ++e) f.dot[e] = dot[e];
    f.M = T;
    f.hc = hc;
    f.slices = dim / 128;
    f.eps = eps;
    f.inv_dim = 1.0f / static_cast<float>(dim);
    f.rsqrt_dim = static_cast<float>(1.0 / __builtin_sqrt(static_cast<double>(dim)));
    if (blocks * layers < kCUs && f.slices <= kFinGroups * kFinPer) {  // few pairs: one memory latency per pair
        const int64_t split_blocks = static_cast<int64_t>(hc) * ((T + 31) / 32);
        hipLaunchKernelGGL(gate_finalize_split_kernel, dim3(static_cast<unsigned>(split_blocks), layers), dim3(256),
                           0, stream, f);
    } else {
        hipLaunchKernelGGL(gate_finalize_kernel, dim3(static_cast<unsigned>(blocks), layers), dim3(256), 0, stream, f);
    }
    return check_launch(what);
}

}  // namespace engram

using namespace engram;

namespace {

// Tokens per tile of the main kernel: 256 (NI = 4), or 128 (NI = 2) when 128-token tiles of all the launch's
// layers still fit the CUs in one pass -- small launches (a decode step of one layer) then use twice the CUs.
int tile_ni(int64_t T, int tiles_n, int K, int layers) {
    return K >= 4 * BK && ((T + 127) / 128) * tiles_n * layers <= kCUs ? 2 : 4;
}

// Launch the persistent main kernel over all tiles of p's `layers` layers (p.tiles_n set; the M tiles here).
template <bool kGate>
int launch_main(WkvArgs& p, int64_t T, int layers, hipStream_t stream, const char* what) {
    const int ni = tile_ni(T, p.tiles_n, p.K, layers);
    // several short layers of the fused projection on 256-token tiles (under 32 waves of tiles each): one launch of
    // the 16 x 16 x 32 form (wkv16.hip) whose workgroups take every layer's key and value tiles, with no ramp or
    // tail between launches (a decode step of two layers: 3.69 -> 3.38 ms; the mid prefill 1.5 % faster).  Longer
    // layers run layer by layer below: in one launch the XCDs would work on several layers' W at once (2.4 %
    // slower at 65,536 tokens per layer).
    if constexpr (kGate) {
        const int64_t tiles_layer = (T + 255) / 256 * p.tiles_n;
        if (ni == 4 && layers > 1 && tiles_layer < 32 * kCUs && wkv16_layers_takes(T, p.K, p.hc, p.dim, layers)) {
            W16Layer lay[kW16MaxLayers];
            for (int e = 0; e < layers; ++e) {
                const LayerPtrs& L = p.lay[e];
                lay[e] = W16Layer{L.a, L.w, L.kv, L.x, L.q, L.k, L.part};
            }
            return launch_wkv16_layers(lay, layers, p.ld_out, T, p.K, p.hc, p.dim, stream, what);
        }
    }
    // 256-token tiles, three slabs or more and launches large enough: the 16 x 16 x 32 form (wkv16.hip), one
    // layer at a time
    if (ni == 4 && wkv16_takes(T, p.K, p.N, p.hc, p.dim, kGate)) {
        for (int e = 0; e < layers; ++e) {
            const LayerPtrs& L = p.lay[e];
            const int rc = launch_wkv16(L.a, L.w, L.kv, p.ld_out, T, p.K, p.N, L.x, L.q, L.k, L.part, p.hc, p.dim,
                                        kGate, stream, what);
            if (rc != ENGRAM_OK) return rc;
        }
        return ENGRAM_OK;
    }
    const int64_t bm = 64 * ni;
    const int64_t tiles_ml = (T + bm - 1) / bm;
    if (tiles_ml * layers * p.tiles_n > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "%s: too many tiles", what);
    p.tiles_ml = static_cast<int>(tiles_ml);
    p.tiles_m = static_cast<int>(tiles_ml * layers);
    const int64_t tiles = static_cast<int64_t>(p.tiles_m) * p.tiles_n;
    const unsigned grid = static_cast<unsigned>(tiles < kCUs ? tiles : kCUs);
    if (ni == 2 && tiles > kCUs) return fail(ENGRAM_EINVAL, "%s: one-tile launch with %lld tiles", what, (long long)tiles);
    if constexpr (kGate) {
        if (p.K == BK) {
            hipLaunchKernelGGL((wkv_kernel<true, 4, true>), dim3(grid), dim3(kMainThreads), 0, stream, p);
            return check_launch(what);
        }
    }
    if (ni == 2)
        hipLaunchKernelGGL((wkv_kernel<kGate, 2>), dim3(grid), dim3(kMainThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((wkv_kernel<kGate, 4>), dim3(grid), dim3(kMainThreads), 0, stream, p);
    return check_launch(what);
}

}  // namespace

extern "C" int engram_wkv(const uint16_t* a, const uint16_t* w, uint16_t* kv, int64_t T, int32_t K, int32_t Nout,
                          void* stream) {
    if (T < 0) return fail(ENGRAM_EINVAL, "engram_wkv: T < 0");
    if (K < 8 || K % 8 != 0) return fail(ENGRAM_EINVAL, "engram_wkv: K=%d must be a positive multiple of 8", K);
    if (Nout < 8 || Nout % 8 != 0) return fail(ENGRAM_EINVAL, "engram_wkv: Nout=%d must be a positive multiple of 8", Nout);
    if (T == 0) return ENGRAM_OK;
    if (!a || !w || !kv) return fail(ENGRAM_EINVAL, "engram_wkv: null pointer");
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(kv, 16)) return fail(ENGRAM_EINVAL, "engram_wkv: misaligned pointer");
    WkvArgs p = {};
    p.lay[0].a = a;
    p.lay[0].w = w;
    p.lay[0].kv = kv;
    p.M = T;
    p.N = Nout;
    p.K = K;
    p.ld_out = Nout;
    p.out_col0 = 0;
    p.tiles_n = (Nout + BN - 1) / BN;
    if (K % BK == 0) return launch_main<false>(p, T, 1, as_stream(stream), "engram_wkv");
    {
        const int64_t tiles_m = (T + BM - 1) / BM;
        if (tiles_m * p.tiles_n > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "engram_wkv: too many tiles");
        p.tiles_m = static_cast<int>(tiles_m);
        p.tiles_ml = p.tiles_m;
        const int64_t tiles = tiles_m * p.tiles_n;
        hipLaunchKernelGGL(wkv_kernel_staged, dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0,
                           as_stream(stream), p);
    }
    return check_launch("engram_wkv");
}

extern "C" int64_t engram_wkv_gate_workspace_bytes(int64_t T, int32_t hc, int32_t dim) {
    if (T < 0 || hc < 1 || hc > 64 || dim < 256 || dim % 256 != 0) return -1;
    return static_cast<int64_t>(hc) * (dim / 128) * 3 * T * static_cast<int64_t>(sizeof(float));
}

// ---- the allocation-free form: the partial sums live in a file-scope device array ----
// Each GPU the library runs on holds its own copy of `scratch` until the process ends.  In host code the
// array's name is only a stand-in for the symbol: its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device and kept below.
namespace {

static __device__ __align__(256) float scratch[ENGRAM_NOALLOC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// the device address of `scratch` on the current GPU (looked up on the first call made on that GPU)
int scratch_address(void** out, const char* what) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ENGRAM_EHIP, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(ENGRAM_EINVAL, "%s: device %d outside [0, %d)", what, dev, kMaxDevices);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p)
                return fail(ENGRAM_EHIP, "%s: hipGetSymbolAddress(scratch): %s", what, hipGetErrorString(e));
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return ENGRAM_OK;
}

// engram_wkv_gate over `layers` layers in one launch of the main kernel and one of the finalize; arrays of
// `layers` entries (host memory).  The workspace holds the layers' partial sums one after another.
// `static_scratch`: the workspace is the library's `scratch` array (workspace and workspace_bytes ignored),
// whose address is looked up only once every argument has been checked.
int wkv_gate_entry(const char* what, int layers, const uint16_t* const* a, const uint16_t* const* w,
                   const uint16_t* const* x, const uint16_t* const* q_weight, const uint16_t* const* k_weight,
                   float eps, uint16_t* const* value, int64_t ld_value, float* const* dot, void* workspace,
                   int64_t workspace_bytes, int64_t T, int32_t K, int32_t hc, int32_t dim, void* stream,
                   bool static_scratch = false) {
    if (T < 0) return fail(ENGRAM_EINVAL, "%s: T < 0", what);
    if (K < BK || K % BK != 0) return fail(ENGRAM_EINVAL, "%s: K=%d must be a positive multiple of %d", what, K, BK);
    if (hc < 1 || hc > 64) return fail(ENGRAM_EINVAL, "%s: hc=%d outside [1, 64]", what, hc);
    if (dim < 256 || dim % 256 != 0)
        return fail(ENGRAM_EINVAL, "%s: dim=%d must be a positive multiple of 256", what, dim);
    if (ld_value < dim || ld_value % 8 != 0)
        return fail(ENGRAM_EINVAL, "%s: ld_value=%lld must be >= dim and a multiple of 8", what, (long long)ld_value);
    const int64_t per_layer = engram_wkv_gate_workspace_bytes(T, hc, dim);
    const int64_t need = per_layer * layers;
    if (static_scratch) {
        if (need > ENGRAM_NOALLOC_SCRATCH_BYTES)
            return fail(ENGRAM_ERANGE, "%s: %d layer(s) of T=%lld need %lld bytes of partial sums, more than the %lld "
                        "bytes of scratch this entry point holds (engram_wkv_gate_layers takes a workspace)", what,
                        layers, (long long)T, (long long)need, (long long)ENGRAM_NOALLOC_SCRATCH_BYTES);
    } else if (workspace_bytes < need) {
        return fail(ENGRAM_ERANGE, "%s: workspace of %lld bytes, %lld needed", what, (long long)workspace_bytes,
                    (long long)need);
    }
    if (T == 0) return ENGRAM_OK;
    if (!static_scratch && !workspace) return fail(ENGRAM_EINVAL, "%s: null pointer", what);
    if (!static_scratch && !aligned(workspace, 16)) return fail(ENGRAM_EINVAL, "%s: misaligned pointer", what);
    const int Nout = (hc + 1) * dim;
    WkvArgs p = {};
    for (int e = 0; e < layers; ++e) {
        if (!a[e] || !w[e] || !x[e] || !q_weight[e] || !k_weight[e] || !value[e] || !dot[e])
            return fail(ENGRAM_EINVAL, "%s: layer %d: null pointer", what, e);
        if (!aligned(a[e], 16) || !aligned(w[e], 16) || !aligned(x[e], 16) || !aligned(q_weight[e], 16) ||
            !aligned(k_weight[e], 16) || !aligned(value[e], 16) || !aligned(dot[e], 4))
            return fail(ENGRAM_EINVAL, "%s: layer %d: misaligned pointer", what, e);
    }
    if (static_scratch) {
        const int rc = scratch_address(&workspace, what);
        if (rc != ENGRAM_OK) return rc;
    }
    for (int e = 0; e < layers; ++e) {
        LayerPtrs& L = p.lay[e];
        L.a = a[e];
        L.w = w[e];
        L.kv = value[e];
        L.x = x[e];
        L.q = q_weight[e];
        L.k = k_weight[e];
        L.part = static_cast<float*>(workspace) + e * (per_layer / static_cast<int64_t>(sizeof(float)));
    }
    p.M = T;
    p.N = Nout;
    p.K = K;
    p.ld_out = ld_value;
    p.out_col0 = hc * dim;
    p.hc = hc;
    p.dim = dim;
    p.tiles_n = Nout / BN;
    int rc = launch_main<true>(p, T, layers, as_stream(stream), what);
    if (rc != ENGRAM_OK) return rc;
    return launch_gate_finalize(static_cast<const float*>(workspace), per_layer / static_cast<int64_t>(sizeof(float)),
                                dot, layers, T, hc, dim, eps, as_stream(stream), what);
}

}  // namespace

extern "C" int engram_wkv_gate(const uint16_t* a, const uint16_t* w, const uint16_t* x, const uint16_t* q_weight,
                               const uint16_t* k_weight, float eps, uint16_t* value, int64_t ld_value, float* dot,
                               void* workspace, int64_t workspace_bytes, int64_t T, int32_t K, int32_t hc,
                               int32_t dim, void* stream) {
    return wkv_gate_entry("engram_wkv_gate", 1, &a, &w, &x, &q_weight, &k_weight, eps, &value, ld_value, &dot,
                          workspace, workspace_bytes, T, K, hc, dim, stream);
}

extern "C" int engram_wkv_gate_layers_noalloc(int32_t layers, const uint16_t* const* a, const uint16_t* const* w,
                                              const uint16_t* const* x, const uint16_t* const* q_weight,
                                              const uint16_t* const* k_weight, float eps, uint16_t* const* value,
                                              int64_t ld_value, float* const* dot, int64_t T, int32_t K, int32_t hc,
                                              int32_t dim, void* stream) {
    const char* what = "engram_wkv_gate_layers_noalloc";
    if (layers < 1 || layers > kMaxLayers)
        return fail(ENGRAM_EINVAL, "%s: layers=%d outside [1, %d]", what, layers, kMaxLayers);
    if (T > 0 && (!a || !w || !x || !q_weight || !k_weight || !value || !dot))
        return fail(ENGRAM_EINVAL, "%s: null pointer array", what);
    return wkv_gate_entry(what, layers, a, w, x, q_weight, k_weight, eps, value, ld_value, dot, nullptr, 0, T, K, hc,
                          dim, stream, true);
}

extern "C" int engram_wkv_gate_layers(int32_t layers, const uint16_t* const* a, const uint16_t* const* w,
                                      const uint16_t* const* x, const uint16_t* const* q_weight,
                                      const uint16_t* const* k_weight, float eps, uint16_t* const* value,
                                      int64_t ld_value, float* const* dot, void* workspace, int64_t workspace_bytes,
                                      int64_t T, int32_t K, int32_t hc, int32_t dim, void* stream) {
    const char* what = "engram_wkv_gate_layers";
    if (layers < 1 || layers > kMaxLayers)
        return fail(ENGRAM_EINVAL, "%s: layers=%d outside [1, %d]", what, layers, kMaxLayers);
    if (T > 0 && (!a || !w || !x || !q_weight || !k_weight || !value || !dot))
        return fail(ENGRAM_EINVAL, "%s: null pointer array", what);
    return wkv_gate_entry(what, layers, a, w, x, q_weight, k_weight, eps, value, ld_value, dot, workspace,
                          workspace_bytes, T, K, hc, dim, stream);
}
