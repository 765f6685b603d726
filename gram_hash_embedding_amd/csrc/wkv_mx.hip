// The `wkv` Linear on fp8 block-scaled operands (the released config's "dtype": "fp8"; DeepSeek V4.1
// "stack-hashes" page: the config block and Engram.__init__), in the OCP microscaling (MX) fp8 format:
// E4M3FN elements, one E8M0 scale per 32 consecutive input columns of a row.
//
//   engram_mx_quant  -- bf16 rows -> MX fp8 (the activation side of the fp8 Linear; also the weights' one-off
//                       conversion): shared exponent floor(log2 amax) - 8 per 32 columns, elements rounded to
//                       nearest even and saturated at 448
//   engram_wkv_mx    -- kv = A * W^T with v_mfma_scale_f32_32x32x64_f8f6f4 (the block scales applied by the
//                       matrix core), fp32 accumulation, one bf16 rounding
//   engram_wkv_mx_gate -- engram_wkv_mx fused with the gate pre-activation (Engram.forward's rstd and dot):
//                       the key columns reduced against the stream in the kernel's epilogue, the value columns
//                       stored, the bf16 path's finalize (wkv.hip) adding the partial sums
//
// Scale layout (both operands): uint8 [K/128][rows4][4], rows4 = rows rounded up to a multiple of 4; byte
// [s][r][b] scales row r's columns 128 s + 32 b .. +32.  A 128-column slab of a 256-row tile then has its
// scales in one contiguous kilobyte, loaded with the slab by one 16-byte-per-lane direct-to-LDS load.
//
// Design (gfx950): the bf16 projection's persistent design (wkv.hip) with fp8 slabs -- 256 x 256 tiles, eight
// waves (two per SIMD, loader waves 0-3 issue every slab load, storer waves 4-7 every store), slabs of 128
// fp8 columns (128-byte rows, the same XOR swizzle as the bf16 slabs of 64 columns) in two stages, XCD-grouped
// tile order.  A stage holds 66 KB (A and W slabs and their scales), so the epilogue exchange is 16 KB and
// runs in eight rounds of 32 tokens x 128 outputs per wave pair -- or, at K >= 384, a tile's last two slabs
// hold back the next tile's first two and the tile leaves in one round through both freed stages (the fused
// kernel's stream rows use them the same way).  Each wave: 128 tokens x 64 outputs = 4 x 2
// MFMA blocks of 32x32 (K 64 per MFMA: two per slab).  Lane l of a 32x32x64 fragment holds row l % 32: in
// its first 16 bytes columns 16h .. 16h + 15 and in its last 16 bytes columns 32 + 16h .. 32 + 16h + 15 of
// the step (h = l / 32); the scale operand of lane half h scales the step's 32-column block h of the row (the
// first 16 bytes of both halves, or the last 16) -- measured on gfx950.  Each lane's slab scale word (byte b:
// block b of the slab) is shifted right by 8 h, and k-step s takes byte 2 s.
#include <type_traits>
#include <utility>

#include "common.h"
#include "mx.h"

namespace engram {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256;
constexpr int kSlabCols = 128;              // fp8 columns (= bytes) per slab row
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kOpBytes = 256 * kSlabCols;   // one operand's slab: 32 KB
constexpr int kScBytes = 256 * 4;           // its scales: 1 KB
constexpr int kStageBytes = 2 * kOpBytes + 2 * kScBytes;
constexpr int kExBytes = 64 * 256;          // epilogue exchange: 64 token rows x 128 outputs (bf16)
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
constexpr int kCUs = 256;
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNonTemporal = 2;             // cache-policy operand of a global load: streamed past L2
constexpr int kXArea = 32 * 128;            // fused gate: a wave's stream rows of one round (32 tokens x 64 bf16)
constexpr int kWaitLgkmcnt0 = 0xC07F;
constexpr int wait_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

struct MxArgs {
    const uint8_t* a;    // [M, K] e4m3
    const uint8_t* as;   // [K/128][M4][4] e8m0
    const uint8_t* w;    // [N, K] e4m3
    const uint8_t* ws;   // [K/128][N4][4] e8m0
    uint16_t* kv;        // [M, ld_out] bf16
    int64_t M;
    int N, K;
    int64_t M4, N4;      // rows of the scale layouts (multiples of 4)
    int tiles_m, tiles_n;
    int64_t ld_out;
    // the fused gate (kGate): every tile's columns are key columns, reduced against the stream, not stored
    const uint16_t* x;   // [M, hc, dim] bf16
    const uint16_t* q;   // [hc, dim] bf16
    const uint16_t* k;   // [hc, dim] bf16
    float* part;         // [hc][dim/128][3][M] fp32: per 128-column slice pair sum(h w key), sum(key^2), sum(h^2)
    int hc, dim;
};

// pid -> (tm, tn): contiguous runs per XCD (pid % 8 is the XCD a workgroup lands on), grouped kGroupM deep
__device__ inline void tile_coords(const MxArgs& p, int pid, int& tm, int& tn) {
    const int n = p.tiles_m * p.tiles_n;
    const int xcd = pid % kXcds, idx = pid / kXcds;
    const int per = n / kXcds, rem = n % kXcds;
    const int logical = xcd * per + min(xcd, rem) + idx;
    const int in_group = kGroupM * p.tiles_n;
    const int group = logical / in_group;
    const int first_m = group * kGroupM;
    const int gsize = min(p.tiles_m - first_m, kGroupM);
    const int r = logical - group * in_group;
    tm = first_m + r % gsize;
    tn = r / gsize;
}

__device__ inline int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
// The lane's index formed where it is used: opaque, so the compiler neither hoists it nor keeps what is derived
// from it live across the slab loop.  With every VGPR taken such loop-invariant values are spilled, and the
// reload of one waits (vmcnt is in order) for every load in flight, the slab just issued included.
__device__ inline int lane_here() {
    int v;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
    return v;
}

__device__ inline uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

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

// Kernel modes.  kStream: the slab loads stream across tile boundaries and each tile is stored through the
// 16 KB exchange in eight rounds (any K).  kHold: a tile's last two slabs hold back the next tile's first two,
// so both stages are free at its end and the whole tile is stored in one round through them (K >= 384).
// kGate: kHold's loop over the key columns only, every tile reduced against the stream in its epilogue
// instead of stored (the fused projection + gate pre-activation; the value columns are a launch of their own).
constexpr int kStream = 0, kHold = 1, kGate = 2;

template <int kMode>
__device__ __forceinline__ void wkv_mx_body(const MxArgs& p) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStageBytes + kExBytes];
    const int tiles = p.tiles_m * p.tiles_n;
    const int G = gridDim.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const bool loader = wave < 4;
    const int KT = p.K / kSlabCols;
    const int row_bytes = p.K;

    auto sync = [&]() {
        __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto sync_epi = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        sync();
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- slab loads (loader waves): wave w fills rows [64w, 64w+64) of the A and of the W slab, 8 rows per
    // instruction, lane l at slot (l & 7) of row base + 8q + (l >> 3), fetching the piece the swizzle puts
    // there; wave 0 also loads the A slab's scales (1 KB), wave 1 the W slab's.  Rows past M or N fall outside
    // their resource and read as zero.
    const int ld_r = lane >> 3, ld_slot = lane & 7;
    const uint32_t vo_piece = static_cast<uint32_t>(ld_r * row_bytes + ((ld_slot ^ (ld_r >> 1)) << 4));
    const uint32_t vo_rows = vo_piece + static_cast<uint32_t>(wave * 64 * row_bytes);
    struct SlabRsrc {
        __amdgpu_buffer_rsrc_t ra, rw, rs;
        uint32_t k0b;
    };
    // a tile of this workgroup: its first row and column; `live` false past the workgroup's last tile, whose
    // loads are then empty (the resources hold no bytes)
    struct TileAt {
        int64_t m0;
        int n0;
        bool live;
    };
    auto slab_rsrc = [&](const TileAt& ta, int kt) {
        const int64_t m0 = ta.m0;
        const int n0 = ta.n0;
        const bool live = ta.live;
        const int a_bytes = live ? static_cast<int>(min<int64_t>(BM, p.M - m0)) * row_bytes : 0;
        const int w_bytes = live ? min(BN, p.N - n0) * row_bytes : 0;
        SlabRsrc r;
        r.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a + m0 * p.K), 0, a_bytes, kBufferWord3);
        r.rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.w + static_cast<int64_t>(n0) * p.K), 0, w_bytes,
                                                 kBufferWord3);
        // slab kt's scales of the tile's 256 rows: bytes [(kt * rows4 + row0) * 4, +1024) of the layout (wave 0:
        // the A side, wave 1: the W side)
        const uint8_t* sbase = wave == 0 ? p.as : p.ws;
        const int64_t rows4 = wave == 0 ? p.M4 : p.N4;
        const int64_t row0 = wave == 0 ? m0 : n0;
        const int valid = live ? static_cast<int>(min<int64_t>(256, rows4 - row0)) * 4 : 0;
        r.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sbase + (static_cast<int64_t>(kt) * rows4 + row0) * 4),
                                                 0, valid, kBufferWord3);
        r.k0b = static_cast<uint32_t>(kt * kSlabCols);
        return r;
    };
    // part q (0..7) of a slab's loads: rows 8q..8q+7 of the wave's A and W rows (2 loads); part 0 of waves 0
    // and 1 also the scales (1 load)
    auto issue_part = [&](const SlabRsrc& r, int stage, int q) {
        uint8_t* st = lds + stage * kStageBytes;
        const uint32_t flip = (q & 1) ? (4u << 4) : 0u;
        const uint32_t qrows = static_cast<uint32_t>(q * 8 * row_bytes);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r.ra, st + (wave * 64 + q * 8) * 128, 16, (vo_rows ^ flip) + qrows,
                                                 r.k0b, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r.rw, st + kOpBytes + (wave * 64 + q * 8) * 128, 16,
                                                 (vo_rows ^ flip) + qrows, r.k0b, 0, 0);
        if (q == 0 && wave < 2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r.rs, st + 2 * kOpBytes + wave * kScBytes, 16,
                                                     static_cast<uint32_t>(lane_here() * 16), 0, 0, 0);
    };
    auto issue_slab = [&](const TileAt& ta, int kt, int stage) {
        const SlabRsrc r = slab_rsrc(ta, kt);
#pragma unroll
        for (int q = 0; q < 8; ++q) issue_part(r, stage, q);
    };

    // ---- fragments: lane reads row (lane % 32) of a 32-row block, for k-step s (columns 64s .. 64s + 63):
    // bytes 0-15 of the fragment hold columns 64s + 16h .. +15 and bytes 16-31 columns 64s + 32 + 16h .. +15
    // (h = lane / 32), i.e. pieces 4s + h and 4s + 2 + h, each at its swizzled slot.  So the first 16 bytes
    // of both lane halves form the step's first 32-column block and the last 16 bytes its second: the scale
    // operand of lane half h is the row's scale of block 2s + h.
    const int h = lane >> 5;
    const int g = (lane >> 1) & 7;  // swizzle key of the lane's rows (blocks start at multiples of 16 rows)
    const int a_row = (wm * 128 + (lane & 31)) * 128;
    const int w_row = kOpBytes + (wn * 64 + (lane & 31)) * 128;
    auto read_piece = [&](int stage, int s, int row_off) -> i32x8 {
        const uint8_t* base = lds + stage * kStageBytes + row_off;
        const u32x4 x0 = *reinterpret_cast<const u32x4*>(base + (((4 * s + h) ^ g) << 4));
        const u32x4 x1 = *reinterpret_cast<const u32x4*>(base + (((4 * s + 2 + h) ^ g) << 4));
        return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    };
    auto read_a = [&](int stage, int s, int i) { return read_piece(stage, s, a_row + i * 32 * 128); };
    auto read_w = [&](int stage, int s, int j) { return read_piece(stage, s, w_row + j * 32 * 128); };
    // the slab's scale words of the lane's rows (raw); shift_scales then moves the lane's K half of k-step 0 /
    // k-step 1 into byte 0 / byte 2
    auto read_scales = [&](int stage, uint32_t* sa, uint32_t* sw) {
        const uint8_t* base = lds + stage * kStageBytes + 2 * kOpBytes + (lane_here() & 31) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = *reinterpret_cast<const uint32_t*>(base + (wm * 128 + i * 32) * 4);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            sw[j] = *reinterpret_cast<const uint32_t*>(base + kScBytes + (wn * 64 + j * 32) * 4);
    };
    auto shift_scales = [&](uint32_t* sa, uint32_t* sw) {
        const int sh = 8 * h;
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] >>= sh;
#pragma unroll
        for (int j = 0; j < 2; ++j) sw[j] >>= sh;
    };

    // ---- epilogue: 8 rounds (4 token blocks x 2 column halves); in round (i, hf) the waves of column half hf
    // (wn >> 1 == hf) put tokens 32i..32i+31 x their 64 outputs into the exchange (64 rows of 256 B, row
    // 32 wm + t, 16-byte pieces XOR-swizzled by row), then the storer waves write 16 rows each with full-line,
    // non-temporal 16-byte stores
    uint8_t* ex = lds + 2 * kStageBytes;
    auto epilogue = [&](const f32x16 (&acc)[4][2], int64_t m0, int n0) {
        const int l = lane_id();
        const int key = l & 15;
        const uint32_t wbase = static_cast<uint32_t>((wm * 32 + (l & 31)) * 256 + (l >> 5) * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                if ((wn >> 1) == hf) {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int gq = 0; gq < 4; ++gq) {
                            const int chunk = (wn & 1) * 8 + 4 * j + gq;
                            const u32x2 v = {pack_bf16(acc[i][j][4 * gq + 0], acc[i][j][4 * gq + 1]),
                                             pack_bf16(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3])};
                            *reinterpret_cast<u32x2*>(ex + wbase + ((chunk ^ key) << 4)) = v;
                        }
                }
                sync_epi();
                if (!loader) {
                    const int s = wave - 4;
                    const int ls = lane_id();
                    const int chunk = ls & 15;
                    const int ncol = n0 + hf * 128 + chunk * 8;
#pragma unroll
                    for (int ins = 0; ins < 4; ++ins) {
                        const int rr = 16 * s + 4 * ins + (ls >> 4);  // exchange row: token half rr / 32
                        const u32x4 v = *reinterpret_cast<const u32x4*>(ex + rr * 256 + ((chunk ^ (rr & 15)) << 4));
                        const int64_t m = m0 + (rr >> 5) * 128 + 32 * i + (rr & 31);
                        if (m < p.M && ncol < p.N)
                            __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p.kv + m * p.ld_out + ncol));
                    }
                }
                sync_epi();
            }
        }
    };

    // ---- one-round epilogue of a held-back tile (kHold): both stages are free.  Every wave writes its 128
    // tokens x 64 outputs as bf16 into stage wm (row t: token 128 wm + t, 512 bytes = the tile's 256 outputs,
    // 16-byte piece c at slot c ^ (t % 32)); after a barrier the storer waves read 64 rows each and write them
    // with full-line non-temporal 16-byte stores (two rows per instruction), and a second barrier frees the
    // stages for the held-back slabs.  The stores drain while the next tile computes.
    auto store_epilogue = [&](const f32x16 (&acc)[4][2], int64_t m0, int n0) {
        const int l = lane_id();
        uint8_t* sb = lds + wm * kStageBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 32 * i + (l & 31);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const int c = wn * 8 + 4 * j + gq;  // the 16-byte piece of the row (8 outputs)
                    const u32x2 v = {pack_bf16(acc[i][j][4 * gq + 0], acc[i][j][4 * gq + 1]),
                                     pack_bf16(acc[i][j][4 * gq + 2], acc[i][j][4 * gq + 3])};
                    *reinterpret_cast<u32x2*>(sb + t * 512 + ((c ^ (t & 31)) << 4) + (l >> 5) * 8) = v;
                }
        }
        sync_epi();
        if (!loader) {
            const int s = wave - 4;
            const int c = l & 31;
            const int ncol = n0 + 8 * c;
#pragma unroll 4
            for (int ins = 0; ins < 32; ++ins) {
                const int r = 64 * s + 2 * ins + (l >> 5);  // row of the tile: token m0 + r
                const u32x4 v = *reinterpret_cast<const u32x4*>(lds + (r >> 7) * kStageBytes + (r & 127) * 512 +
                                                               ((c ^ (r & 31)) << 4));
                const int64_t m = m0 + r;
                if (m < p.M && ncol < p.N)
                    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p.kv + m * p.ld_out + ncol));
            }
        }
        sync_epi();
    };

    // ---- fused gate epilogue of a key tile (kGate): the product is not stored.  The tile's 256 columns lie in
    // one copy c; wave (wm, wn) owns the 64-column slice (n0 - c dim) / 64 + wn of that copy and tokens
    // [128 wm, +128).  Lane l holds, in round i < 4, token 32i + l%32 and 32 of the slice's columns (4
    // consecutive ones per (j, gq), as the MFMA leaves them).  Each accumulator is rounded to bf16 (the product
    // is a bf16 tensor before it is used) and reduced against the stream's matching element: sum(h w key),
    // sum(key^2), sum(h^2) over the lane's columns, then over the two lane halves.  The stream rows come in by
    // direct-to-LDS loads that the tile's last two slabs issue (they hold back the next tile's first two, so
    // each stage is free from the barrier of the slab that read it last): the second-to-last slab fetches the
    // slice's q and k elements and rounds 2 and 3 into its own stage, the last slab rounds 0 and 1 into its
    // own, st.  Round r: stage st (r < 2) or st ^ 1, at (r & 1) * 32 KB, the wave's 4 KB area; row t is token
    // 32 r + t of the wave's 128, 16-byte piece q at slot q ^ ((t >> 1) & 7).  Each wave waits only for its own
    // loads.  Loader waves hand their sums to their SIMD partner (storer wave w + 4: the same tokens, the slice
    // 128 columns to the right), which adds them to its own and stores one value per (copy, pair of slices,
    // token).
    auto own_wait = [&](auto n_tag) {  // this wave's own loads down to n outstanding; LDS reads stay after it
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(decltype(n_tag)::value));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto lds_fence = [&]() {  // this wave's LDS reads are done
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto round_base = [&](int r, int st) { return lds + (r < 2 ? st : st ^ 1) * kStageBytes + (r & 1) * 8 * kXArea; };
    // The stream rows of this wave's 128 tokens and 64 columns through a buffer resource based at token
    // m0 + 128 wm, column n0 + 64 wn of x ([M, hc dim] bf16; the key columns n0 + 64 wn .. +63 of copy c are
    // x's columns of the same numbers): tokens past M fall outside it and read as zero.  Lane l loads row l / 8
    // of an 8-row group, the 16-byte piece its slot l % 8 holds under the swizzle: x_voff, flipped by 64 bytes
    // for odd groups (the swizzle key of group g's rows is 4 g + l / 16, mod 8).
    const uint32_t x_row_bytes = static_cast<uint32_t>(p.hc * p.dim * 2);  // < 2^24
    const uint32_t x_voff = (lane >> 3) * x_row_bytes + (((lane & 7) ^ (lane >> 4)) << 4);
    auto x_rsrc = [&](int64_t m0, int n0) {
        const int64_t t0 = m0 + wm * 128;
        const int64_t rows = min<int64_t>(128, p.M - t0);
        const int64_t col = n0 + wn * 64;
        const int bytes = rows > 0 ? static_cast<int>(rows * x_row_bytes - 2 * col) : 0;  // < 2^31
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.x + t0 * (x_row_bytes / 2) + col), 0, bytes,
                                                 kBufferWord3);
    };
    // load `ins` (0..3) of round r: rows 8 ins .. 8 ins + 7 of the round's 32 tokens (the whole offset in the
    // range-checked VGPR operand; the host keeps 128 rows of x under 2^31 bytes)
    auto dma_piece = [&](__amdgpu_buffer_rsrc_t xr, int r, int ins, int st) {
        uint32_t v = x_voff;
        asm volatile("" : "+v"(v));  // formed here, not hoisted out of the tile loop as 8 live registers
        const uint32_t voff = ((ins & 1) ? (v ^ 64u) : v) + static_cast<uint32_t>(32 * r + 8 * ins) * x_row_bytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, round_base(r, st) + wave * kXArea + ins * 1024, 16, voff, 0, 0,
                                                 kNonTemporal);
    };
    // the slice's 64 q and 64 k elements into the wave's 512 bytes of the exchange area (unused by the fused
    // kernel): q column j at byte 2 j, k column j at 256 + 2 j; two loads of 4 bytes a lane whose upper 32
    // lanes fall outside their 128-byte resource
    auto dma_qk = [&](int n0, int which) {
        const uint16_t* src = (which == 0 ? p.q : p.k) + (n0 + wn * 64);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), 0, 128, kBufferWord3),
            ex + wave * 512 + which * 256, 4, static_cast<uint32_t>(lane * 4), 0, 0, 0);
    };
    // The accumulators of a key tile whose last two slabs issued, in this order, the q and k loads and rounds 2
    // and 3 (10 loads), then rounds 0 and 1 (8 loads): rounds 2 and 3 are reduced first.
    auto gate_epilogue = [&](const f32x16 (&acc)[4][2], int64_t m0, int n0, int st) {
        const int l = lane_id();
        const int c = n0 / p.dim;
        own_wait(std::integral_constant<int, 8>{});  // q, k and rounds 2 and 3 (rounds 0 and 1 may fly)
        // q * k (exact in fp32) for the lane's 32 columns
        float wgt[2][4][4];
        {
            const uint8_t* qk = ex + wave * 512 + 8 * (l >> 5);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq) {
                    const u32x2 qv = *reinterpret_cast<const u32x2*>(qk + 2 * (32 * j + 8 * gq));
                    const u32x2 kv = *reinterpret_cast<const u32x2*>(qk + 256 + 2 * (32 * j + 8 * gq));
                    wgt[j][gq][0] = lo_bf16(qv[0]) * lo_bf16(kv[0]);
                    wgt[j][gq][1] = hi_bf16(qv[0]) * hi_bf16(kv[0]);
                    wgt[j][gq][2] = lo_bf16(qv[1]) * lo_bf16(kv[1]);
                    wgt[j][gq][3] = hi_bf16(qv[1]) * hi_bf16(kv[1]);
                }
        }
        float res[4][3];
        auto reduce = [&](auto i_tag) {
            constexpr int i = decltype(i_tag)::value;
            const uint8_t* xl = round_base(i, st) + wave * kXArea;
            u32x2 xr[2][4];
            {
                const int rr = l & 31, hx = l >> 5;
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq)
                        xr[j][gq] = *reinterpret_cast<const u32x2*>(
                            xl + rr * 128 + (((4 * j + gq) ^ ((rr >> 1) & 7)) << 4) + hx * 8);
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
        };
        reduce(std::integral_constant<int, 2>{});
        reduce(std::integral_constant<int, 3>{});
        own_wait(std::integral_constant<int, 4>{});
        reduce(std::integral_constant<int, 0>{});
        own_wait(std::integral_constant<int, 0>{});
        reduce(std::integral_constant<int, 1>{});
        // hand-over: a loader wave leaves its sums in its own area of round 1 (read out above); its SIMD partner
        // adds them to its own and stores both
        uint8_t* const hand = round_base(1, st);
        if (loader) {
            lds_fence();
            if (l < 32) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int q = 0; q < 3; ++q)
                        reinterpret_cast<float*>(hand + wave * kXArea)[(i * 3 + q) * 32 + l] = res[i][q];
            }
        }
        sync_epi();
        if (!loader && l < 32) {
            // the storer adds its partner's sums (slice wn - 2 of the tile) to its own (slice wn): one value per
            // (copy, 128-column slice pair, token), always summed in this order
            const float* partner = reinterpret_cast<const float*>(hand + (wave - 4) * kXArea);
            const int64_t tbase = m0 + wm * 128 + l;
            const int pair = (n0 - c * p.dim) / 128 + (wn - 2);
            float* out = p.part + (static_cast<int64_t>(c) * (p.dim / 128) + pair) * 3 * p.M;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t t = tbase + 32 * i;
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    const float v = res[i][q] + partner[(i * 3 + q) * 32 + l];
                    if (t < p.M) __builtin_nontemporal_store(v, out + q * p.M + t);
                }
            }
        }
        sync_epi();  // the partner's sums, the stream rows and q and k are read before the stages are refilled
    };

    if (static_cast<int>(blockIdx.x) >= tiles) return;
    const int my_tiles = (tiles - 1 - static_cast<int>(blockIdx.x)) / G + 1;
    // this workgroup's tile t (its tile coordinates are computed once per tile, not per slab: their integer
    // divisions run on the scalar unit)
    auto tile_at = [&](int t) {
        int tm, tn;
        tile_coords(p, static_cast<int>(blockIdx.x) + (t < my_tiles ? t : 0) * G, tm, tn);
        return TileAt{static_cast<int64_t>(tm) * BM, tn * BN, t < my_tiles};
    };

    // One k-step: acc[i][j] += (W fragment j) x (A fragment i) scaled by byte kSel of the lane's scale words,
    // in W-fragment-major order; each fragment is reloaded, for k-step `ns` of stage `nst`, right after its last
    // use here (one set of 48 fragment registers; every reload is issued three or more MFMAs before its use).
    // Each MFMA with its reloads and `extra(u)` (u = 0..7: a share of the slab loads) is one scheduling unit.
    // kReload false (the last slab of a fused key tile): no reloads, the fragments are dead after the k-step.
    auto kstep = [&](auto sel_tag, auto zero_tag, f32x16 (&acc)[4][2], i32x8 (&fa)[4], i32x8 (&fw)[2],
                     const uint32_t* sa, const uint32_t* sw, int nst, int ns, auto&& extra, auto reload_tag) {
        constexpr int kSel = decltype(sel_tag)::value;
        constexpr bool kZero = decltype(zero_tag)::value;
        constexpr bool kReload = decltype(reload_tag)::value;
        const f32x16 z = {};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[i][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[0], fa[i], kZero ? z : acc[i][0], 0, 0,
                                                                        kSel, sw[0], kSel, sa[i]);
            if (kReload && i == 3) fw[0] = read_w(nst, ns, 0);
            extra(i);
            asm volatile("" ::: "memory");  // keeps the unit's LDS reads and loads in the unit
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[i][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[1], fa[i], kZero ? z : acc[i][1], 0, 0,
                                                                        kSel, sw[1], kSel, sa[i]);
            if (kReload) fa[i] = read_a(nst, ns, i);
            if (kReload && i == 3) fw[1] = read_w(nst, ns, 1);
            extra(4 + i);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto no_extra = [](int) {};

    auto run = [&](auto loader_tag) {
        constexpr bool kLoader = decltype(loader_tag)::value;
        // the workgroup's tiles t and t + 1
        TileAt cur = tile_at(0), nx1 = tile_at(1);
        if (kLoader) {
            issue_slab(cur, 0, 0);
            if (KT > 1)
                issue_slab(cur, 1, 1);
            else
                issue_slab(nx1, 0, 1);
            __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
        }
        sync();
        f32x16 acc[4][2];
        i32x8 fa[4], fw[2];
        uint32_t sa[4], sw[2];
        int stage = 0;
        read_scales(0, sa, sw);
        shift_scales(sa, sw);
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = read_a(0, 0, i);
        fw[0] = read_w(0, 0, 0);
        fw[1] = read_w(0, 0, 1);
        if constexpr (kMode == kStream) {
            for (int t = 0; t < my_tiles; ++t) {
                const int64_t m0 = cur.m0;
                const int n0 = cur.n0;
                for (int kt = 0; kt < KT; ++kt) {
                    // k-step 0 of the slab (its fragments and scales already in registers), reloading k-step 1's
                    if (kt == 0)
                        kstep(std::integral_constant<int, 0>{}, std::true_type{}, acc, fa, fw, sa, sw, stage, 1, no_extra, std::true_type{});
                    else
                        kstep(std::integral_constant<int, 0>{}, std::false_type{}, acc, fa, fw, sa, sw, stage, 1, no_extra, std::true_type{});
                    // the next slab has landed (the loaders waited for it) and this stage is read out: publish one
                    // stage, refill the other with the slab after next
                    if (kLoader) __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
                    sync();
                    // k-step 1, reloading k-step 0 of the next slab (and its scales) from the other stage; the loaders
                    // spread the slab after next over its MFMAs
                    uint32_t sa_n[4], sw_n[2];
                    const int nst = stage ^ 1;
                    if (kLoader) {
                        // the slab after next: slab kt + 2 of this tile, or of the next one (or, when KT = 1, of the
                        // one after)
                        const int k2 = kt + 2;
                        const bool in1 = k2 >= KT, in2 = k2 >= 2 * KT;
                        const SlabRsrc r = slab_rsrc(in2 ? tile_at(t + 2) : (in1 ? nx1 : cur),
                                                     k2 - (in2 ? 2 * KT : (in1 ? KT : 0)));
                        const int st = stage;
                        kstep(std::integral_constant<int, 2>{}, std::false_type{}, acc, fa, fw, sa, sw, nst, 0, [&](int u) {
                            if (u == 0) read_scales(nst, sa_n, sw_n);  // (past the last slab: stale, unused)
                            issue_part(r, st, u);
                        }, std::true_type{});
                    } else {
                        kstep(std::integral_constant<int, 2>{}, std::false_type{}, acc, fa, fw, sa, sw, nst, 0, [&](int u) {
                            if (u == 0) read_scales(nst, sa_n, sw_n);
                        }, std::true_type{});
                    }
                    shift_scales(sa_n, sw_n);
#pragma unroll
                    for (int i = 0; i < 4; ++i) sa[i] = sa_n[i];
#pragma unroll
                    for (int j = 0; j < 2; ++j) sw[j] = sw_n[j];
                    stage ^= 1;
                }
                epilogue(acc, m0, n0);
                cur = nx1;
                nx1 = tile_at(t + 2);
            }
        } else {
            // One slab: k-step 0, the barrier, k-step 1.  kIssue false: the loaders issue nothing (the held-back
            // slabs of a key tile's end); kReload false: the tile's last slab, no fragments are reloaded and no
            // load is waited for (its slab has landed).  kFirst: the tile's first slab (zero C operand: the
            // accumulators are dead between tiles).  hook(u): every wave's share of k-step 1's units in a slab
            // that issues nothing (the tile's last two: the gate epilogue's loads, if any)
            int kt = 0;  // the slab's index in its tile
            auto slab = [&](auto first_tag, auto issue_tag, auto reload_tag, auto&& hook) {
                constexpr bool kIssue = decltype(issue_tag)::value;
                constexpr bool kReload = decltype(reload_tag)::value;
                kstep(std::integral_constant<int, 0>{}, first_tag, acc, fa, fw, sa, sw, stage, 1, no_extra,
                      std::true_type{});
                if (kLoader && kReload) __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
                sync();
                uint32_t sa_n[4], sw_n[2];
                const int nst = stage ^ 1;
                if constexpr (!kReload) {
                    kstep(std::integral_constant<int, 2>{}, std::false_type{}, acc, fa, fw, sa, sw, nst, 0, hook,
                          std::false_type{});
                } else if (kLoader && kIssue) {
                    const SlabRsrc r = slab_rsrc(cur, kt + 2);  // (an issuing slab is followed by two more)
                    const int st = stage;
                    kstep(std::integral_constant<int, 2>{}, std::false_type{}, acc, fa, fw, sa, sw, nst, 0, [&](int u) {
                        if (u == 0) read_scales(nst, sa_n, sw_n);  // (past the last slab: stale, unused)
                        issue_part(r, st, u);
                    }, std::true_type{});
                } else {
                    kstep(std::integral_constant<int, 2>{}, std::false_type{}, acc, fa, fw, sa, sw, nst, 0, [&](int u) {
                        if (u == 0) read_scales(nst, sa_n, sw_n);
                        if constexpr (!kIssue) hook(u);
                    }, std::true_type{});
                }
                if constexpr (kReload) {
                    shift_scales(sa_n, sw_n);
#pragma unroll
                    for (int i = 0; i < 4; ++i) sa[i] = sa_n[i];
#pragma unroll
                    for (int j = 0; j < 2; ++j) sw[j] = sw_n[j];
                }
                stage ^= 1;
                ++kt;
            };
            for (int t = 0; t < my_tiles; ++t) {
                const int64_t m0 = cur.m0;
                const int n0 = cur.n0;
                kt = 0;
                using T_ = std::true_type;
                using F_ = std::false_type;
                // KT >= 3: the tile's last two slabs hold back the next tile's first two (and, for a key tile,
                // fetch what the gate epilogue reads, each into its own stage once its barrier has passed)
                slab(T_{}, T_{}, T_{}, no_extra);
                while (kt < KT - 2) slab(F_{}, T_{}, T_{}, no_extra);
                if constexpr (kMode == kGate) {
                    const int st = stage ^ 1;  // the last slab's stage
                    const __amdgpu_buffer_rsrc_t xr = x_rsrc(m0, n0);
                    slab(F_{}, F_{}, T_{}, [&](int u) {
                        if (u < 2) dma_qk(n0, u);
                        dma_piece(xr, 2 + (u >> 2), u & 3, st);
                    });
                    slab(F_{}, F_{}, F_{}, [&](int u) { dma_piece(xr, u >> 2, u & 3, st); });
                    gate_epilogue(acc, m0, n0, st);
                } else {
                    slab(F_{}, F_{}, T_{}, no_extra);
                    slab(F_{}, F_{}, F_{}, no_extra);
                    store_epilogue(acc, m0, n0);
                }
                // the held-back slabs 0 and 1 of the next tile (past the workgroup's last: empty issues) into the
                // two stages; the first must land before its fragments are read, the second may still fly
                cur = nx1;
                nx1 = tile_at(t + 2);
                if (kLoader) {
                    issue_slab(cur, 0, stage);
                    issue_slab(cur, 1, stage ^ 1);
                    if (wave < 2)
                        __builtin_amdgcn_s_waitcnt(wait_vmcnt(17));  // (waves 0 and 1 also load a slab's scales)
                    else
                        __builtin_amdgcn_s_waitcnt(wait_vmcnt(16));
                }
                sync();
                read_scales(stage, sa, sw);
                shift_scales(sa, sw);
#pragma unroll
                for (int i = 0; i < 4; ++i) fa[i] = read_a(stage, 0, i);
                fw[0] = read_w(stage, 0, 0);
                fw[1] = read_w(stage, 0, 1);
            }
        }
        // loads issued past this workgroup's last slab (empty resources) still write LDS: let them land
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    };
    if (loader)
        run(std::true_type{});
    else
        run(std::false_type{});
}

__global__ __launch_bounds__(kThreads, 1) void wkv_mx_kernel(MxArgs p) { wkv_mx_body<kStream>(p); }
__global__ __launch_bounds__(kThreads, 1) void wkv_mx_hold_kernel(MxArgs p) { wkv_mx_body<kHold>(p); }
__global__ __launch_bounds__(kThreads, 1) void wkv_mx_gate_kernel(MxArgs p) { wkv_mx_body<kGate>(p); }

// ---- OCP MX quantisation of bf16 rows ----
// A thread owns 8 consecutive columns (one 16-byte load); the 4 threads of a 32-column block reduce their
// amax with two lane swaps; the block is then encoded by mx_shared_exp / mx_encode4 (mx.h).
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint16_t* x, int64_t rows, int K, int64_t rows4,
                                                      uint8_t* q, uint8_t* scale) {
    const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int per_row = K / 8;
    const int64_t r = gid / per_row;
    const int c8 = static_cast<int>(gid - r * per_row);  // 8-column group
    const bool ok = r < rows;
    u32x4 v = {0, 0, 0, 0};
    if (ok) v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(x + r * K) + c8);
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    // the 4 threads of a block are lanes 4b .. 4b+3 of the wave (K / 8 is a multiple of 4)
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int shared = mx_shared_exp(amax);
    const uint32_t p0 = mx_encode4(f[0], f[1], f[2], f[3], shared);
    const uint32_t p1 = mx_encode4(f[4], f[5], f[6], f[7], shared);
    if (!ok) return;
    *reinterpret_cast<u32x2*>(q + r * K + 8 * c8) = u32x2{p0, p1};
    if ((c8 & 3) == 0) scale[mx_scale_offset(r, c8 / 4, rows4)] = static_cast<uint8_t>(shared + 127);
}

}  // namespace
}  // namespace engram

using namespace engram;

extern "C" int64_t engram_mx_scale_bytes(int64_t rows, int32_t K) {
    if (rows < 0 || K < kSlabCols || K % kSlabCols != 0) return -1;
    return (K / kSlabCols) * ((rows + 3) / 4 * 4) * 4;
}

extern "C" int engram_mx_quant(const uint16_t* x, int64_t rows, int32_t K, uint8_t* q, uint8_t* scale, void* stream) {
    const char* what = "engram_mx_quant";
    if (rows < 0) return fail(ENGRAM_EINVAL, "%s: rows < 0", what);
    if (K < kSlabCols || K % kSlabCols != 0) return fail(ENGRAM_EINVAL, "%s: K=%d must be a positive multiple of %d", what, K, kSlabCols);
    if (rows == 0) return ENGRAM_OK;
    if (!x || !q || !scale) return fail(ENGRAM_EINVAL, "%s: null pointer", what);
    if (!aligned(x, 16) || !aligned(q, 8)) return fail(ENGRAM_EINVAL, "%s: misaligned pointer", what);
    const int64_t threads = rows * (K / 8);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "%s: too many rows", what);
    hipLaunchKernelGGL(mx_quant_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, as_stream(stream), x, rows, K,
                       (rows + 3) / 4 * 4, q, scale);
    return check_launch(what);
}

extern "C" int engram_wkv_mx(const uint8_t* a, const uint8_t* a_scale, const uint8_t* w, const uint8_t* w_scale,
                             uint16_t* kv, int64_t T, int32_t K, int32_t Nout, void* stream) {
    const char* what = "engram_wkv_mx";
    if (T < 0) return fail(ENGRAM_EINVAL, "%s: T < 0", what);
    if (K < kSlabCols || K % kSlabCols != 0) return fail(ENGRAM_EINVAL, "%s: K=%d must be a positive multiple of %d", what, K, kSlabCols);
    if (Nout < 8 || Nout % 8 != 0) return fail(ENGRAM_EINVAL, "%s: Nout=%d must be a positive multiple of 8", what, Nout);
    if (T == 0) return ENGRAM_OK;
    if (!a || !a_scale || !w || !w_scale || !kv) return fail(ENGRAM_EINVAL, "%s: null pointer", what);
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(a_scale, 16) || !aligned(w_scale, 16) || !aligned(kv, 16))
        return fail(ENGRAM_EINVAL, "%s: misaligned pointer", what);
    MxArgs p = {};
    p.a = a;
    p.as = a_scale;
    p.w = w;
    p.ws = w_scale;
    p.kv = kv;
    p.M = T;
    p.N = Nout;
    p.K = K;
    p.M4 = (T + 3) / 4 * 4;
    p.N4 = (static_cast<int64_t>(Nout) + 3) / 4 * 4;
    p.ld_out = Nout;
    const int64_t tiles_m = (T + BM - 1) / BM;
    p.tiles_n = (Nout + BN - 1) / BN;
    if (tiles_m * p.tiles_n > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "%s: too many tiles", what);
    p.tiles_m = static_cast<int>(tiles_m);
    const int64_t tiles = tiles_m * p.tiles_n;
    const unsigned grid = static_cast<unsigned>(tiles < kCUs ? tiles : kCUs);
    if (K >= 3 * kSlabCols)  // three slabs or more: the held-back loop and its one-round epilogue
        hipLaunchKernelGGL(wkv_mx_hold_kernel, dim3(grid), dim3(kThreads), 0, as_stream(stream), p);
    else
        hipLaunchKernelGGL(wkv_mx_kernel, dim3(grid), dim3(kThreads), 0, as_stream(stream), p);
    return check_launch(what);
}

extern "C" int engram_wkv_mx_gate(const uint8_t* a, const uint8_t* a_scale, const uint8_t* w, const uint8_t* w_scale,
                                  const uint16_t* x, const uint16_t* q_weight, const uint16_t* k_weight, float eps,
                                  uint16_t* value, int64_t ld_value, float* dot, void* workspace,
                                  int64_t workspace_bytes, int64_t T, int32_t K, int32_t hc, int32_t dim,
                                  void* stream) {
    const char* what = "engram_wkv_mx_gate";
    if (T < 0) return fail(ENGRAM_EINVAL, "%s: T < 0", what);
    if (K < 3 * kSlabCols || K % kSlabCols != 0)
        return fail(ENGRAM_EINVAL, "%s: K=%d must be a multiple of %d, at least %d", what, K, kSlabCols, 3 * kSlabCols);
    if (hc < 1 || hc > 64) return fail(ENGRAM_EINVAL, "%s: hc=%d outside [1, 64]", what, hc);
    if (dim < 256 || dim % 256 != 0)
        return fail(ENGRAM_EINVAL, "%s: dim=%d must be a positive multiple of 256", what, dim);
    if (static_cast<int64_t>(hc + 1) * dim > (1 << 22))  // 128 rows of x stay under 2^31 bytes
        return fail(ENGRAM_EINVAL, "%s: (hc + 1) * dim = %lld exceeds 2^22", what, static_cast<long long>(hc + 1) * dim);
    if (ld_value < dim || ld_value % 8 != 0)
        return fail(ENGRAM_EINVAL, "%s: ld_value=%lld must be >= dim and a multiple of 8", what, (long long)ld_value);
    const int64_t need = engram_wkv_gate_workspace_bytes(T, hc, dim);
    if (workspace_bytes < need)
        return fail(ENGRAM_ERANGE, "%s: workspace of %lld bytes, %lld needed", what, (long long)workspace_bytes,
                    (long long)need);
    if (T == 0) return ENGRAM_OK;
    if (!a || !a_scale || !w || !w_scale || !x || !q_weight || !k_weight || !value || !dot || !workspace)
        return fail(ENGRAM_EINVAL, "%s: null pointer", what);
    if (!aligned(a, 16) || !aligned(w, 16) || !aligned(a_scale, 16) || !aligned(w_scale, 16) || !aligned(x, 16) ||
        !aligned(q_weight, 16) || !aligned(k_weight, 16) || !aligned(value, 16) || !aligned(dot, 4) ||
        !aligned(workspace, 16))
        return fail(ENGRAM_EINVAL, "%s: misaligned pointer", what);
    const int Nout = (hc + 1) * dim;
    const int64_t tiles_m = (T + BM - 1) / BM;
    if (tiles_m * (Nout / BN) > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "%s: too many tiles", what);
    // launch 1: the hc * dim key rows of w, reduced against the stream (every tile a key tile)
    MxArgs p = {};
    p.a = a;
    p.as = a_scale;
    p.w = w;
    p.ws = w_scale;
    p.M = T;
    p.N = hc * dim;
    p.K = K;
    p.M4 = (T + 3) / 4 * 4;
    p.N4 = Nout;  // w's scale rows (Nout is a multiple of 256)
    p.x = x;
    p.q = q_weight;
    p.k = k_weight;
    p.part = static_cast<float*>(workspace);
    p.hc = hc;
    p.dim = dim;
    p.tiles_m = static_cast<int>(tiles_m);
    p.tiles_n = p.N / BN;
    int64_t tiles = tiles_m * p.tiles_n;
    hipLaunchKernelGGL(wkv_mx_gate_kernel, dim3(static_cast<unsigned>(tiles < kCUs ? tiles : kCUs)), dim3(kThreads),
                       0, as_stream(stream), p);
    int rc = check_launch(what);
    if (rc != ENGRAM_OK) return rc;
    // launch 2: the dim value rows of w (rows hc * dim on; their scales sit at that row of every 128-column block
    // of the scale layout, whose row count stays Nout), stored into `value`
    MxArgs v = {};
    v.a = a;
    v.as = a_scale;
    v.w = w + static_cast<int64_t>(hc) * dim * K;
    v.ws = w_scale + static_cast<int64_t>(hc) * dim * 4;
    v.kv = value;
    v.M = T;
    v.N = dim;
    v.K = K;
    v.M4 = p.M4;
    v.N4 = Nout;
    v.ld_out = ld_value;
    v.tiles_m = p.tiles_m;
    v.tiles_n = dim / BN;
    tiles = tiles_m * v.tiles_n;
    hipLaunchKernelGGL(wkv_mx_hold_kernel, dim3(static_cast<unsigned>(tiles < kCUs ? tiles : kCUs)), dim3(kThreads),
                       0, as_stream(stream), v);
    rc = check_launch(what);
    if (rc != ENGRAM_OK) return rc;
    float* dots[1] = {dot};
    return launch_gate_finalize(static_cast<const float*>(workspace), 0, dots, 1, T, hc, dim, eps, as_stream(stream),
                                what);
}
