// The bf16 `wkv` projection, and its fused gate pre-activation, on v_mfma_f32_16x16x32_bf16: the form the
// main launches take (DeepSeek V4.1 "stack-hashes" page: Engram.__init__'s `wkv`, and Engram.forward's
// kv = self.wkv(...) with the gate's rstd and dot).  wkv.hip's entry points launch it for one layer's 256-token
// tiles when K is a multiple of 64 with at least three slabs and the layer makes at least two waves of tiles over
// the CUs (a several-layer launch of long layers, layer by layer); several shorter layers of the fused projection
// (a decode step's two) go as one launch of the mixed form, whose workgroups take every layer's key and value
// tiles.  Launches small enough for one pass of 128-token tiles, and other K, keep wkv.hip's own kernels.
//
// Why 16 x 16 x 32: on gfx950 a register-only loop of v_mfma_f32_16x16x32_bf16 on random operands sustains
// about 14 % more flops than one of v_mfma_f32_32x32x16_bf16 (about 1.99 against 1.74 PF on one box; the
// clock is set by power).
//
// Design (gfx950): the fp8 projection's held-back persistent loop (wkv_mx.hip) on bf16 slabs of 64 columns --
// the same 128-byte LDS rows with 16-byte pieces XOR-swizzled by (row / 2) mod 8, two stages of 64 KB (A and
// W slabs), eight waves (loader waves 0-3 issue every slab load), 256 x 256 tiles in XCD-grouped order.  A
// tile's last two slabs hold back the next tile's first two, so both stages are free at its end: the whole tile
// leaves in one store round through them (kHold), or they take the stream rows of the fused gate epilogue
// (kGate).  Each wave: 128 tokens x 64 outputs = 8 x 4 MFMA blocks of 16 x 16, issued as
// W fragment x token fragment, so that lane l holds, per block, token l % 16 and the four consecutive outputs
// 4 (l / 16) .. +3 (the lane layout measured on gfx950: operand lane l holds row l % 16 and K elements
// 8 (l / 16) .. +7; result lane l holds rows 4 (l / 16) .. +3 of column l % 16).  A slab is two k-steps of 32
// columns, 32 MFMAs each; the 12 fragments of a k-step (16 bytes a lane each) are reloaded in place right
// after their last use.  The slab's one barrier sits fourteen MFMAs into its second k-step, where the next
// slab's first fragment read follows it.
#include <type_traits>
#include <utility>

#include "common.h"

namespace engram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256;
constexpr int kSlabCols = 64;               // bf16 columns per slab row (128 bytes)
constexpr int kThreads = 512;
constexpr int kOpBytes = 256 * 128;         // one operand's slab: 32 KB
constexpr int kStageBytes = 2 * kOpBytes;   // 64 KB
constexpr int kQkBytes = 8 * 512;           // fused gate: every wave's 64 q and 64 k elements
constexpr int kXArea = 32 * 128;            // fused gate: a wave's stream rows of one round (32 tokens x 64 bf16)
constexpr int kGroupM = 8;
constexpr int kXcds = 8;
constexpr int kCUs = 256;
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNonTemporal = 2;             // cache-policy operand of a load: streamed past L2
constexpr int kWaitLgkmcnt0 = 0xC07F;
constexpr int wait_vmcnt(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kSlabLoads = 16;              // direct-to-LDS loads per loader wave and slab
constexpr int kBar = 14;                     // the slab barrier precedes unit kBar of a slab's second k-step

constexpr int kHold = 1, kGate = 2, kMixed = 3;

struct W16Args {
    const uint16_t* a;   // [M, K] bf16
    const uint16_t* w;   // [N, K] bf16: the launch's rows of W
    uint16_t* kv;        // kHold: [M, ld_out] bf16, the launch's N columns
    int64_t M;
    int N, K;
    int tiles_m, tiles_n;
    int64_t ld_out;
    // kGate: every tile's columns are key columns, reduced against the stream, not stored
    const uint16_t* x;   // [M, hc, dim] bf16
    const uint16_t* q;   // [hc, dim] bf16
    const uint16_t* k;   // [hc, dim] bf16
    float* part;         // [hc][dim/128][3][M] fp32: per 128-column slice pair sum(h w key), sum(key^2), sum(h^2)
    int hc, dim;
    // kMixed: the key and value tiles of several layers in one launch.  tiles_m = layers x tiles_ml (layer e's M
    // tiles are e tiles_ml .. e tiles_ml + tiles_ml - 1, each starting at its own token 0); every layer's w holds
    // N = (hc + 1) dim rows, a tile of columns below n_key = hc dim is a key tile (kGate's epilogue), any other a
    // value tile (kHold's, into kv columns n0 - n_key).  Layer e's tensors are lay[e]'s (a, w, kv, x, q, k and
    // part above are unused).
    int tiles_ml, n_key;
    W16Layer lay[kW16MaxLayers];
};

// pid -> (tm, tn): contiguous runs per XCD (pid % 8 is the XCD a workgroup lands on), grouped kGroupM deep
__device__ inline void tile_coords(const W16Args& p, int pid, int& tm, int& tn) {
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
// from it live across the slab loop (a spilled loop invariant's reload would wait for every load in flight).
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

template <int kMode>
__device__ __forceinline__ void wkv16_body(const W16Args& p) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStageBytes + kQkBytes];
    const int tiles = p.tiles_m * p.tiles_n;
    const int G = gridDim.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;
    const bool loader = wave < 4;
    const int KT = p.K / kSlabCols;
    const int row_bytes = p.K * 2;

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
    // there.  Rows past M or N fall outside their resource and read as zero; the row offset sits in the
    // range-checked VGPR operand, the SGPR operand carries only the slab's column.
    const int ld_r = lane >> 3, ld_slot = lane & 7;
    const uint32_t vo_piece = static_cast<uint32_t>(ld_r * row_bytes + ((ld_slot ^ (ld_r >> 1)) << 4));
    const uint32_t vo_rows = vo_piece + static_cast<uint32_t>(wave * 64 * row_bytes);
    struct SlabRsrc {
        __amdgpu_buffer_rsrc_t ra, rw;
        uint32_t k0b;
    };
    // a tile of this workgroup: its first row and column; `live` false past the workgroup's last tile, whose
    // loads are then empty (the resources hold no bytes)
    struct TileAt {
        int64_t m0;  // first token of the tile (in its layer)
        int n0;
        int flags;   // bit 0: live; kMixed: bit 1 a key tile, bits 2.. its layer
        __device__ bool live() const { return (flags & 1) != 0; }
        __device__ bool key() const { return (flags & 2) != 0; }
        __device__ int e() const { return flags >> 2; }
    };
    // layer e's tensors (kMixed), else the launch's own; e is wave-uniform
    auto a_of = [&](int e) -> const uint16_t* { if constexpr (kMode == kMixed) return p.lay[e].a; else return p.a; };
    auto w_of = [&](int e) -> const uint16_t* { if constexpr (kMode == kMixed) return p.lay[e].w; else return p.w; };
    auto kv_of = [&](int e) -> uint16_t* { if constexpr (kMode == kMixed) return p.lay[e].kv; else return p.kv; };
    auto x_of = [&](int e) -> const uint16_t* { if constexpr (kMode == kMixed) return p.lay[e].x; else return p.x; };
    auto q_of = [&](int e) -> const uint16_t* { if constexpr (kMode == kMixed) return p.lay[e].q; else return p.q; };
    auto k_of = [&](int e) -> const uint16_t* { if constexpr (kMode == kMixed) return p.lay[e].k; else return p.k; };
    auto part_of = [&](int e) -> float* { if constexpr (kMode == kMixed) return p.lay[e].part; else return p.part; };
    auto slab_rsrc = [&](const TileAt& ta, int kt) {
        int e = ta.e();
        if constexpr (kMode == kMixed) asm volatile("" : "+s"(e));
        const int a_bytes = ta.live() ? static_cast<int>(min<int64_t>(BM, p.M - ta.m0)) * row_bytes : 0;
        const int w_bytes = ta.live() ? min(BN, p.N - ta.n0) * row_bytes : 0;
        SlabRsrc r;
        r.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a_of(e) + ta.m0 * p.K), 0, a_bytes,
                                                 kBufferWord3);
        r.rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(w_of(e) + static_cast<int64_t>(ta.n0) * p.K),
                                                 0, w_bytes, kBufferWord3);
        r.k0b = static_cast<uint32_t>(kt * kSlabCols * 2);
        return r;
    };
    // part q (0..7) of a slab's loads: rows 8q..8q+7 of the wave's A and W rows
    auto issue_part = [&](const SlabRsrc& r, int stage, int q) {
        uint8_t* st = lds + stage * kStageBytes;
        const uint32_t flip = (q & 1) ? (4u << 4) : 0u;
        const uint32_t qrows = static_cast<uint32_t>(q * 8 * row_bytes);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r.ra, st + (wave * 64 + q * 8) * 128, 16, (vo_rows ^ flip) + qrows,
                                                 r.k0b, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r.rw, st + kOpBytes + (wave * 64 + q * 8) * 128, 16,
                                                 (vo_rows ^ flip) + qrows, r.k0b, 0, 0);
    };
    auto issue_slab = [&](const TileAt& ta, int kt, int stage) {
        const SlabRsrc r = slab_rsrc(ta, kt);
#pragma unroll
        for (int q = 0; q < 8; ++q) issue_part(r, stage, q);
    };

    // ---- fragments: lane l reads row (l % 16) of a 16-row block, for k-step s (columns 32s .. 32s + 31) the
    // 16-byte piece 4s + l / 16 at its swizzled slot (the key of row 16b + l % 16 is (l / 2) mod 8; 4s + l / 16
    // = (l / 16) ^ 4s, so k-step 1's offset is k-step 0's with bit 6 flipped).  frag_off: the lane's part of the
    // offset, formed once per k-step from an opaque lane index.
    auto frag_off = [&]() -> uint32_t {
        const int l = lane_here();
        return static_cast<uint32_t>((l & 15) * 128 + (((l >> 4) ^ ((l >> 1) & 7)) << 4));
    };
    auto read_a = [&](uint32_t fo, int stage, int s, int i) {
        return *reinterpret_cast<const bf16x8*>(lds + stage * kStageBytes + (wm * 128 + 16 * i) * 128 + (fo ^ (s << 6)));
    };
    auto read_w = [&](uint32_t fo, int stage, int s, int j) {  // the W rows follow the 256 A rows
        return *reinterpret_cast<const bf16x8*>(lds + stage * kStageBytes + (256 + wn * 64 + 16 * j) * 128 +
                                               (fo ^ (s << 6)));
    };

    // ---- one-round store epilogue (kHold): both stages are free.  Every wave writes its 128 tokens x 64
    // outputs as bf16 into stage wm (row t: token 128 wm + t, 512 bytes = the tile's 256 outputs, 16-byte
    // piece c at slot c ^ (t % 32)); after a barrier every wave reads 32 rows into registers (the accumulators
    // are dead by then), a second barrier frees the stages, every wave writes its rows with full-line
    // non-temporal 16-byte stores (two rows per instruction), and `refill()` issues the held-back slabs; the
    // stores drain while those land and the next tile computes.
    auto store_epilogue = [&](const f32x4 (&acc)[8][4], int e, int64_t m0, int n0, auto&& refill) {
        const int l = kMode == kMixed ? lane_here() : lane_id();  // kMixed: nothing of it hoisted over the loop
        const int g = l >> 4;
        // kMixed: the wave's index formed here, so that nothing derived from it is held over the tile loop
        int wv = wave;
        if constexpr (kMode == kMixed) asm volatile("" : "+s"(wv));
        const int wmv = kMode == kMixed ? (wv & 1) : wm, wnv = kMode == kMixed ? (wv >> 1) : wn;
        uint8_t* sb = lds + wmv * kStageBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = 16 * i + (l & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = wnv * 8 + 2 * j + (g >> 1);  // outputs 64 wn + 16 j + 4 g .. +3
                const u32x2 v = {pack_bf16(acc[i][j][0], acc[i][j][1]), pack_bf16(acc[i][j][2], acc[i][j][3])};
                *reinterpret_cast<u32x2*>(sb + t * 512 + ((c ^ (t & 31)) << 4) + (g & 1) * 8) = v;
            }
        }
        sync_epi();
        const int c = l & 31;
        u32x4 v[16];
#pragma unroll
        for (int ins = 0; ins < 16; ++ins) {
            const int r = 32 * wv + 2 * ins + (l >> 5);  // row of the tile: token m0 + r
            v[ins] = *reinterpret_cast<const u32x4*>(lds + (r >> 7) * kStageBytes + (r & 127) * 512 + ((c ^ (r & 31)) << 4));
        }
        sync_epi();
        // kMixed: a value tile's columns n0 - n_key .. of layer e's value rows
        const int ncol = (kMode == kMixed ? n0 - p.n_key : n0) + 8 * c;
#pragma unroll
        for (int ins = 0; ins < 16; ++ins) {
            const int64_t m = m0 + 32 * wv + 2 * ins + (l >> 5);
            if (m < p.M && ncol < (kMode == kMixed ? p.N - p.n_key : p.N))
                __builtin_nontemporal_store(v[ins], reinterpret_cast<u32x4*>(kv_of(e) + m * p.ld_out + ncol));
        }
        refill();
    };

    // ---- fused gate epilogue of a key tile (kGate): the product is not stored.  The tile's 256 columns lie in
    // one copy c; wave (wm, wn) owns the 64-column slice (n0 - c dim) / 64 + wn of that copy and tokens
    // [128 wm, +128).  In round r < 4 (tokens 32r .. 32r + 31 of the wave's 128: blocks i = 2r, 2r + 1) lane l
    // holds tokens 32r + l % 16 and 32r + 16 + l % 16, each with 16 of the slice's columns (four consecutive ones
    // per block j, as the MFMA leaves them).  Each accumulator is rounded to bf16 (the product is a bf16 tensor
    // before it is used) and reduced against the stream's matching element: sum(h w key), sum(key^2), sum(h^2)
    // over the lane's columns, then over the four lanes of the token (l, l ^ 16, l ^ 32, l ^ 48).  The stream
    // rows come in by direct-to-LDS loads that the tile's last two slabs issue (they hold back the next tile's
    // first two, so each stage is free from the barrier of the slab that read it last): the second-to-last slab
    // fetches the slice's q and k elements and rounds 2 and 3 into its own stage, the last slab rounds 0 and 1
    // into its own, st.  Round r: stage st (r < 2) or st ^ 1, at (r & 1) * 32 KB, the wave's 4 KB area; row t
    // is token 32 r + t of the wave's 128, 16-byte piece q at slot q ^ ((t >> 1) & 7).  Each wave waits only for
    // its own loads.  Loader waves hand their sums to their SIMD partner (storer wave w + 4: the same tokens,
    // the slice 128 columns to the right), which adds them to its own and stores one value per (copy, pair of
    // slices, token).
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
    uint8_t* const qk_area = lds + 2 * kStageBytes;
    // The stream rows of this wave's 128 tokens and 64 columns through a buffer resource based at token
    // m0 + 128 wm, column n0 + 64 wn of x ([M, hc dim] bf16; the key columns n0 + 64 wn .. +63 of copy c are
    // x's columns of the same numbers): tokens past M fall outside it and read as zero.  Lane l loads row l / 8
    // of an 8-row group, the 16-byte piece its slot l % 8 holds under the swizzle: x_voff, flipped by 64 bytes
    // for odd groups (the swizzle key of group g's rows is 4 g + l / 16, mod 8).
    const uint32_t x_row_bytes = static_cast<uint32_t>(p.hc * p.dim * 2);  // < 2^24
    const uint32_t x_voff = (lane >> 3) * x_row_bytes + (((lane & 7) ^ (lane >> 4)) << 4);
    auto x_rsrc = [&](int e, int64_t m0, int n0, bool on) {
        const int64_t t0 = m0 + wm * 128;
        const int64_t rows = min<int64_t>(128, p.M - t0);
        const int64_t col = n0 + wn * 64;
        const int bytes = on && rows > 0 ? static_cast<int>(rows * x_row_bytes - 2 * col) : 0;  // < 2^31
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x_of(e) + t0 * (x_row_bytes / 2) + col), 0,
                                                 bytes, kBufferWord3);
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
    // the slice's 64 q and 64 k elements into the wave's 512 bytes of the q/k area: q column j at byte 2 j, k
    // column j at 256 + 2 j; two loads of 4 bytes a lane whose upper 32 lanes fall outside their 128-byte resource
    auto dma_qk = [&](int e, int n0, int which, bool on) {
        const uint16_t* src = (which == 0 ? q_of(e) : k_of(e)) + (on ? n0 + wn * 64 : 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), 0, on ? 128 : 0, kBufferWord3),
            qk_area + wave * 512 + which * 256, 4, static_cast<uint32_t>(lane_here() * 4), 0, 0, 0);
    };
    // The accumulators of a key tile whose last two slabs issued, in this order, the q and k loads and rounds 2
    // and 3 (10 loads), then rounds 0 and 1 (8 loads): rounds 2 and 3 are reduced first.
    auto gate_epilogue = [&](const f32x4 (&acc)[8][4], int e, int64_t m0, int n0, int st) {
        const int l = kMode == kMixed ? lane_here() : lane_id();
        const int g = l >> 4;
        const int c = n0 / p.dim;
        own_wait(std::integral_constant<int, 8>{});  // q, k and rounds 2 and 3 (rounds 0 and 1 may fly)
        // q * k (exact in fp32) for the lane's 16 columns 16 j + 4 g + e
        float wgt[4][4];
        {
            const uint8_t* qk = qk_area + wave * 512 + 8 * g;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x2 qv = *reinterpret_cast<const u32x2*>(qk + 32 * j);
                const u32x2 kv = *reinterpret_cast<const u32x2*>(qk + 256 + 32 * j);
                wgt[j][0] = lo_bf16(qv[0]) * lo_bf16(kv[0]);
                wgt[j][1] = hi_bf16(qv[0]) * hi_bf16(kv[0]);
                wgt[j][2] = lo_bf16(qv[1]) * lo_bf16(kv[1]);
                wgt[j][3] = hi_bf16(qv[1]) * hi_bf16(kv[1]);
            }
        }
        float res[4][2][3];  // [round][token of the lane: 32 r + 16 b + l % 16][sum]
        auto reduce = [&](auto r_tag) {
            constexpr int r = decltype(r_tag)::value;
            const uint8_t* xl = round_base(r, st) + wave * kXArea;
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int t = 16 * b + (l & 15);  // row of the round's area
                u32x2 xr[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    xr[j] = *reinterpret_cast<const u32x2*>(xl + t * 128 + (((2 * j + (g >> 1)) ^ ((t >> 1) & 7)) << 4) +
                                                             (g & 1) * 8);
                float hwk = 0.f, kk = 0.f, hh = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4& a4 = acc[2 * r + b][j];
                    const uint32_t k01 = cvt_pk_bf16(a4[0], a4[1]);
                    const uint32_t k23 = cvt_pk_bf16(a4[2], a4[3]);
                    const float key[4] = {lo_bf16(k01), hi_bf16(k01), lo_bf16(k23), hi_bf16(k23)};
                    const float h[4] = {lo_bf16(xr[j][0]), hi_bf16(xr[j][0]), lo_bf16(xr[j][1]), hi_bf16(xr[j][1])};
#pragma unroll
                    for (int e = 0; e < 4; ++e) hwk += h[e] * wgt[j][e] * key[e];
                    kk = dot2_bf16(k01, k01, kk);
                    kk = dot2_bf16(k23, k23, kk);
                    hh = dot2_bf16(xr[j][0], xr[j][0], hh);
                    hh = dot2_bf16(xr[j][1], xr[j][1], hh);
                }
                hwk += __shfl_xor(hwk, 16, 64);
                kk += __shfl_xor(kk, 16, 64);
                hh += __shfl_xor(hh, 16, 64);
                res[r][b][0] = hwk + __shfl_xor(hwk, 32, 64);
                res[r][b][1] = kk + __shfl_xor(kk, 32, 64);
                res[r][b][2] = hh + __shfl_xor(hh, 32, 64);
            }
        };
        reduce(std::integral_constant<int, 2>{});
        reduce(std::integral_constant<int, 3>{});
        own_wait(std::integral_constant<int, 4>{});
        reduce(std::integral_constant<int, 0>{});
        own_wait(std::integral_constant<int, 0>{});
        reduce(std::integral_constant<int, 1>{});
        // lane l < 32 carries token 32 r + l of each round (block l / 16: every lane of a token holds its sums)
        const bool hi16 = (l & 16) != 0;
        // hand-over: a loader wave leaves its sums in its own area of round 1 (read out above); its SIMD partner
        // adds them to its own and stores both
        uint8_t* const hand = round_base(1, st);
        if (loader) {
            lds_fence();
            if (l < 32) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int q = 0; q < 3; ++q)
                        reinterpret_cast<float*>(hand + wave * kXArea)[(r * 3 + q) * 32 + l] =
                            hi16 ? res[r][1][q] : res[r][0][q];
            }
        }
        sync_epi();
        if (!loader && l < 32) {
            // the storer adds its partner's sums (slice wn - 2 of the tile) to its own (slice wn): one value per
            // (copy, 128-column slice pair, token), always summed in this order
            const float* partner = reinterpret_cast<const float*>(hand + (wave - 4) * kXArea);
            const int64_t tbase = m0 + wm * 128 + l;
            const int pair = (n0 - c * p.dim) / 128 + (wn - 2);
            float* out = part_of(e) + (static_cast<int64_t>(c) * (p.dim / 128) + pair) * 3 * p.M;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = tbase + 32 * r;
#pragma unroll
                for (int q = 0; q < 3; ++q) {
                    const float v = (hi16 ? res[r][1][q] : res[r][0][q]) + partner[(r * 3 + q) * 32 + l];
                    if (t < p.M) __builtin_nontemporal_store(v, out + q * p.M + t);
                }
            }
        }
        sync_epi();  // the partner's sums, the stream rows and q and k are read before the stages are refilled
    };

    if (static_cast<int>(blockIdx.x) >= tiles) return;
    const int my_tiles = (tiles - 1 - static_cast<int>(blockIdx.x)) / G + 1;
    // this workgroup's tile t (its tile coordinates are computed once per tile, not per slab)
    auto tile_at = [&](int t) {
        int tm, tn;
        tile_coords(p, static_cast<int>(blockIdx.x) + (t < my_tiles ? t : 0) * G, tm, tn);
        int flags = t < my_tiles ? 1 : 0;
        if constexpr (kMode == kMixed) {
            int e = 0;
            while (tm >= p.tiles_ml) {  // at most kW16MaxLayers - 1 steps
                tm -= p.tiles_ml;
                ++e;
            }
            flags |= (tn * BN < p.n_key ? 2 : 0) | (e << 2);
        }
        return TileAt{static_cast<int64_t>(tm) * BM, tn * BN, flags};
    };

    // One k-step: acc[i][j] += (W fragment j) x (token fragment i) in two halves, W fragments 0-1 then 2-3, each
    // walking the 8 token fragments against its pair; each fragment is reloaded, for k-step `ns` of stage `nst`,
    // right after its last use here (token fragment i after its block (i, 3); W fragments 0-1 at the end of the
    // first half, 2-3 at the end of the second), so every reload is issued fifteen or more MFMAs before its next
    // use, and the k-step's first LDS read comes at unit 14.  Each MFMA with its reloads and `extra(u)` (u = 0..31)
    // is one scheduling unit.  kReload false (the last slab of a tile): no reloads, the fragments are dead after
    // the k-step.
    auto kstep = [&](auto zero_tag, f32x4 (&acc)[8][4], bf16x8 (&fa)[8], bf16x8 (&fw)[4], int nst, int ns,
                     auto&& extra, auto reload_tag) {
        constexpr bool kZero = decltype(zero_tag)::value;
        constexpr bool kReload = decltype(reload_tag)::value;
        const f32x4 z = {};
        const uint32_t fo = kReload ? frag_off() : 0u;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    const int j = 2 * jj + jb;
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[j], fa[i], kZero ? z : acc[i][j], 0, 0, 0);
                    if (kReload && j == 3) fa[i] = read_a(fo, nst, ns, i);
                    if (kReload && i == 7) fw[j] = read_w(fo, nst, ns, j);
                    extra(16 * jj + 2 * i + jb);
                    asm volatile("" ::: "memory");  // keeps the unit's LDS reads and loads in the unit
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    };
    auto no_extra = [](int) {};

    auto run = [&](auto loader_tag) {
        constexpr bool kLoader = decltype(loader_tag)::value;
        // the workgroup's tiles t and t + 1
        TileAt cur = tile_at(0), nx1 = tile_at(1);
        if (kLoader) {
            issue_slab(cur, 0, 0);
            issue_slab(cur, 1, 1);
            __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
        }
        sync();
        f32x4 acc[8][4];
        bf16x8 fa[8], fw[4];
        int stage = 0;
        {
            const uint32_t fo = frag_off();
#pragma unroll
            for (int i = 0; i < 8; ++i) fa[i] = read_a(fo, 0, 0, i);
#pragma unroll
            for (int j = 0; j < 4; ++j) fw[j] = read_w(fo, 0, 0, j);
        }
        // One slab: k-step 0, the barrier, k-step 1.  kIssue false: the loaders issue nothing (the held-back
        // slabs of a tile's end); kReload false: the tile's last slab, no fragments are reloaded and no load is
        // waited for (its slab has landed).  kFirst: the tile's first slab (zero C operand: the accumulators are
        // dead between tiles).  hook(u): every wave's share of k-step 1's units in a slab that issues nothing
        // (the tile's last two: the gate epilogue's loads, if any)
        int kt = 0;  // the slab's index in its tile
        auto slab = [&](auto first_tag, auto issue_tag, auto reload_tag, auto&& hook) {
            constexpr bool kIssue = decltype(issue_tag)::value;
            constexpr bool kReload = decltype(reload_tag)::value;
            kstep(first_tag, acc, fa, fw, stage, 1, no_extra, std::true_type{});
            const int nst = stage ^ 1;
            // The slab barrier sits after unit kBar - 1 of k-step 1, just before its first LDS read (W fragment
            // 0's reload at unit 14): the k-step's first MFMAs run while this wave's last reads of the stage
            // complete and the other waves arrive.  Everything that writes the freed stage comes after it: the
            // loaders' slab loads (one part every second unit) or the gate's loads (hook(n), one per unit).
            auto bar = [&]() {
                if (kLoader && kReload) __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
                sync();
            };
            if constexpr (!kReload) {
                kstep(std::false_type{}, acc, fa, fw, nst, 0, [&](int u) {
                    if (u == kBar - 1) bar();
                    if (u >= kBar) hook(u - kBar);
                }, std::false_type{});
            } else if (kLoader && kIssue) {
                const SlabRsrc r = slab_rsrc(cur, kt + 2);  // (an issuing slab is followed by two more)
                const int st = stage;
                kstep(std::false_type{}, acc, fa, fw, nst, 0, [&](int u) {
                    if (u == kBar - 1) bar();
                    if (u >= kBar && (u - kBar) % 2 == 0 && (u - kBar) / 2 < 8) issue_part(r, st, (u - kBar) / 2);
                }, std::true_type{});
            } else {
                kstep(std::false_type{}, acc, fa, fw, nst, 0, [&](int u) {
                    if (u == kBar - 1) bar();
                    if constexpr (!kIssue) {
                        if (u >= kBar) hook(u - kBar);
                    }
                }, std::true_type{});
            }
            stage ^= 1;
            ++kt;
        };
        for (int t = 0; t < my_tiles; ++t) {
            const int64_t m0 = cur.m0;
            const int n0 = cur.n0;
            const int e = cur.e();
            const bool key_tile = cur.key();
            kt = 0;
            using T_ = std::true_type;
            using F_ = std::false_type;
            // KT >= 3: the tile's last two slabs hold back the next tile's first two (and, for a key tile, fetch
            // what the gate epilogue reads, each into its own stage once its barrier has passed)
            slab(T_{}, T_{}, T_{}, no_extra);
            while (kt < KT - 2) slab(F_{}, T_{}, T_{}, no_extra);
            // the held-back slabs 0 and 1 of the next tile (past the workgroup's last: empty issues), issued into
            // the two stages once the epilogue has freed them; the first must land before its fragments are
            // read, the second may still fly (a loader's vmcnt also counts the stores it issued before them)
            cur = nx1;
            nx1 = tile_at(t + 2);
            auto refill = [&]() {
                if (kLoader) {
                    issue_slab(cur, 0, stage);
                    issue_slab(cur, 1, stage ^ 1);
                }
            };
            if constexpr (kMode != kMixed) {
                if constexpr (kMode == kGate) {
                    const int st = stage ^ 1;  // the last slab's stage
                    const __amdgpu_buffer_rsrc_t xr = x_rsrc(e, m0, n0, true);
                    // one load per unit after the slab barrier: q, k, then round 2's and round 3's four
                    slab(F_{}, F_{}, T_{}, [&](int n) {
                        if (n < 2) dma_qk(e, n0, n, true);
                        else if (n < 10) dma_piece(xr, 2 + ((n - 2) >> 2), (n - 2) & 3, st);
                    });
                    // rounds 0 and 1
                    slab(F_{}, F_{}, F_{}, [&](int n) {
                        if (n < 8) dma_piece(xr, n >> 2, n & 3, st);
                    });
                    gate_epilogue(acc, e, m0, n0, st);
                    refill();
                } else {
                    slab(F_{}, F_{}, T_{}, no_extra);
                    slab(F_{}, F_{}, F_{}, no_extra);
                    store_epilogue(acc, e, m0, n0, refill);
                }
            } else {
                // A value tile runs the key tile's last two slabs with empty resources for its loads (they write
                // zeros), so that the slabs are one code for both kinds of tile; before the store epilogue
                // writes the stages, every wave's loads have landed.  The whole workgroup takes one side of the
                // test: n0 comes from the tile order alone.
                const bool key = key_tile;
                const int st = stage ^ 1;
                // the layer's epilogue tensors are looked up here, not held in scalar registers over the tile
                int el = e;
                asm volatile("" : "+s"(el));
                const __amdgpu_buffer_rsrc_t xr = x_rsrc(el, m0, n0, key);
                slab(F_{}, F_{}, T_{}, [&](int n) {
                    if (n < 2) dma_qk(el, n0, n, key);
                    else if (n < 10) dma_piece(xr, 2 + ((n - 2) >> 2), (n - 2) & 3, st);
                });
                slab(F_{}, F_{}, F_{}, [&](int n) {
                    if (n < 8) dma_piece(xr, n >> 2, n & 3, st);
                });
                asm volatile("" : "+s"(el));
                if (key) {
                    gate_epilogue(acc, el, m0, n0, st);
                    refill();
                } else {
                    own_wait(std::integral_constant<int, 0>{});
                    sync_epi();
                    store_epilogue(acc, el, m0, n0, refill);
                }
            }
            if (kLoader) __builtin_amdgcn_s_waitcnt(wait_vmcnt(kSlabLoads));
            sync();
            const uint32_t fo = frag_off();
#pragma unroll
            for (int i = 0; i < 8; ++i) fa[i] = read_a(fo, stage, 0, i);
#pragma unroll
            for (int j = 0; j < 4; ++j) fw[j] = read_w(fo, stage, 0, j);
        }
        // loads issued past this workgroup's last slab (empty resources) still write LDS: let them land
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    };
    if (loader)
        run(std::true_type{});
    else
        run(std::false_type{});
}

__global__ __launch_bounds__(kThreads, 1) void wkv16_hold_kernel(W16Args p) { wkv16_body<kHold>(p); }
__global__ __launch_bounds__(kThreads, 1) void wkv16_gate_kernel(W16Args p) { wkv16_body<kGate>(p); }
__global__ __launch_bounds__(kThreads, 1) void wkv16_mixed_kernel(W16Args p) { wkv16_body<kMixed>(p); }

// one persistent launch over p's tiles (p.tiles_m, p.tiles_n set)
template <int kMode>
int launch_one(const W16Args& p, hipStream_t stream, const char* what) {
    const int64_t tiles = static_cast<int64_t>(p.tiles_m) * p.tiles_n;
    const unsigned grid = static_cast<unsigned>(tiles < kCUs ? tiles : kCUs);
    if constexpr (kMode == kGate)
        hipLaunchKernelGGL(wkv16_gate_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
    else if constexpr (kMode == kMixed)
        hipLaunchKernelGGL(wkv16_mixed_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(wkv16_hold_kernel, dim3(grid), dim3(kThreads), 0, stream, p);
    return check_launch(what);
}

}  // namespace

bool wkv16_takes(int64_t T, int K, int N, int hc, int dim, bool gate) {
    if (T < 1 || K % kSlabCols != 0 || K < 3 * kSlabCols || K > (1 << 20)) return false;
    const int64_t tiles_m = (T + BM - 1) / BM;
    if (tiles_m > 0x7FFFFF) return false;
    // at least two waves of tiles over the CUs; a fused launch counts all (hc + 1) dim columns, so that it takes
    // these kernels exactly when the plain launch of the same weights does (its value columns are then those of
    // the plain launch, bit for bit)
    if (!gate) return tiles_m * ((N + BN - 1) / BN) >= 2 * kCUs;
    return static_cast<int64_t>(hc + 1) * dim <= (1 << 22) &&  // 128 rows of x under 2^31 bytes
           tiles_m * ((hc + 1) * dim / BN) >= 2 * kCUs;
}

int launch_wkv16(const uint16_t* a, const uint16_t* w, uint16_t* kv, int64_t ld_out, int64_t T, int K, int N,
                 const uint16_t* x, const uint16_t* q, const uint16_t* k, float* part, int hc, int dim, bool gate,
                 hipStream_t stream, const char* what) {
    W16Args p = {};
    p.a = a;
    p.M = T;
    p.K = K;
    p.tiles_m = static_cast<int>((T + BM - 1) / BM);
    if (!gate) {
        p.w = w;
        p.kv = kv;
        p.ld_out = ld_out;
        p.N = N;
        p.tiles_n = (N + BN - 1) / BN;
        if (static_cast<int64_t>(p.tiles_m) * p.tiles_n > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "%s: too many tiles", what);
        return launch_one<kHold>(p, stream, what);
    }
    // the hc * dim key rows of w, reduced against the stream (every tile a key tile); then the dim value rows
    // (rows hc * dim on), stored into kv
    p.w = w;
    p.N = hc * dim;
    p.tiles_n = p.N / BN;
    p.x = x;
    p.q = q;
    p.k = k;
    p.part = part;
    p.hc = hc;
    p.dim = dim;
    if (static_cast<int64_t>(p.tiles_m) * p.tiles_n > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "%s: too many tiles", what);
    int rc = launch_one<kGate>(p, stream, what);
    if (rc != ENGRAM_OK) return rc;
    W16Args v = {};
    v.a = a;
    v.w = w + static_cast<int64_t>(hc) * dim * K;
    v.kv = kv;
    v.ld_out = ld_out;
    v.M = T;
    v.N = dim;
    v.K = K;
    v.tiles_m = p.tiles_m;
    v.tiles_n = dim / BN;
    return launch_one<kHold>(v, stream, what);
}

bool wkv16_layers_takes(int64_t T, int K, int hc, int dim, int layers) {
    if (T < 1 || layers < 1 || layers > kW16MaxLayers) return false;
    if (K % kSlabCols != 0 || K < 3 * kSlabCols || K > (1 << 20)) return false;
    if (dim < BN || dim % BN != 0 || static_cast<int64_t>(hc + 1) * dim > (1 << 22)) return false;
    const int64_t tiles_ml = (T + BM - 1) / BM;
    return tiles_ml * layers * ((hc + 1) * dim / BN) <= 0x7FFFFFFF;
}

int launch_wkv16_layers(const W16Layer* lay, int layers, int64_t ld_out, int64_t T, int K, int hc, int dim,
                        hipStream_t stream, const char* what) {
    if (!wkv16_layers_takes(T, K, hc, dim, layers)) return fail(ENGRAM_EINVAL, "%s: no several-layer launch", what);
    W16Args p = {};
    p.M = T;
    p.K = K;
    p.N = (hc + 1) * dim;
    p.ld_out = ld_out;
    p.hc = hc;
    p.dim = dim;
    p.tiles_ml = static_cast<int>((T + BM - 1) / BM);
    p.tiles_m = p.tiles_ml * layers;
    p.tiles_n = p.N / BN;
    p.n_key = hc * dim;
    for (int e = 0; e < layers; ++e) p.lay[e] = lay[e];
    return launch_one<kMixed>(p, stream, what);
}

}  // namespace engram
