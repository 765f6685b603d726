// engram_hash: n-gram hash ids over the compressed-id cache.
//
// Computes the engram hash module's forward of the DeepSeek V4.1
// "stack-hashes" page: compressed ids through token_map, DEAD at masked
// positions, the cache write, the shifted lookback window with cumulative
// blocking to the pad id, the int64 products with the per-(layer, lookback)
// multipliers, the running XOR, the per-(layer, n-gram size, head) prime
// modulo and the column offsets.
//
// Design (gfx950):
// - One workgroup of 256 lanes per tile of 64 consecutive tokens (flattened
//   over batch and position).
// - Phase 1, one lane per token: the lane builds its N-slot window.  Slots
//   inside this chunk are recomputed from input_ids/token_map/mask instead
//   of being read back from the cache this same launch writes, so no lane
//   ever depends on another workgroup's cache write; only positions before
//   start_pos are read from the cache.  The lane then forms the running XOR
//   of the products for every layer and parks the N-1 running values of
//   each layer in LDS.
// - Phase 2, all 256 lanes: the tile's ids ([64 tokens, E, C], contiguous),
//   written with coalesced int64 stores.
//   Each id costs one 64-bit floor modulo, done as a Barrett reduction
//   (a 64 x 64 -> high-64 multiply by floor((2^64 - 1) / p), at most two
//   corrections): exact integer arithmetic, without a 64-bit division per
//   id.  A lane keeps one (layer, column) for the whole tile, so its prime,
//   offset and reciprocal are fetched and computed once.
// - A small call (a 256-token decode step) shrinks the tile, down to one
//   token per workgroup, so its arithmetic spreads over the CUs.
//
// engram_hash_gather_packed: the same kernel with a phase 3 -- the tile's ids
// stay in LDS and its lanes fetch and dequantise every layer's rows from the
// packed tables (ParallelEngramEmbedding.forward of the same page, as
// engram_gather_dequant_packed computes it), so a decode step makes one
// launch and one memory round trip fewer per layer.
#include "dequant.h"

namespace engram {
namespace {

constexpr int kMaxN = 8;
constexpr int kMaxE = 8;
constexpr int kMaxC = 1024;
constexpr int kTileTokens = 64;
// The fused gather: at most 16 tokens per workgroup and 8 rows per lane in flight (measured against 64 and
// 4: equal at decode, 4 % faster on a long prefill's ids, 9 % on uniform ids).
constexpr int kGatherTileTokens = 16;
constexpr int kGatherUnroll = 8;
constexpr int kSpreadBlocks = 256;  // a launch gets at least this many workgroups while tiles can shrink
constexpr int kMaxTileIds = 4096;   // ids a tile keeps in LDS for the fused gather (32 KB)
constexpr int kThreads = 256;

struct HashArgs {
    const int64_t* input_ids;
    const uint8_t* mask;
    const int64_t* token_map;
    int64_t vocab;
    int64_t* cache;
    int64_t cache_L;
    const int64_t* mult;
    const int64_t* primes;
    const int64_t* offsets;
    int64_t T, L, start_pos, pad, dead;
    int E, N, H, C;
    int tile;  // tokens per workgroup (a power of two, at most kTileTokens)
    int64_t* out;  // may be null when the rows are gathered
    int32_t* out32;  // the ids as int32 (ids outside [0, 2^31) stored as -1), or null
};

// Phase 3 of the fused call: per layer e, its packed table [R, 2D] and its rows [T, C, D] out.
struct GatherSide {
    const uint8_t* table[kMaxE];
    int64_t R[kMaxE];
    int64_t row_start[kMaxE];
    uint16_t* out[kMaxE];
    int blk;
};

// x mod p for x < 2^64 and p >= 1, given m = floor((2^64 - 1) / p): q = floor(x m / 2^64) is at most 2 below
// floor(x / p) (x m / 2^64 > x / p - x / (p 2^64) - x / 2^64 > x / p - 2), so x - q p lies in [0, 3p).
__device__ inline uint64_t mod_barrett(uint64_t x, uint64_t p, uint64_t m) {
    uint64_t r = x - __umul64hi(x, m) * p;
    if (r >= p) r -= p;
    if (r >= p) r -= p;
    return r;
}

// floor modulo by a positive divisor: the result takes the divisor's sign.
__device__ inline int64_t floor_mod_pos(int64_t r, int64_t p, uint64_t m) {
    const uint64_t up = static_cast<uint64_t>(p);
    if (r >= 0) return static_cast<int64_t>(mod_barrett(static_cast<uint64_t>(r), up, m));
    // r < 0:  r = -(a + 1) with a = ~r >= 0, and floormod(r, p) = p - 1 - (a mod p)
    const uint64_t a = ~static_cast<uint64_t>(r);
    return static_cast<int64_t>(up - 1 - mod_barrett(a, up, m));
}

// D = 0: hash only.  D > 0: the ids also go to LDS (after the running values) and phase 3 gathers the rows.
template <int D>
__global__ __launch_bounds__(kThreads) void hash_kernel(HashArgs a, GatherSide gs) {
    extern __shared__ int64_t roll[];  // [tile][E][N-1], then (D > 0) the ids [tile][E * C]
    const int NR = a.N - 1;
    const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * a.tile;
    const int ntok = static_cast<int>(min<int64_t>(a.tile, a.T - tile0));
    const int tid = threadIdx.x;
    const int EC = a.E * a.C;

    if (tid < ntok) {
        const int64_t t = tile0 + tid;
        const int64_t b = t / a.L;
        const int64_t l = t - b * a.L;
        const int64_t p = a.start_pos + l;
        // Every slot's loads go out together (indices clamped into range, results selected afterwards), so
        // the window costs two memory round trips (ids, then token_map) rather than one per slot.  The cache
        // is read only where a slot comes from it (before this chunk, after the sequence start): those
        // positions were written by an earlier call, never by this launch.
        int64_t raw[kMaxN], cached[kMaxN];
        uint8_t mk[kMaxN];
#pragma unroll
        for (int s = 0; s < kMaxN; ++s) {
            if (s < a.N) {
                const int64_t flat = b * a.L + (l >= s ? l - s : 0);
                raw[s] = a.input_ids[flat];
                mk[s] = a.mask != nullptr ? a.mask[flat] : 1;
                cached[s] = (l < s && p >= s) ? a.cache[b * a.cache_L + (p - s)] : 0;
            }
        }
        int64_t slot[kMaxN];
#pragma unroll
        for (int s = 0; s < kMaxN; ++s) {
            if (s < a.N) {
                const int64_t id = raw[s];
                const bool in_vocab = id >= 0 && id < a.vocab;
                const int64_t mapped = a.token_map[in_vocab ? id : 0];
                slot[s] = (in_vocab && mk[s] != 0) ? mapped : a.dead;
            }
        }
        bool blocked = false;
#pragma unroll
        for (int s = 0; s < kMaxN; ++s) {
            if (s < a.N) {
                if (p < s) {
                    blocked = true;  // before the start of the sequence
                } else {
                    const int64_t v = l - s >= 0 ? slot[s] : cached[s];
                    if (s == 0) a.cache[b * a.cache_L + p] = v;
                    if (v == a.dead) blocked = true;
                    slot[s] = v;
                }
                if (blocked) slot[s] = a.pad;
            }
        }
        int64_t* my = roll + static_cast<int64_t>(tid) * a.E * NR;
        for (int e = 0; e < a.E; ++e) {
            const int64_t* m = a.mult + static_cast<int64_t>(e) * a.N;
            uint64_t r = static_cast<uint64_t>(slot[0]) * static_cast<uint64_t>(m[0]);
#pragma unroll
            for (int s = 1; s < kMaxN; ++s) {
                if (s < a.N) {
                    r ^= static_cast<uint64_t>(slot[s]) * static_cast<uint64_t>(m[s]);
                    my[e * NR + (s - 1)] = static_cast<int64_t>(r);
                }
            }
        }
    }
    __syncthreads();

    const int total = ntok * EC;
    int64_t* out = a.out != nullptr ? a.out + tile0 * EC : nullptr;
    int64_t* ids = roll + static_cast<int64_t>(a.tile) * a.E * NR;
    int32_t* out32 = a.out32 != nullptr ? a.out32 + tile0 * EC : nullptr;
    auto put = [&](int idx, int64_t id) {
        if (out != nullptr) out[idx] = id;
        if (out32 != nullptr) out32[idx] = (id >= 0 && id <= 0x7FFFFFFF) ? static_cast<int32_t>(id) : -1;
        if (D > 0) ids[idx] = id;
    };
    if (EC <= kThreads) {
        // Lane l keeps one (layer, column) pc = l % EC for the whole tile: its prime, offset and Barrett
        // reciprocal are fetched once, then it walks tokens l / EC, + G, + 2G, ... (G = 256 / EC); the
        // lanes of one step write G consecutive token rows, so the stores stay coalesced.
        const int G = kThreads / EC;
        if (tid < G * EC) {
            const int pc = tid % EC;  // = e * C + (n - 2) * H + h: primes [E, N-1, H] flat is [E, C] in column order
            const int e = pc / a.C;
            const int n1 = (pc - e * a.C) / a.H;  // n-gram size minus 2
            const int64_t prime = a.primes[pc];
            const int64_t off = a.offsets[pc];
            const uint64_t m = prime > 0 ? ~0ull / static_cast<uint64_t>(prime) : 0;
            for (int i = tid / EC; i < ntok; i += G) {
                const int64_t r = roll[(static_cast<int64_t>(i) * a.E + e) * NR + n1];
                put(i * EC + pc, floor_mod_pos(r, prime, m) + off);
            }
        }
    } else {
        for (int idx = tid; idx < total; idx += kThreads) {  // more than 256 ids per token: one id per lane and step
            const int i = idx / EC;
            const int pc = idx - i * EC;
            const int e = pc / a.C;
            const int n1 = (pc - e * a.C) / a.H;
            const int64_t prime = a.primes[pc];
            const int64_t r = roll[(static_cast<int64_t>(i) * a.E + e) * NR + n1];
            put(idx, floor_mod_pos(r, prime, prime > 0 ? ~0ull / static_cast<uint64_t>(prime) : 0) + a.offsets[pc]);
        }
    }
    if constexpr (D > 0) {
        // Phase 3: D/16 lanes per row (one 16-byte piece each); layer by layer, the layer's rows (token,
        // column) of the tile in order, kUnroll rows per lane in flight.  A row outside its layer's
        // [row_start, row_start + R) is zero; the record's scales sit after its D bytes.
        constexpr int LPR = D / 16;
        constexpr int RPP = kThreads / LPR;  // rows per pass
        constexpr int kUnroll = kGatherUnroll;
        __syncthreads();
        const int lr = tid % LPR;
        const int sidx = (lr * 16) / gs.blk;
        const int rows = ntok * a.C;  // one layer's rows of the tile: row r = (token r / C, column r % C)
        // consecutive rows of a lane are RPP apart: (RPP / C, RPP % C) in (token, column), one carry
        const int step_i = RPP / a.C, step_c = RPP - step_i * a.C;
        for (int e = 0; e < a.E; ++e) {
            // the layer's arguments, read with a wave-uniform index from the kernel arguments
            const uint8_t* table = gs.table[e];
            const int64_t R = gs.R[e], rs = gs.row_start[e];
            uint16_t* o = gs.out[e];
            for (int r0 = tid / LPR; r0 < rows; r0 += RPP * kUnroll) {
                u32x4 v[kUnroll];
                float sc[kUnroll];
                bool ok[kUnroll];
                uint16_t* dst[kUnroll];
                int i = r0 / a.C;
                int c = r0 - i * a.C;
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const int r = r0 + u * RPP;
                    const bool live = r < rows;
                    const int ri = i * EC + e * a.C + c;  // the id's place in the tile's [token, layer, column]
                    const int64_t local = (live ? ids[ri] : rs) - rs;
                    ok[u] = live && local >= 0 && local < R;
                    const uint8_t* rec = table + (ok[u] ? local : 0) * (2 * D);
                    v[u] = *reinterpret_cast<const u32x4*>(rec + lr * 16);
                    sc[u] = reinterpret_cast<const float*>(rec + D)[sidx];
                    dst[u] = live ? o + ((tile0 + i) * a.C + c) * D + lr * 16 : nullptr;
                    i += step_i;
                    c += step_c;
                    if (c >= a.C) {
                        c -= a.C;
                        ++i;
                    }
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    if (dst[u] == nullptr) continue;
                    u32x4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
                    if (ok[u]) dequant16(v[u], sc[u], o0, o1);
                    u32x4* d = reinterpret_cast<u32x4*>(dst[u]);
                    d[0] = o0;
                    d[1] = o1;
                }
            }
        }
    }
}

}  // namespace
}  // namespace engram

using namespace engram;

namespace {

// Validation and launch shared by both entry points; `gs` null = hash only.
int hash_entry(const char* name, const int64_t* input_ids, int64_t B, int64_t L, int64_t start_pos,
               const uint8_t* token_mask, const int64_t* token_map, int64_t vocab, int64_t* cache, int64_t cache_B,
               int64_t cache_L, const int64_t* multipliers, const int64_t* primes, const int64_t* offsets, int32_t E,
               int32_t N, int32_t H, int64_t pad_id, int64_t dead, int64_t* hash_ids, int D, const GatherSide* gs,
               void* stream, int32_t* hash_ids32 = nullptr) {
    if (B < 0 || L < 0 || start_pos < 0) return fail(ENGRAM_EINVAL, "%s: negative B, L or start_pos", name);
    if (N < 2 || N > kMaxN) return fail(ENGRAM_EINVAL, "%s: N=%d outside [2, %d]", name, N, kMaxN);
    if (E < 1 || E > kMaxE) return fail(ENGRAM_EINVAL, "%s: E=%d outside [1, %d]", name, E, kMaxE);
    if (H < 1 || static_cast<int64_t>(N - 1) * H > kMaxC)
        return fail(ENGRAM_EINVAL, "%s: H=%d gives more than %d columns", name, H, kMaxC);
    if (vocab < 1) return fail(ENGRAM_EINVAL, "%s: vocab < 1", name);
    if (B > cache_B || cache_L < 0 || start_pos + L > cache_L)
        return fail(ENGRAM_ERANGE, "%s: B=%lld, positions up to %lld need a cache of at least [%lld, %lld], "
                    "have [%lld, %lld]", name, (long long)B, (long long)(start_pos + L), (long long)B,
                    (long long)(start_pos + L), (long long)cache_B, (long long)cache_L);
    const int64_t T = B * L;
    if (T == 0) return ENGRAM_OK;
    if (!input_ids || !token_map || !cache || !multipliers || !primes || !offsets || (!hash_ids && !hash_ids32 && !gs))
        return fail(ENGRAM_EINVAL, "%s: null required pointer", name);
    if (!aligned(hash_ids32, 4)) return fail(ENGRAM_EINVAL, "%s: int32 ids not 4-byte aligned", name);
    for (const void* p : {(const void*)input_ids, (const void*)token_map, (const void*)cache,
                          (const void*)multipliers, (const void*)primes, (const void*)offsets,
                          (const void*)hash_ids})
        if (!aligned(p, 8)) return fail(ENGRAM_EINVAL, "%s: int64 array not 8-byte aligned", name);

    HashArgs a;
    a.input_ids = input_ids;
    a.mask = token_mask;
    a.token_map = token_map;
    a.vocab = vocab;
    a.cache = cache;
    a.cache_L = cache_L;
    a.mult = multipliers;
    a.primes = primes;
    a.offsets = offsets;
    a.T = T;
    a.L = L;
    a.start_pos = start_pos;
    a.pad = pad_id;
    a.dead = dead;
    a.E = E;
    a.N = N;
    a.H = H;
    a.C = (N - 1) * H;
    a.out = hash_ids;
    a.out32 = hash_ids32;
    // A small call (a 256-token decode step) is spread over the CUs, down to one token per workgroup: its
    // time is the dependent memory round trips plus the id arithmetic, which then runs on many CUs.  With
    // the gather, a tile's ids must also fit the LDS beside the running values (at most 32 KB of ids).
    const int EC = E * a.C;
    int tile = gs != nullptr ? kGatherTileTokens : kTileTokens;
    while (tile > 1 && gs != nullptr && tile * EC > kMaxTileIds) tile /= 2;
    while (tile > 1 && (T + tile - 1) / tile < kSpreadBlocks) tile /= 2;
    a.tile = tile;
    const int64_t blocks = (T + tile - 1) / tile;
    if (blocks > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "%s: too many tokens", name);
    const size_t smem = sizeof(int64_t) * tile * (E * (N - 1) + (gs != nullptr ? EC : 0));
    const GatherSide none{};
    const dim3 grid(static_cast<unsigned>(blocks));
    hipStream_t st = as_stream(stream);
    switch (gs != nullptr ? D : 0) {
        case 0: hipLaunchKernelGGL(hash_kernel<0>, grid, dim3(kThreads), smem, st, a, none); break;
        case 32: hipLaunchKernelGGL(hash_kernel<32>, grid, dim3(kThreads), smem, st, a, *gs); break;
        case 64: hipLaunchKernelGGL(hash_kernel<64>, grid, dim3(kThreads), smem, st, a, *gs); break;
        case 128: hipLaunchKernelGGL(hash_kernel<128>, grid, dim3(kThreads), smem, st, a, *gs); break;
        default: hipLaunchKernelGGL(hash_kernel<256>, grid, dim3(kThreads), smem, st, a, *gs); break;
    }
    return check_launch(name);
}

}  // namespace

extern "C" int engram_hash(const int64_t* input_ids, int64_t B, int64_t L, int64_t start_pos,
                           const uint8_t* token_mask, const int64_t* token_map, int64_t vocab,
                           int64_t* cache, int64_t cache_B, int64_t cache_L,
                           const int64_t* multipliers, const int64_t* primes, const int64_t* offsets,
                           int32_t E, int32_t N, int32_t H, int64_t pad_id, int64_t dead,
                           int64_t* hash_ids, void* stream) {
    return hash_entry("engram_hash", input_ids, B, L, start_pos, token_mask, token_map, vocab, cache, cache_B,
                      cache_L, multipliers, primes, offsets, E, N, H, pad_id, dead, hash_ids, 0, nullptr, stream);
}

extern "C" int engram_hash_i32(const int64_t* input_ids, int64_t B, int64_t L, int64_t start_pos,
                               const uint8_t* token_mask, const int64_t* token_map, int64_t vocab,
                               int64_t* cache, int64_t cache_B, int64_t cache_L,
                               const int64_t* multipliers, const int64_t* primes, const int64_t* offsets,
                               int32_t E, int32_t N, int32_t H, int64_t pad_id, int64_t dead,
                               int32_t* hash_ids, void* stream) {
    if (B * L > 0 && !hash_ids) return fail(ENGRAM_EINVAL, "engram_hash_i32: null required pointer");
    return hash_entry("engram_hash_i32", input_ids, B, L, start_pos, token_mask, token_map, vocab, cache, cache_B,
                      cache_L, multipliers, primes, offsets, E, N, H, pad_id, dead, nullptr, 0, nullptr, stream,
                      hash_ids);
}

extern "C" int engram_hash_gather_packed(const int64_t* input_ids, int64_t B, int64_t L, int64_t start_pos,
                                         const uint8_t* token_mask, const int64_t* token_map, int64_t vocab,
                                         int64_t* cache, int64_t cache_B, int64_t cache_L,
                                         const int64_t* multipliers, const int64_t* primes, const int64_t* offsets,
                                         int32_t E, int32_t N, int32_t H, int64_t pad_id, int64_t dead,
                                         int64_t* hash_ids, const uint8_t* const* tables, const int64_t* rows,
                                         const int64_t* row_starts, int32_t D, int32_t blk,
                                         uint16_t* const* out_bf16, void* stream) {
    const char* name = "engram_hash_gather_packed";
    if (D != 32 && D != 64 && D != 128 && D != 256)
        return fail(ENGRAM_EINVAL, "%s: D=%d not in {32, 64, 128, 256}", name, D);
    if (blk < 16 || blk % 16 != 0 || D % blk != 0)
        return fail(ENGRAM_EINVAL, "%s: blk=%d must be a multiple of 16 dividing D=%d", name, blk, D);
    if (E < 1 || E > kMaxE) return fail(ENGRAM_EINVAL, "%s: E=%d outside [1, %d]", name, E, kMaxE);
    if (N >= 2 && H >= 1 && static_cast<int64_t>(E) * (N - 1) * H > kMaxTileIds)
        return fail(ENGRAM_EINVAL, "%s: E*(N-1)*H=%lld ids per token, at most %d (a token's ids stay in LDS)", name,
                    static_cast<long long>(E) * (N - 1) * H, kMaxTileIds);
    if (B >= 0 && L >= 0 && B * L == 0)  // nothing to gather: the hash's own checks decide
        return hash_entry(name, input_ids, B, L, start_pos, token_mask, token_map, vocab, cache, cache_B, cache_L,
                          multipliers, primes, offsets, E, N, H, pad_id, dead, hash_ids, 0, nullptr, stream);
    if (!tables || !rows || !out_bf16) return fail(ENGRAM_EINVAL, "%s: null pointer array", name);
    GatherSide gs{};
    gs.blk = blk;
    for (int e = 0; e < kMaxE; ++e) {
        const int k = e < E ? e : 0;  // unused slots repeat layer 0 (never selected)
        if (e < E) {
            if (rows[e] < 1) return fail(ENGRAM_EINVAL, "%s: layer %d: R < 1", name, e);
            if (!tables[e] || !out_bf16[e]) return fail(ENGRAM_EINVAL, "%s: layer %d: null pointer", name, e);
            if (!aligned(tables[e], 2 * D) || !aligned(out_bf16[e], 16))
                return fail(ENGRAM_EINVAL, "%s: layer %d: misaligned pointer", name, e);
        }
        gs.table[e] = tables[k];
        gs.R[e] = rows[k];
        gs.row_start[e] = row_starts != nullptr ? row_starts[k] : 0;
        gs.out[e] = out_bf16[k];
    }
    return hash_entry(name, input_ids, B, L, start_pos, token_mask, token_map, vocab, cache, cache_B, cache_L,
                      multipliers, primes, offsets, E, N, H, pad_id, dead, hash_ids, D, &gs, stream);
}
