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
#include "common.h"

namespace engram {
namespace {

constexpr int kMaxN = 8;
constexpr int kMaxE = 8;
constexpr int kMaxC = 1024;
constexpr int kTileTokens = 64;
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
    int64_t* out;
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

__global__ __launch_bounds__(kThreads) void hash_kernel(HashArgs a) {
    extern __shared__ int64_t roll[];  // [kTileTokens][E][N-1]
    const int NR = a.N - 1;
    const int64_t tile0 = static_cast<int64_t>(blockIdx.x) * kTileTokens;
    const int ntok = static_cast<int>(min<int64_t>(kTileTokens, a.T - tile0));
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
    int64_t* out = a.out + tile0 * EC;
    if (EC <= kThreads) {
        // Lane l keeps one (layer, column) pc = l % EC for the whole tile: its prime, offset and Barrett
        // reciprocal are fetched once, then it walks tokens l / EC, + G, + 2G, ... (G = 256 / EC); the
        // lanes of one step write G consecutive token rows, so the stores stay coalesced.
        const int G = kThreads / EC;
        if (tid >= G * EC) return;
        const int pc = tid % EC;  // = e * C + (n - 2) * H + h: primes [E, N-1, H] flat is [E, C] in column order
        const int e = pc / a.C;
        const int n1 = (pc - e * a.C) / a.H;  // n-gram size minus 2
        const int64_t prime = a.primes[pc];
        const int64_t off = a.offsets[pc];
        const uint64_t m = prime > 0 ? ~0ull / static_cast<uint64_t>(prime) : 0;
        for (int i = tid / EC; i < ntok; i += G) {
            const int64_t r = roll[(static_cast<int64_t>(i) * a.E + e) * NR + n1];
            out[i * EC + pc] = floor_mod_pos(r, prime, m) + off;
        }
        return;
    }
    for (int idx = tid; idx < total; idx += kThreads) {  // more than 256 ids per token: one id per lane and step
        const int i = idx / EC;
        const int pc = idx - i * EC;
        const int e = pc / a.C;
        const int n1 = (pc - e * a.C) / a.H;
        const int64_t prime = a.primes[pc];
        const int64_t r = roll[(static_cast<int64_t>(i) * a.E + e) * NR + n1];
        out[idx] = floor_mod_pos(r, prime, prime > 0 ? ~0ull / static_cast<uint64_t>(prime) : 0) + a.offsets[pc];
    }
}

}  // namespace
}  // namespace engram

using namespace engram;

extern "C" int engram_hash(const int64_t* input_ids, int64_t B, int64_t L, int64_t start_pos,
                           const uint8_t* token_mask, const int64_t* token_map, int64_t vocab,
                           int64_t* cache, int64_t cache_B, int64_t cache_L,
                           const int64_t* multipliers, const int64_t* primes, const int64_t* offsets,
                           int32_t E, int32_t N, int32_t H, int64_t pad_id, int64_t dead,
                           int64_t* hash_ids, void* stream) {
    if (B < 0 || L < 0 || start_pos < 0) return fail(ENGRAM_EINVAL, "engram_hash: negative B, L or start_pos");
    if (N < 2 || N > kMaxN) return fail(ENGRAM_EINVAL, "engram_hash: N=%d outside [2, %d]", N, kMaxN);
    if (E < 1 || E > kMaxE) return fail(ENGRAM_EINVAL, "engram_hash: E=%d outside [1, %d]", E, kMaxE);
    if (H < 1 || static_cast<int64_t>(N - 1) * H > kMaxC)
        return fail(ENGRAM_EINVAL, "engram_hash: H=%d gives more than %d columns", H, kMaxC);
    if (vocab < 1) return fail(ENGRAM_EINVAL, "engram_hash: vocab < 1");
    if (B > cache_B || cache_L < 0 || start_pos + L > cache_L)
        return fail(ENGRAM_ERANGE, "engram_hash: B=%lld, positions up to %lld need a cache of at least [%lld, %lld], "
                    "have [%lld, %lld]", (long long)B, (long long)(start_pos + L), (long long)B,
                    (long long)(start_pos + L), (long long)cache_B, (long long)cache_L);
    const int64_t T = B * L;
    if (T == 0) return ENGRAM_OK;
    if (!input_ids || !token_map || !cache || !multipliers || !primes || !offsets || !hash_ids)
        return fail(ENGRAM_EINVAL, "engram_hash: null required pointer");
    for (const void* p : {(const void*)input_ids, (const void*)token_map, (const void*)cache,
                          (const void*)multipliers, (const void*)primes, (const void*)offsets,
                          (const void*)hash_ids})
        if (!aligned(p, 8)) return fail(ENGRAM_EINVAL, "engram_hash: int64 array not 8-byte aligned");

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
    const int64_t blocks = (T + kTileTokens - 1) / kTileTokens;
    if (blocks > 0x7FFFFFFF) return fail(ENGRAM_EINVAL, "engram_hash: too many tokens");
    const size_t smem = sizeof(int64_t) * kTileTokens * E * (N - 1);
    hipLaunchKernelGGL(hash_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), smem, as_stream(stream), a);
    return check_launch("engram_hash");
}
