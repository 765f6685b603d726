/*
 * Drives every function of the CPU oracle once on small inputs, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py):
 * out-of-bounds accesses, signed overflow, bad shifts and the like abort the
 * run.  The inputs cover the edge cases the oracle handles: masked spans,
 * sequence starts, chunked calls that read the cache, full-range int64
 * multipliers whose products wrap, ids outside the table, every fp8 byte,
 * NaN/subnormal/-0 rounding, zero tokens.  Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "engram_oracle.h"

static uint64_t state = 0x1234567887654321ull;
static uint64_t next_u64(void) { /* xorshift64*, a fixed driver input stream */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return state * 0x2545F4914F6CDD1Dull;
}

static int fails = 0;
#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
            ++fails;                                                   \
        }                                                              \
    } while (0)

static void drive_hash(void) {
    enum { B = 3, L = 40, E = 2, N = 4, H = 2, V = 50 };
    const int C = (N - 1) * H;
    int64_t ids[B * L], tmap[V], mult[E * N], primes[E * (N - 1) * H], offs[E * C];
    uint8_t mask[B * L];
    for (int i = 0; i < B * L; ++i) {
        ids[i] = (int64_t)(next_u64() % (V + 3)) - 1; /* includes -1 and ids past the vocabulary */
        mask[i] = (i % 11) < 8;
    }
    for (int i = 0; i < V; ++i) tmap[i] = (int64_t)(next_u64() % 30);
    for (int i = 0; i < E * N; ++i) mult[i] = (int64_t)next_u64(); /* full range: products wrap */
    int64_t acc = 0;
    for (int i = 0; i < E * (N - 1) * H; ++i) primes[i] = 101 + 2 * i;
    for (int e = 0; e < E; ++e)
        for (int c = 0; c < C; ++c) { offs[e * C + c] = acc; acc += primes[e * C + c]; }
    int64_t cache[B * (L + 8)];
    memset(cache, 0, sizeof cache);
    int64_t out[B * L * E * C];
    EXPECT(oracle_hash(ids, B, L, 0, mask, tmap, V, cache, B, L + 8, mult, primes, offs, E, N, H, 2, -1, out) == 0);
    for (int i = 0; i < B * L * E * C; ++i) EXPECT(out[i] >= 0 && out[i] < acc);
    /* chunked: the same tokens in calls of 7 and 1, reading the cache */
    int64_t cache2[B * (L + 8)], out2[B * 7 * E * C];
    memset(cache2, 0, sizeof cache2);
    int64_t chunk_ids[B * 7];
    uint8_t chunk_mask[B * 7];
    for (int s0 = 0; s0 + 7 <= L; s0 += 7) {
        for (int b = 0; b < B; ++b)
            for (int l = 0; l < 7; ++l) {
                chunk_ids[b * 7 + l] = ids[b * L + s0 + l];
                chunk_mask[b * 7 + l] = mask[b * L + s0 + l];
            }
        EXPECT(oracle_hash(chunk_ids, B, 7, s0, chunk_mask, tmap, V, cache2, B, L + 8, mult, primes, offs, E, N, H,
                           2, -1, out2) == 0);
        for (int b = 0; b < B; ++b)
            EXPECT(memcmp(out2 + b * 7 * E * C, out + (b * L + s0) * E * C, sizeof(int64_t) * 7 * E * C) == 0);
    }
    /* errors and zero tokens */
    EXPECT(oracle_hash(ids, B, L, 9, NULL, tmap, V, cache, B, L + 8, mult, primes, offs, E, N, H, 2, -1, out) ==
           ORACLE_ERANGE);
    EXPECT(oracle_hash(ids, 0, 0, 0, NULL, tmap, V, cache, B, L + 8, mult, primes, offs, E, N, H, 2, -1, out) == 0);
}

static void drive_gather(void) {
    enum { R = 37, D = 64, BLK = 32, T = 9, STRIDE = 5, C = 4 };
    uint8_t w[R * D];
    float sc[R * (D / BLK)];
    for (int i = 0; i < R * D; ++i) w[i] = (uint8_t)(i * 7 + 3);
    for (int i = 0; i < R * (D / BLK); ++i) sc[i] = ldexpf(1.0f + (float)(next_u64() % 1000) / 1000.0f, -(int)(i % 9));
    sc[3] = 1e-40f; /* subnormal scale */
    int64_t ids[T * STRIDE];
    for (int i = 0; i < T * STRIDE; ++i) ids[i] = (int64_t)(next_u64() % (R + 20)) + 5; /* both sides of [10, 10+R) */
    ids[0] = INT64_MIN;
    ids[1] = INT64_MAX;
    ids[2] = 10;          /* the first row of the share */
    ids[3] = 10 + R - 1;  /* its last row */
    ids[4] = 10 + R;      /* one past it */
    uint16_t out[T * C * D];
    uint8_t raw[T * C * D];
    float rsc[T * C * (D / BLK)];
    EXPECT(oracle_gather_dequant(ids, T, STRIDE, C, w, sc, R, 10, D, BLK, out, raw, rsc) == 0);
    EXPECT(oracle_gather_dequant(ids, T, STRIDE, C, w, sc, R, 10, D, BLK, out, NULL, NULL) == 0);
    EXPECT(oracle_gather_dequant(ids, 0, STRIDE, C, w, sc, R, 0, D, BLK, out, NULL, NULL) == 0);
    EXPECT(oracle_gather_dequant(ids, T, STRIDE, C, w, sc, R, 0, D, 24, out, NULL, NULL) == ORACLE_EINVAL);
    /* the one-byte scale formats and int32 ids */
    uint8_t sc8[R * (D / 16)], rsc8[T * C * (D / 16)];
    int32_t ids32[T * STRIDE];
    for (int i = 0; i < R * (D / 16); ++i) sc8[i] = (uint8_t)next_u64();
    for (int i = 0; i < T * STRIDE; ++i) ids32[i] = (int32_t)(ids[i] > INT32_MAX || ids[i] < INT32_MIN ? -1 : ids[i]);
    EXPECT(oracle_gather_dequant_fmt(ids32, 4, T, STRIDE, C, w, sc8, 1, R, 10, D, 32, out, raw, rsc8) == 0);
    EXPECT(oracle_gather_dequant_fmt(ids, 8, T, STRIDE, C, w, sc8, 2, R, 10, D, 16, out, raw, rsc8) == 0);
    EXPECT(oracle_gather_dequant_fmt(ids, 8, T, STRIDE, C, w, sc, 0, R, 10, D, 32, out, raw, rsc) == 0);
    EXPECT(oracle_gather_dequant_fmt(ids, 2, T, STRIDE, C, w, sc, 0, R, 10, D, 32, out, raw, rsc) == ORACLE_EINVAL);
    for (int b = 0; b < 256; ++b) {
        const float v = oracle_e4m3fn_decode((uint8_t)b);
        EXPECT(isnan(v) == ((b & 0x7F) == 0x7F));
    }
    EXPECT(oracle_bf16_rne(NAN) != 0);
    EXPECT(oracle_bf16_rne(-0.0f) == 0x8000);
    EXPECT(oracle_bf16_rne(1e-40f) == 0x0001);
    EXPECT(oracle_bf16_rne(INFINITY) == 0x7F80);
}

static void drive_wkv_gate(void) {
    enum { T = 5, K = 48, HC = 3, DIM = 16, NOUT = (HC + 1) * DIM };
    uint16_t a[T * K], w[NOUT * K], x[T * HC * DIM], q[HC * DIM], k[HC * DIM], kvb[T * NOUT];
    for (int i = 0; i < T * K; ++i) a[i] = (uint16_t)(0x3F80 + (next_u64() % 0x7F)) ^ (uint16_t)((i & 1) << 15);
    for (int i = 0; i < NOUT * K; ++i) w[i] = (uint16_t)(0x3C00 + (next_u64() % 0x100));
    for (int i = 0; i < T * HC * DIM; ++i) x[i] = (uint16_t)(0x3F00 + (next_u64() % 0x100));
    for (int i = 0; i < HC * DIM; ++i) { q[i] = 0x3F80; k[i] = 0x4000; }
    double kv[T * NOUT];
    EXPECT(oracle_wkv(a, w, kv, T, K, NOUT) == 0);
    for (int i = 0; i < T * NOUT; ++i) kvb[i] = oracle_bf16_rne((float)kv[i]);
    memset(kvb, 0, sizeof(uint16_t) * DIM); /* a zero key: the eps path */
    double dot[T * HC], gate[T * HC], out[T * HC * DIM];
    EXPECT(oracle_gate_dot(x, kvb, NOUT, q, k, 1e-20, dot, T, HC, DIM) == 0);
    uint8_t mask[T] = {1, 0, 1, 1, 0};
    EXPECT(oracle_gate_output(x, kvb, NOUT, dot, mask, gate, out, T, HC, DIM) == 0);
    EXPECT(oracle_gate_output(x, kvb, NOUT, dot, NULL, gate, out, T, HC, DIM) == 0);
    EXPECT(oracle_gate_dot(x, kvb, HC * DIM - 1, q, k, 1e-20, dot, T, HC, DIM) == ORACLE_EINVAL);
    EXPECT(oracle_wkv(a, w, kv, 0, K, NOUT) == 0);
}

static void drive_mx(void) {
    enum { T = 4, K = 96, N = 7, BLK = 32 };
    uint16_t x[T * K], w[N * K];
    for (int i = 0; i < T * K; ++i) x[i] = (uint16_t)next_u64();  /* any bf16 pattern but NaN/inf: */
    for (int i = 0; i < T * K; ++i)
        if ((x[i] & 0x7F80) == 0x7F80) x[i] &= 0xBFFF;
    for (int i = 0; i < N * K; ++i) w[i] = (uint16_t)(0x3C00 + (next_u64() % 0x200));
    memset(x + K, 0, sizeof(uint16_t) * BLK);  /* an all-zero block */
    x[2 * K] = 0x0001;                         /* the smallest subnormal */
    uint8_t aq[T * K], as_[T * (K / BLK)], wq[N * K], ws[N * (K / BLK)];
    EXPECT(oracle_mx_quant(x, T, K, BLK, aq, as_) == 0);
    EXPECT(oracle_mx_quant(w, N, K, BLK, wq, ws) == 0);
    EXPECT(as_[K / BLK] == 0); /* row 1, block 0: all zero */
    double kv[T * N];
    EXPECT(oracle_wkv_mx(aq, as_, wq, ws, kv, T, K, N, BLK) == 0);
    EXPECT(oracle_mx_quant(x, T, K, 40, aq, as_) == ORACLE_EINVAL); /* 96 % 40 != 0 */
    for (int b = 0; b < 256; ++b) {
        const double v = oracle_e8m0_decode((uint8_t)b);
        EXPECT(isnan(v) == (b == 255));
        if ((b & 0x7F) != 0x7F) EXPECT(oracle_e4m3fn_encode_sat(oracle_e4m3fn_decode((uint8_t)b)) == b);
    }
    EXPECT(oracle_e4m3fn_encode_sat(1e300) == 0x7E);
    EXPECT(oracle_e4m3fn_encode_sat(-1e-300) == 0x80);
    EXPECT(oracle_e4m3fn_encode_sat(NAN) == 0x7F);
}

int main(void) {
    drive_hash();
    drive_gather();
    drive_wkv_gate();
    drive_mx();
    if (fails) {
        fprintf(stderr, "%d expectations failed\n", fails);
        return 1;
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
