/*
 * engram.h -- C ABI of libengram.so, the Engram forward hot path on AMD
 * Instinct MI355X (gfx950).
 *
 * The operations are those of the DeepSeek V4.1 model pages
 * (open-model-atlas.klimov-ivan-k.chatgpt.site, "stack-hashes" page; the same
 * classes appear on atlas.klimoza.dev "engram-first/lookup" and
 * "engram-first/streams"):
 *
 *   engram_hash            -- the engram hash module's forward
 *   engram_gather_dequant  -- ParallelEngramEmbedding.forward (one rank)
 *   engram_wkv             -- the `wkv` Linear inside Engram.forward
 *   engram_gate_dot        -- Engram.forward up to the gate pre-activation `dot`
 *   engram_gate_output     -- the rest of Engram.forward: the dot, the gate,
 *                             the token mask and the residual add
 *   engram_wkv_gate        -- engram_wkv and engram_gate_dot in one pass: the
 *                             keys are reduced where they are computed and
 *                             never written; only the value columns are stored
 *   engram_gate_residual   -- the gate, the token mask and the residual add
 *                             from a given dot (after engram_wkv_gate)
 *
 * and forms of the same steps that save memory traffic or launches:
 *
 *   engram_pack_table, engram_gather_dequant_packed
 *                          -- the table as one record per row (its fp8 bytes
 *                             and its scales), gathered with one line per row
 *   engram_hash_gather_packed
 *                          -- engram_hash and every layer's packed gather in
 *                             one launch
 *   engram_hash_i32, engram_gather_dequant_fmt
 *                          -- int32 ids, and the table's block scales as E8M0
 *                             or float8_e4m3fn bytes
 *   engram_wkv_gate_layers -- engram_wkv_gate for every layer in one launch
 *
 * the fp8 block-scaled (OCP MX) form of the `wkv` Linear:
 *
 *   engram_mx_quant        -- bf16 rows to MX fp8 (E4M3 + an E8M0 scale per 32 columns)
 *   engram_gather_mx, engram_gather_mx_packed
 *                          -- the gather + dequant writing its rows as MX fp8
 *                             (engram_mx_quant of engram_gather_dequant's rows)
 *   engram_wkv_mx          -- the projection on MX fp8 operands
 *   engram_wkv_mx_gate     -- engram_wkv_mx fused with the gate pre-activation
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array argument is a DEVICE pointer (memory the caller allocated on
 *   the current HIP device), row-major and contiguous unless a stride is
 *   given -- except the per-layer lists of engram_hash_gather_packed and
 *   engram_wkv_gate_layers, which are HOST arrays of device pointers (or of
 *   sizes), read during the call only.  The caller owns all memory; the
 *   library allocates nothing and keeps no pointer after a call returns.
 * - bf16 values are passed as their 16-bit patterns (uint16_t).
 * - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *   kernels on it and never synchronise; results are ready when the stream
 *   reaches them.
 * - Arguments are validated on the host before anything is enqueued.  A call
 *   returns ENGRAM_OK, or an error status and enqueues nothing (ENGRAM_EHIP
 *   is the exception: the launch itself failed).  engram_last_error() gives
 *   a one-line description of the last failure on the calling thread.
 * - A size of zero tokens is valid and enqueues nothing.
 * - Pointers to arrays read or written with 16-byte vector accesses must be
 *   16-byte aligned; this is stated per argument below.
 */
#ifndef ENGRAM_H
#define ENGRAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum engram_status {
    ENGRAM_OK = 0,
    ENGRAM_EINVAL = 1, /* a null pointer, a bad size, an unsupported shape or a misaligned pointer */
    ENGRAM_ERANGE = 2, /* the compressed-id cache is too small for the batch / positions */
    ENGRAM_EHIP = 3    /* the HIP runtime rejected a launch */
};

/* Static description of a status code. */
const char* engram_status_string(int status);

/* Description of the last failure on the calling thread ("" if none). */
const char* engram_last_error(void);

/* Version of the ABI described here (currently 1). */
int engram_abi_version(void);

/*
 * engram_hash -- n-gram hash ids of a chunk of tokens (stack-hashes page: the
 * hash module's forward).
 *
 * For each sequence b < B and position p = start_pos + l (l < L):
 *   c[p] = token_map[input_ids[b,l]], or `dead` where token_mask[b,l] == 0
 *          (an id outside [0, vocab) is treated the same way);
 *   cache[b, p] = c[p];
 *   slot s = 0..N-1 holds c[p-s], read from this chunk when p-s >= start_pos
 *          and from the cache when p-s < start_pos; once a slot is blocked
 *          (p < s, or c[p-s] == dead) it and every longer slot hold pad_id;
 *   r_n = XOR over s < n of (slot_s * multipliers[e,s]), int64 wrap-around;
 *   hash_ids[b,l,e,(n-2)*H + h] = floormod(r_n, primes[e,n-2,h]) + offsets[e,(n-2)*H + h]
 *          for n = 2..N, h < H (floormod takes the divisor's sign).
 *
 * input_ids    int64 [B, L]
 * token_mask   uint8 [B, L], nonzero = the token takes part; NULL = all take part
 * token_map    int64 [vocab], values in [0, compressed vocab)
 * cache        int64 [cache_B, cache_L], in/out.  Positions [start_pos, start_pos+L)
 *              of rows 0..B-1 are written; positions [start_pos-N+1, start_pos)
 *              are read.  Row b is sequence b across calls.
 * multipliers  int64 [E, N]
 * primes       int64 [E, N-1, H], every entry > 0
 * offsets      int64 [E, (N-1)*H]
 * dead         the sentinel stored for masked positions; must differ from every
 *              token_map value
 * hash_ids     int64 [B, L, E, (N-1)*H], out
 * Limits: B, L >= 0; start_pos >= 0; 2 <= N <= 8; 1 <= E <= 8; H >= 1;
 *         (N-1)*H <= 1024.  ERANGE if B > cache_B or start_pos + L > cache_L.
 * Calls that share a cache row must be ordered on one stream.
 */
int engram_hash(const int64_t* input_ids, int64_t B, int64_t L, int64_t start_pos,
                const uint8_t* token_mask, const int64_t* token_map, int64_t vocab,
                int64_t* cache, int64_t cache_B, int64_t cache_L,
                const int64_t* multipliers, const int64_t* primes, const int64_t* offsets,
                int32_t E, int32_t N, int32_t H, int64_t pad_id, int64_t dead,
                int64_t* hash_ids, void* stream);

/*
 * engram_hash_i32 -- engram_hash with int32 ids: hash_ids int32 [B, L, E,
 * (N-1)*H], out, 4-byte aligned; an id outside [0, 2^31) is stored as -1 (so
 * every gather treats it as outside its rows).  Half the id bytes of
 * engram_hash for the released tables, whose ids are all below 384,016,682.
 * Everything else as engram_hash.
 */
int engram_hash_i32(const int64_t* input_ids, int64_t B, int64_t L, int64_t start_pos,
                    const uint8_t* token_mask, const int64_t* token_map, int64_t vocab,
                    int64_t* cache, int64_t cache_B, int64_t cache_L,
                    const int64_t* multipliers, const int64_t* primes, const int64_t* offsets,
                    int32_t E, int32_t N, int32_t H, int64_t pad_id, int64_t dead,
                    int32_t* hash_ids, void* stream);

/*
 * engram_gather_dequant -- fetch and dequantise the fp8 rows of one layer's
 * hash ids (stack-hashes page: ParallelEngramEmbedding.forward, one rank's
 * rows [row_start, row_start + R)).
 *
 * For token t < T and column c < C, id = hash_ids[t * id_token_stride + c]:
 *   ok   = row_start <= id < row_start + R;  row = ok ? id - row_start : 0
 *   out_bf16[t,c,j]  = ok ? bf16(fp32(e4m3fn(weight[row,j])) * scale[row, j/blk]) : +0
 *                      (fp32 product rounded to nearest even, then bf16 rounded
 *                      to nearest even: two roundings, as the page does)
 *   out_fp8[t,c,j]   = weight[row,j]        (optional)
 *   out_scale[t,c,s] = scale[row,s]         (optional)
 * The bf16 output is the [T, C*D] operand of engram_wkv.
 *
 * hash_ids         int64, row stride id_token_stride >= C (e.g. layer e of
 *                  engram_hash's output: hash_ids + e*C with stride E*C); 8-byte aligned
 * weight           uint8 [R, D], float8_e4m3fn (OCP E4M3FN) bytes; 16-byte aligned
 * scale            float32 [R, D/blk]; 4-byte aligned
 * out_bf16         uint16 [T, C, D] bf16 bits, out; 16-byte aligned
 * out_fp8          uint8 [T, C, D] or NULL; 16-byte aligned
 * out_scale        float32 [T, C, D/blk] or NULL
 * Limits: D in {32, 64, 128, 256}; blk a multiple of 16 that divides D;
 *         1 <= C <= 1024; R >= 1; T >= 0.
 */
int engram_gather_dequant(const int64_t* hash_ids, int64_t T, int64_t id_token_stride, int32_t C,
                          const uint8_t* weight, const float* scale, int64_t R, int64_t row_start,
                          int32_t D, int32_t blk, uint16_t* out_bf16, uint8_t* out_fp8,
                          float* out_scale, void* stream);

/*
 * engram_gather_dequant_fmt -- engram_gather_dequant with the table's block
 * scales in another `scale_dtype` (stack-hashes page: ParallelEngramEmbedding's
 * `scale` and `scales.float()`; the page names the dtype but does not fix it)
 * and with int32 or int64 ids.  Scale formats: 0 = float32 [R, D/blk] (exactly
 * engram_gather_dequant); 1 = E8M0 bytes [R, D/blk], scale 2^(s-127) (0xFF NaN),
 * the pages' indexer format (blocks of 32); 2 = float8_e4m3fn bytes [R, D/blk],
 * the pages' compressed-KV format (blocks of 16).  The dequant is unchanged: the
 * decoded scale (exact in fp32) times the decoded fp8 value rounded to fp32,
 * then to bf16, both to nearest even.
 *
 * hash_ids   int64 (id_bytes 8, 8-byte aligned) or int32 (id_bytes 4, 4-byte aligned)
 *            [T, id_token_stride], first C columns used (engram_hash or engram_hash_i32)
 * scale      [R, D/blk] elements of the format; float32 4-byte aligned
 * out_scale  [T, C, D/blk] elements of the format, the gathered scales as stored, or NULL
 * Other arguments, limits and errors: as engram_gather_dequant.
 */
int engram_gather_dequant_fmt(const void* hash_ids, int32_t id_bytes, int64_t T, int64_t id_token_stride,
                              int32_t C, const uint8_t* weight, const void* scale, int32_t scale_format, int64_t R,
                              int64_t row_start, int32_t D, int32_t blk, uint16_t* out_bf16, uint8_t* out_fp8,
                              void* out_scale, void* stream);

/*
 * engram_pack_table -- copy one layer's table (the pages' two tensors: the
 * fp8 rows `weight` [R, D] and their fp32 block scales `scale` [R, D/blk]) into
 * one packed table of R records of 2*D bytes:
 *   packed[r, 0 : D)               = weight[r, :]
 *   packed[r, D : D + 4*(D/blk))   = scale[r, :] (little-endian fp32)
 *   packed[r, D + 4*(D/blk) : 2*D) = 0
 * A record is aligned to its size, so at D <= 64 a row and its scales share one
 * 128-byte line and a random lookup reads one line instead of two.  A one-off
 * layout conversion (at table load), not a step of the forward.
 *
 * weight  uint8 [R, D]; 16-byte aligned
 * scale   float32 [R, D/blk]; 4-byte aligned
 * packed  uint8 [R, 2*D], out; aligned to 2*D bytes; caller-owned
 * Limits: D in {32, 64, 128, 256}; blk a multiple of 16 that divides D; R >= 0.
 */
int engram_pack_table(const uint8_t* weight, const float* scale, int64_t R, int32_t D, int32_t blk,
                      uint8_t* packed, void* stream);

/*
 * engram_gather_dequant_packed -- engram_gather_dequant on a packed table
 * (engram_pack_table's layout): the same outputs, bit for bit, with
 * weight[row, j] = table[row, j] and scale[row, s] = fp32 at table[row, D + 4s].
 *
 * table  uint8 [R, 2*D]; aligned to 2*D bytes.  Other arguments, outputs,
 *        limits and errors as engram_gather_dequant.
 */
int engram_gather_dequant_packed(const int64_t* hash_ids, int64_t T, int64_t id_token_stride, int32_t C,
                                 const uint8_t* table, int64_t R, int64_t row_start, int32_t D, int32_t blk,
                                 uint16_t* out_bf16, uint8_t* out_fp8, float* out_scale, void* stream);

/*
 * engram_hash_gather_packed -- engram_hash, then engram_gather_dequant_packed
 * of every layer's ids, in one launch (stack-hashes page: the hash module's
 * forward, then ParallelEngramEmbedding.forward per engram layer).  The ids
 * stay on chip between the two; the results are those of the two entry points
 * called in turn, bit for bit.
 *
 * For token t < B*L, layer e < E and column c < C = (N-1)*H, with
 * id = the engram_hash id [t, e, c]:
 *   ok = row_starts[e] <= id < row_starts[e] + rows[e]
 *   out_bf16[e][t, c, j] = ok ? bf16(fp32(e4m3fn(byte j of record r)) * scale) : +0,
 *   r = id - row_starts[e], scale = fp32 at byte D + 4*(j/blk) of record r.
 *
 * Hash arguments, the cache update, limits and errors: as engram_hash, except
 * hash_ids  int64 [B, L, E, C] out, or NULL (the ids are then not stored).
 * tables    host array of E device pointers: layer e's packed table,
 *           uint8 [rows[e], 2*D] (engram_pack_table's layout), aligned to 2*D
 * rows      host array of E row counts, each >= 1
 * row_starts host array of E first rows (this GPU's share), or NULL = all 0
 * D, blk    row width in {32, 64, 128, 256}; block size, a multiple of 16
 *           that divides D
 * out_bf16  host array of E device pointers: layer e's rows, uint16
 *           [B*L, C, D] bf16 bits, out; 16-byte aligned
 * Limits: engram_hash's, and E*C <= 4096 ids per token.
 * The host arrays are read during the call only.
 */
int engram_hash_gather_packed(const int64_t* input_ids, int64_t B, int64_t L, int64_t start_pos,
                              const uint8_t* token_mask, const int64_t* token_map, int64_t vocab,
                              int64_t* cache, int64_t cache_B, int64_t cache_L,
                              const int64_t* multipliers, const int64_t* primes, const int64_t* offsets,
                              int32_t E, int32_t N, int32_t H, int64_t pad_id, int64_t dead,
                              int64_t* hash_ids, const uint8_t* const* tables, const int64_t* rows,
                              const int64_t* row_starts, int32_t D, int32_t blk,
                              uint16_t* const* out_bf16, void* stream);

/*
 * engram_wkv -- the projection kv = A * W^T (stack-hashes page: Engram's
 * `wkv` Linear, n_hash_cols*head_dim -> dim*(hc_mult+1), no bias).
 *
 * a    uint16 [T, K] bf16 bits (the flattened gathered rows); 16-byte aligned
 * w    uint16 [Nout, K] bf16 bits; 16-byte aligned
 * kv   uint16 [T, Nout] bf16 bits, out: fp32 accumulation, rounded to nearest
 *      even once.  Columns [0, hc*dim) are the hc keys, [hc*dim, Nout) the value.
 *      16-byte aligned.
 * Limits: T >= 0; K >= 8 and K % 8 == 0; Nout >= 1 and Nout % 8 == 0.
 */
int engram_wkv(const uint16_t* a, const uint16_t* w, uint16_t* kv, int64_t T, int32_t K, int32_t Nout,
               void* stream);

/*
 * engram_gate_dot -- the gate pre-activation per (token, hc copy)
 * (stack-hashes page: Engram.forward, `rstd` and `dot`).
 *
 *   w[c,j]   = fp32(q_weight[c,j]) * fp32(k_weight[c,j])
 *   dot[t,c] = sum_j h[j] w[c,j] key[j]
 *              * rsqrt(mean_j h[j]^2 + eps) * rsqrt(mean_j key[j]^2 + eps) * dim^-1/2
 *   with h = x[t,c,:], key = kv[t, c*dim : (c+1)*dim]; sums in fp32.
 *
 * x          uint16 [T, hc, dim] bf16 bits; 16-byte aligned
 * kv         uint16 bf16 bits, row stride ld_kv >= hc*dim (engram_wkv's output,
 *            ld_kv = Nout); 16-byte aligned, ld_kv % 8 == 0
 * q_weight, k_weight  uint16 [hc, dim] bf16 bits; 16-byte aligned
 * dot        float32 [T, hc], out
 * Limits: T >= 0; 1 <= hc <= 64; dim >= 8 and dim % 8 == 0.
 */
int engram_gate_dot(const uint16_t* x, const uint16_t* kv, int64_t ld_kv, const uint16_t* q_weight,
                    const uint16_t* k_weight, float eps, float* dot, int64_t T, int32_t hc, int32_t dim,
                    void* stream);

/*
 * engram_gate_output -- the end of Engram.forward (stack-hashes page: `dot`,
 * `gate`, the token mask and the returned sum), one pass over the stream.
 *
 *   dot[t,c]   as engram_gate_dot computes it
 *   gate[t,c]  = sigmoid(copysign(sqrt(max(|dot|, 1e-6)), dot)); 0 if token_mask[t] == 0
 *   out[t,c,j] = bf16(fp32(h[j] + fp32(gate[t,c] * value[j])))
 *   with h = x[t,c,:], value = kv[t, hc*dim : (hc+1)*dim] (one value row per token,
 *   shared by its hc copies).  The product and the sum are rounded separately (no
 *   fused multiply-add), then the sum is rounded to bf16 to nearest even, so a
 *   masked token's output equals x bit for bit (x = -0 with value >= +0 gives +0,
 *   by IEEE addition).
 *
 * x          uint16 [T, hc, dim] bf16 bits; 16-byte aligned
 * kv         uint16 bf16 bits, row stride ld_kv >= (hc+1)*dim: keys in columns
 *            [0, hc*dim), value in [hc*dim, (hc+1)*dim) (engram_wkv's output,
 *            ld_kv = Nout); 16-byte aligned, ld_kv % 8 == 0
 * q_weight, k_weight  uint16 [hc, dim] bf16 bits; 16-byte aligned
 * eps        the RMS epsilon (norm_eps)
 * token_mask uint8 [T], nonzero = the token takes part, 0 = its gate is shut;
 *            NULL = every token takes part
 * out        uint16 [T, hc, dim] bf16 bits, out; 16-byte aligned; must not
 *            overlap x or kv
 * dot        float32 [T, hc], out, optional (NULL = not written); 4-byte aligned
 * Limits: T >= 0; 1 <= hc <= 64; 8 <= dim <= 8192 and dim % 8 == 0.
 */
int engram_gate_output(const uint16_t* x, const uint16_t* kv, int64_t ld_kv, const uint16_t* q_weight,
                       const uint16_t* k_weight, float eps, const uint8_t* token_mask, uint16_t* out,
                       float* dot, int64_t T, int32_t hc, int32_t dim, void* stream);

/*
 * engram_wkv_gate -- the `wkv` Linear and the gate pre-activation of
 * Engram.forward (stack-hashes page: `kv`, its key/value split, `rstd`, `dot`)
 * fused: the product's key columns are rounded to bf16 and reduced against
 * the stream inside the projection, so the [T, hc*dim] keys are never
 * written; only the value columns are stored.
 *
 *   kv       = bf16(a * w^T)  (fp32 accumulation), Nout = (hc+1)*dim
 *   value    = kv[:, hc*dim : (hc+1)*dim]                       -> value
 *   dot[t,c] = as engram_gate_dot, with key = kv[t, c*dim : (c+1)*dim]  -> dot
 * The sums of a (token, copy) are formed per 128 columns (fp32) in the
 * projection, kept in `workspace`, and added in slice order by a second
 * kernel on the same stream, so results are deterministic.
 *
 * a          uint16 [T, K] bf16 bits; 16-byte aligned
 * w          uint16 [(hc+1)*dim, K] bf16 bits; 16-byte aligned
 * x          uint16 [T, hc, dim] bf16 bits (the stream); 16-byte aligned
 * q_weight, k_weight  uint16 [hc, dim] bf16 bits; 16-byte aligned
 * eps        the RMS epsilon (norm_eps)
 * value      uint16 [T, ld_value] bf16 bits, out (first dim columns of each row
 *            written); ld_value >= dim, ld_value % 8 == 0; 16-byte aligned
 * dot        float32 [T, hc], out; 4-byte aligned
 * workspace  device scratch of at least engram_wkv_gate_workspace_bytes(T, hc,
 *            dim) bytes, 16-byte aligned, owned by the caller; its contents
 *            are overwritten and need no initialisation.  Two calls in flight
 *            at once must not share it.
 * Limits: T >= 0; K >= 64 and K % 64 == 0; 1 <= hc <= 64; dim >= 256 and
 * dim % 256 == 0 (each 256-column tile of the product lies in one key copy
 * or in the value).  Too small a workspace -> ENGRAM_ERANGE.
 */
int engram_wkv_gate(const uint16_t* a, const uint16_t* w, const uint16_t* x, const uint16_t* q_weight,
                    const uint16_t* k_weight, float eps, uint16_t* value, int64_t ld_value, float* dot,
                    void* workspace, int64_t workspace_bytes, int64_t T, int32_t K, int32_t hc, int32_t dim,
                    void* stream);

/*
 * engram_gate_residual -- the end of Engram.forward after `dot` (stack-hashes
 * page: `gate`, the token mask, the returned sum) for a dot computed
 * elsewhere (engram_wkv_gate's):
 *
 *   gate[t,c]  = sigmoid(copysign(sqrt(max(|dot[t,c]|, 1e-6)), dot[t,c])); 0 if token_mask[t] == 0
 *   out[t,c,j] = bf16(fp32(h[j] + fp32(gate[t,c] * value[t,j]))),  h = x[t,c,:]
 * with the same rounding as engram_gate_output.
 *
 * x          uint16 [T, hc, dim] bf16 bits; 16-byte aligned
 * value      uint16 [T, ld_value] bf16 bits (first dim columns used); ld_value
 *            >= dim, ld_value % 8 == 0; 16-byte aligned
 * dot        float32 [T, hc]; 4-byte aligned
 * token_mask uint8 [T] (nonzero = takes part) or NULL = every token
 * out        uint16 [T, hc, dim] bf16 bits, out; 16-byte aligned; may be x itself
 *            (each element is read before it is written, by the same thread)
 * Limits: T >= 0; 1 <= hc <= 64; dim >= 8 and dim % 8 == 0.
 */
int engram_gate_residual(const uint16_t* x, const uint16_t* value, int64_t ld_value, const float* dot,
                         const uint8_t* token_mask, uint16_t* out, int64_t T, int32_t hc, int32_t dim,
                         void* stream);

/* Bytes of workspace engram_wkv_gate needs for T tokens (hc * dim/128 * 3 * T
 * floats), or -1 if hc or dim is outside the limits above. */
int64_t engram_wkv_gate_workspace_bytes(int64_t T, int32_t hc, int32_t dim);

/*
 * engram_wkv_gate_layers -- engram_wkv_gate for `layers` engram layers of one
 * forward call (stack-hashes page: each engram layer's Engram.forward, up to
 * `dot`), as one launch of the projection and one of the finalize: the layers'
 * tiles share the CUs, so a call too small to fill them with one layer (a
 * decode step) fills them with all.  Per layer the results are engram_wkv_gate's
 * (the value columns bit for bit; the dot up to the order of its fp32 sums).
 *
 * a, w, x, q_weight, k_weight, value, dot  host arrays of `layers` device
 *          pointers, each as engram_wkv_gate takes it; one T, K, hc, dim and
 *          ld_value for all layers
 * workspace  layers * engram_wkv_gate_workspace_bytes(T, hc, dim) bytes, 16-byte
 *          aligned; caller-owned scratch
 * Limits and errors: as engram_wkv_gate; 1 <= layers <= 8.  The host arrays are
 * read during the call only.
 */
int engram_wkv_gate_layers(int32_t layers, const uint16_t* const* a, const uint16_t* const* w,
                           const uint16_t* const* x, const uint16_t* const* q_weight,
                           const uint16_t* const* k_weight, float eps, uint16_t* const* value, int64_t ld_value,
                           float* const* dot, void* workspace, int64_t workspace_bytes, int64_t T, int32_t K,
                           int32_t hc, int32_t dim, void* stream);

/*
 * The fp8 block-scaled form of the `wkv` Linear (stack-hashes page: the released
 * config's "dtype": "fp8" and Engram.__init__'s `wkv`; the pages name the fp8
 * Linear without showing it).  Operands are in the OCP microscaling (MX) fp8
 * format: float8_e4m3fn elements, and for every 32 consecutive columns of a
 * row one E8M0 scale byte s meaning 2^(s-127) -- the block-32 / E8M0 format
 * the pages use for the indexer's quantised activations.
 *
 * MX scale layout of this library: uint8 [K/128][rows4][4], rows4 = rows
 * rounded up to a multiple of 4; byte [c][r][b] is the scale of row r,
 * columns 128c + 32b .. 128c + 32b + 31 (engram_mx_scale_bytes gives the size;
 * bytes of the padding rows are never written and never affect an output).
 */

/* Bytes of an MX scale array for `rows` rows of K columns, or -1 if K is not a
 * positive multiple of 128. */
int64_t engram_mx_scale_bytes(int64_t rows, int32_t K);

/*
 * engram_mx_quant -- bf16 rows to MX fp8 by the OCP MX rule: for each row and
 * 32-column block with largest magnitude amax, e = floor(log2 amax) - 8 (8 being
 * E4M3's largest exponent), kept in [-127, 127] (-127 for an all-zero block);
 * scale = e + 127; q = x * 2^-e rounded to the nearest E4M3FN value, ties to even,
 * magnitudes past 448 saturated to 448, the sign kept (so -0 gives 0x80).  The
 * activation side of the fp8 Linear (its bf16 input, the gathered rows), and the
 * one-off conversion of bf16 weights.
 *
 * x      uint16 [rows, K] bf16 bits, finite values; 16-byte aligned
 * q      uint8 [rows, K], out; 8-byte aligned
 * scale  uint8, engram_mx_scale_bytes(rows, K) bytes in the layout above, out
 * Limits: rows >= 0; K >= 128 and K % 128 == 0.
 */
int engram_mx_quant(const uint16_t* x, int64_t rows, int32_t K, uint8_t* q, uint8_t* scale, void* stream);

/*
 * engram_gather_mx -- engram_gather_dequant's rows as MX fp8, without the bf16
 * tensor: q, q_scale = engram_mx_quant(engram_gather_dequant(...)) viewed as
 * [T, K], K = C*D, bit for bit (the same bf16 values, the same encoding; an id
 * outside the rank's rows gives a zero row: bytes 0 and scale 0).  The fp8
 * projection's A operand straight from the table (stack-hashes page,
 * ParallelEngramEmbedding.forward, followed by the fp8 `wkv` Linear's
 * activation quantisation).
 *
 * hash_ids, T, id_token_stride, C, weight, scale, R, row_start, D, blk
 *          as engram_gather_dequant
 * q        uint8 [T, C*D] E4M3FN bytes, out; 16-byte aligned; caller-owned
 * q_scale  uint8, engram_mx_scale_bytes(T, C*D) bytes in the MX scale layout,
 *          out; caller-owned (its padding rows are not written)
 * Limits and errors: as engram_gather_dequant, and C*D % 128 == 0.
 */
int engram_gather_mx(const int64_t* hash_ids, int64_t T, int64_t id_token_stride, int32_t C, const uint8_t* weight,
                     const float* scale, int64_t R, int64_t row_start, int32_t D, int32_t blk, uint8_t* q,
                     uint8_t* q_scale, void* stream);

/* engram_gather_mx on a packed table (engram_pack_table's layout; `table` as in
 * engram_gather_dequant_packed): the same outputs, bit for bit. */
int engram_gather_mx_packed(const int64_t* hash_ids, int64_t T, int64_t id_token_stride, int32_t C,
                            const uint8_t* table, int64_t R, int64_t row_start, int32_t D, int32_t blk, uint8_t* q,
                            uint8_t* q_scale, void* stream);

/*
 * engram_wkv_mx -- the projection on MX fp8 operands:
 *   kv[t,o] = bf16( sum over 32-column blocks b of
 *                   2^(a_scale[t,b]-127) * 2^(w_scale[o,b]-127) * sum_{k in b} e4m3(a[t,k]) * e4m3(w[o,k]) )
 * with fp32 accumulation and one bf16 rounding (round to nearest even).
 *
 * a        uint8 [T, K] E4M3FN bytes; 16-byte aligned
 * a_scale  MX scales of a (T rows), layout above; 16-byte aligned
 * w        uint8 [Nout, K] E4M3FN bytes; 16-byte aligned
 * w_scale  MX scales of w (Nout rows); 16-byte aligned
 * kv       uint16 [T, Nout] bf16 bits, out: the hc keys then the value, as engram_wkv;
 *          16-byte aligned
 * Limits: T >= 0; K >= 128 and K % 128 == 0; Nout >= 8 and Nout % 8 == 0.
 */
int engram_wkv_mx(const uint8_t* a, const uint8_t* a_scale, const uint8_t* w, const uint8_t* w_scale,
                  uint16_t* kv, int64_t T, int32_t K, int32_t Nout, void* stream);

/*
 * engram_wkv_mx_gate -- engram_wkv_mx fused with the gate dot, as engram_wkv_gate
 * is for the bf16 projection (stack-hashes page, Engram.forward: `kv`, its
 * key/value split, `rstd`, `dot`, with the released config's fp8 `Linear`): the
 * key columns of the product are rounded to bf16 and reduced against the stream
 * inside the projection, never written; the value columns are stored.
 *
 *   kv       = engram_wkv_mx(a, w), Nout = (hc+1)*dim
 *   value    = kv[:, hc*dim : (hc+1)*dim]                       -> value
 *   dot[t,c] = as engram_gate_dot, with key = kv[t, c*dim : (c+1)*dim]  -> dot
 * The value columns equal engram_wkv_mx's bit for bit; the dot equals
 * engram_gate_dot on engram_wkv_mx's kv up to the order of its fp32 sums (per 128
 * columns in the projection, then added in slice order by a second kernel).
 *
 * a, a_scale, w, w_scale  as engram_wkv_mx, w having (hc+1)*dim rows
 * x, q_weight, k_weight, eps, value, ld_value, dot  as engram_wkv_gate
 * workspace  at least engram_wkv_gate_workspace_bytes(T, hc, dim) bytes, 16-byte
 *            aligned, caller-owned scratch (no initialisation needed)
 * Limits: T >= 0; K >= 384 and K % 128 == 0; 1 <= hc <= 64; dim >= 256 and
 * dim % 256 == 0; (hc+1)*dim <= 2^22; ld_value >= dim, ld_value % 8 == 0.
 * Too small a workspace -> ENGRAM_ERANGE.
 */
int engram_wkv_mx_gate(const uint8_t* a, const uint8_t* a_scale, const uint8_t* w, const uint8_t* w_scale,
                       const uint16_t* x, const uint16_t* q_weight, const uint16_t* k_weight, float eps,
                       uint16_t* value, int64_t ld_value, float* dot, void* workspace, int64_t workspace_bytes,
                       int64_t T, int32_t K, int32_t hc, int32_t dim, void* stream);

/*
 * engram_wkv_gate_layers_noalloc -- engram_wkv_gate_layers without a workspace
 * argument, for callers that cannot allocate device memory: code recorded
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The per-slice partial sums go to a file-scope device array of
 * ENGRAM_NOALLOC_SCRATCH_BYTES bytes inside the library (one per GPU, held
 * until the process ends); the call itself allocates nothing.  Results equal
 * engram_wkv_gate_layers' bit for bit (same kernels, same launch shape).
 *
 * Arguments, limits and errors: as engram_wkv_gate_layers without
 * `workspace`/`workspace_bytes`; ENGRAM_ERANGE if the layers need more than
 * ENGRAM_NOALLOC_SCRATCH_BYTES of partial sums (layers * hc * dim/128 * 3 * T
 * floats: e.g. 2 layers of 256 tokens at hc 4, dim 5120 need 983,040 bytes; at
 * most 8,738 token-layers fit at that shape).  The scratch needs no
 * initialisation (every call overwrites what it reads).
 * Every call on one GPU shares that GPU's scratch: calls that may overlap in
 * time on one GPU (on different streams, or from several host threads without
 * ordering) race and give wrong dots.  Order them on one stream.
 */
#define ENGRAM_NOALLOC_SCRATCH_BYTES (16ll << 20)
int engram_wkv_gate_layers_noalloc(int32_t layers, const uint16_t* const* a, const uint16_t* const* w,
                                   const uint16_t* const* x, const uint16_t* const* q_weight,
                                   const uint16_t* const* k_weight, float eps, uint16_t* const* value,
                                   int64_t ld_value, float* const* dot, int64_t T, int32_t K, int32_t hc,
                                   int32_t dim, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ENGRAM_H */
