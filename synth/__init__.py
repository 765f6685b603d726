"""Seeded synthetic inputs for the Engram forward path.

This module serves both sides of the parity check -- the HIP library and the
CPU oracle -- and therefore holds none of the method's arithmetic: no hashing,
no gathering, no dequantisation, no projection and no gate.  It only draws
inputs (token ids, masks, the compressed-vocab map, hash multipliers, the
prime-sized column layout, fp8 table rows and their scales, projection
weights, the residual stream) from fixed seeds.

The tables of the full-size workloads (384M rows of fp8) never exist on the
host: their bytes come from a counter-based generator, SplitMix64 (Steele,
Lea and Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014;
the constants are those of Vigna's public-domain reference), so any row can
be produced on its own.  `table_rows` is the numpy implementation; the device
implementation of the same definition is `synth/fill.hip`.

Element n (n = 0, 1, ...) of the stream with seed s is mix(s + (n + 1) * G),
G = 0x9E3779B97F4A7C15.  Row r of a table with D columns and block size blk
uses elements n = r * W + w, W = D/4 + D/blk:

* word w < D/4 gives the four fp8 bytes 4w..4w+3: byte 4w+i is
  LUT[(u >> 16 i) & 0xFFFF], where LUT maps a 16-bit draw to the E4M3 byte of
  the N(0,1) quantile at (i + 1/2) / 65536 (clipped to +-448);
* word D/4 + j gives scale j: fp32 with 23 random mantissa bits (u & 0x7FFFFF)
  and unbiased exponent -8 + ((u >> 32) mod 6), i.e. a value in [2^-8, 2^-2).
"""
from __future__ import annotations

import dataclasses
import functools
import math
from typing import Optional

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)

# Sentinel for masked positions in the compressed-id cache.  The pages use a
# DEAD sentinel without defining it; any value outside [0, compressed vocab)
# works because a DEAD slot is always replaced by the pad id before it can be
# multiplied.
DEAD = -1


# ----------------------------------------------------------------------------
# workload configurations
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class EngramConfig:
    """Sizes of one workload.  Field names follow the pages' model arguments."""

    name: str
    index: int                 # 1..5, selects the seed family 1000*index + k
    batch: int                 # B
    seqlen: int                # L (per call)
    start_pos: int
    vocab_size: int            # raw tokenizer vocab
    compressed_vocab_size: int  # Vc, the range of token_map
    max_ngram_size: int        # N
    n_heads: int               # H (engram hash heads)
    n_layers: int              # E (engram layers hashed in one call)
    head_dim: int              # D, fp8 row width
    block_size: int            # fp8 scale block
    dim: int                   # model dim
    hc_mult: int               # hyper-connection copies
    prime_base: int            # primes are searched above this value
    rows_alloc: tuple          # allocated table rows per layer (>= used)
    token_dist: str            # "uniform" or "zipf"
    zipf_s: float = 1.1
    mask_frac: float = 0.0
    pad_id: int = 2
    eps: float = 1e-20
    decode_steps: int = 0      # >0: L=1 steps after a prefill of start_pos tokens

    @property
    def n_hash_cols(self) -> int:
        return (self.max_ngram_size - 1) * self.n_heads

    @property
    def K(self) -> int:
        return self.n_hash_cols * self.head_dim

    @property
    def n_out(self) -> int:
        return self.dim * (self.hc_mult + 1)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def seed(self, k: int) -> int:
        return 1000 * self.index + k


def _cfg(**kw) -> EngramConfig:
    base = dict(max_ngram_size=4, block_size=32, hc_mult=4, pad_id=2, eps=1e-20)
    base.update(kw)
    return EngramConfig(**base)


CONFIGS = {
    1: _cfg(name="tiny", index=1, batch=1, seqlen=64, start_pos=0, vocab_size=1000,
            compressed_vocab_size=500, n_heads=2, n_layers=1, head_dim=32, dim=256,
            prime_base=1600, rows_alloc=(9670,), token_dist="uniform"),
    2: _cfg(name="mid_prefill", index=2, batch=4, seqlen=2048, start_pos=0, vocab_size=129280,
            compressed_vocab_size=99092, n_heads=8, n_layers=2, head_dim=64, dim=5120,
            prime_base=166000, rows_alloc=(4000037, 4000037), token_dist="zipf", mask_frac=0.10),
    3: _cfg(name="long_prefill", index=3, batch=1, seqlen=65536, start_pos=0, vocab_size=129280,
            compressed_vocab_size=99092, n_heads=8, n_layers=1, head_dim=64, dim=5120,
            prime_base=16000000, rows_alloc=(384006168,), token_dist="zipf"),
    4: _cfg(name="decode", index=4, batch=256, seqlen=1, start_pos=4096, vocab_size=129280,
            compressed_vocab_size=99092, n_heads=8, n_layers=2, head_dim=64, dim=5120,
            prime_base=16000000, rows_alloc=(384006168, 384016682), token_dist="zipf",
            decode_steps=64),
    5: _cfg(name="gather_stress", index=5, batch=8, seqlen=16384, start_pos=0, vocab_size=129280,
            compressed_vocab_size=99092, n_heads=8, n_layers=2, head_dim=64, dim=5120,
            prime_base=16000000, rows_alloc=(384006168, 384016682), token_dist="uniform",
            mask_frac=0.05),
    # The released model's row width (engram_head_dim = 256, so K = 24 * 256 = 6144) on a table of the
    # mid-prefill size: the path at the D the config block of the pages gives, beside the D = 64 above.
    6: _cfg(name="released_head_dim", index=6, batch=2, seqlen=4096, start_pos=0, vocab_size=129280,
            compressed_vocab_size=99092, n_heads=8, n_layers=1, head_dim=256, dim=5120,
            prime_base=166000, rows_alloc=(3988006,), token_dist="zipf", mask_frac=0.05),
}


# ----------------------------------------------------------------------------
# primes, offsets, multipliers (the hash's layout data)
# ----------------------------------------------------------------------------
def _is_prime(n: int) -> bool:
    if n < 2:
        return False
    small = (2, 3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37)
    for p in small:
        if n % p == 0:
            return n == p
    # deterministic Miller-Rabin for n < 3.3e24 with these bases
    d, r = n - 1, 0
    while d % 2 == 0:
        d //= 2
        r += 1
    for a in small:
        x = pow(a, d, n)
        if x in (1, n - 1):
            continue
        for _ in range(r - 1):
            x = x * x % n
            if x == n - 1:
                break
        else:
            return False
    return True


def primes_above(base: int, count: int) -> list:
    """The `count` smallest primes strictly greater than `base`, ascending."""
    out, n = [], base + 1
    while len(out) < count:
        if _is_prime(n):
            out.append(n)
        n += 1
    return out


def layout_primes(prime_base: int, n_layers: int, max_ngram_size: int, n_heads: int) -> np.ndarray:
    """primes[e, n-2, h] (int64 [E, N-1, H]).

    Consecutive distinct primes above `prime_base`, layer-outer; inside a layer
    in column order (n-gram size outer, head inner).
    """
    C = (max_ngram_size - 1) * n_heads
    flat = primes_above(prime_base, n_layers * C)
    return np.asarray(flat, dtype=np.int64).reshape(n_layers, max_ngram_size - 1, n_heads)


def layout_offsets(primes: np.ndarray) -> np.ndarray:
    """offsets[e, c]: exclusive prefix sum of layer e's primes in column order."""
    E = primes.shape[0]
    flat = primes.reshape(E, -1)
    off = np.zeros_like(flat)
    off[:, 1:] = np.cumsum(flat, axis=1)[:, :-1]
    return off


def multipliers(seed: int, n_layers: int, max_ngram_size: int, compressed_vocab_size: int,
                full_range: bool = False) -> np.ndarray:
    """multipliers[e, s] (int64 [E, N]), odd.

    Bounded (default): uniform in [1, floor((2^63-1)/Vc)] so no product of a
    compressed id with a multiplier overflows.  full_range: any odd int64,
    to exercise wrap-around and negative running values.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if full_range:
        m = rng.integers(np.iinfo(np.int64).min, np.iinfo(np.int64).max, size=(n_layers, max_ngram_size),
                         dtype=np.int64, endpoint=True)
    else:
        hi = (2**63 - 1) // compressed_vocab_size
        m = rng.integers(1, hi, size=(n_layers, max_ngram_size), dtype=np.int64, endpoint=True)
    return m | np.int64(1)


# ----------------------------------------------------------------------------
# token ids, masks, token_map
# ----------------------------------------------------------------------------
@functools.lru_cache(maxsize=8)
def _zipf_cdf(vocab: int, s: float) -> np.ndarray:
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def token_ids(seed: int, shape, vocab: int, dist: str, zipf_s: float = 1.1) -> np.ndarray:
    """int64 token ids: uniform over [0, vocab), or Zipf(s) by rank (id = rank - 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if dist == "uniform":
        return rng.integers(0, vocab, size=shape, dtype=np.int64)
    if dist == "zipf":
        u = rng.random(size=shape)
        idx = np.searchsorted(_zipf_cdf(vocab, zipf_s), u, side="right")
        return np.minimum(idx, vocab - 1).astype(np.int64)
    raise ValueError(dist)


def token_map(seed: int, vocab: int, compressed_vocab_size: int) -> np.ndarray:
    """int64 [vocab] -> [0, Vc): stands in for the tokenizer normalisation map."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, compressed_vocab_size, size=vocab, dtype=np.int64)


def mask_spans(seed: int, batch: int, seqlen: int, frac: float, min_len: int = 16,
               max_len: int = 256) -> np.ndarray:
    """uint8 [B, L] token mask: 1 = takes part in n-grams, 0 = masked (an image span).

    Per row: non-overlapping, non-touching spans of length U[min_len, max_len]
    at random starts until round(frac * L) positions are masked; the last span
    is trimmed to hit the target exactly.
    """
    m = np.ones((batch, seqlen), dtype=np.uint8)
    if frac <= 0:
        return m
    rng = np.random.Generator(np.random.PCG64(seed))
    target = int(round(frac * seqlen))
    for b in range(batch):
        count, tries = 0, 0
        while count < target:
            tries += 1
            if tries > 100000:
                raise RuntimeError("mask_spans: could not place spans")
            n = int(rng.integers(min_len, max_len, endpoint=True))
            n = min(n, target - count, seqlen)
            s = int(rng.integers(0, seqlen - n, endpoint=True))
            lo, hi = max(0, s - 1), min(seqlen, s + n + 1)
            if (m[b, lo:hi] == 0).any():
                continue
            m[b, s:s + n] = 0
            count += n
    return m


# ----------------------------------------------------------------------------
# fp8 table rows (counter-based)
# ----------------------------------------------------------------------------
def splitmix64(seed: int, n: np.ndarray) -> np.ndarray:
    """Element n of the SplitMix64 stream with the given seed (uint64)."""
    n = np.ascontiguousarray(n, dtype=np.uint64)
    flat_n = n.reshape(-1)
    out = np.empty(flat_n.shape, dtype=np.uint64)
    chunk = 1 << 16
    tmp = np.empty(chunk, dtype=np.uint64)
    s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    for lo in range(0, flat_n.size, chunk):
        z = out[lo:lo + chunk]
        t = tmp[: z.size]
        np.add(flat_n[lo:lo + chunk], np.uint64(1), out=z)
        np.multiply(z, GOLDEN_GAMMA, out=z)
        np.add(z, s, out=z)
        for shift, mul in ((30, _MIX1), (27, _MIX2)):
            np.right_shift(z, np.uint64(shift), out=t)
            np.bitwise_xor(z, t, out=z)
            np.multiply(z, mul, out=z)
        np.right_shift(z, np.uint64(31), out=t)
        np.bitwise_xor(z, t, out=z)
    return out.reshape(n.shape)


@functools.lru_cache(maxsize=1)
def normal_fp8_lut() -> np.ndarray:
    """uint8 [65536]: E4M3FN byte of the N(0,1) quantile at (i + 1/2)/65536, clipped to +-448."""
    import scipy.special
    import torch

    q = scipy.special.ndtri((np.arange(65536, dtype=np.float64) + 0.5) / 65536.0)
    q = np.clip(q, -448.0, 448.0)
    return torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def words_per_row(head_dim: int, block_size: int) -> int:
    return head_dim // 4 + head_dim // block_size


def table_rows(seed: int, rows: np.ndarray, head_dim: int, block_size: int):
    """(weight uint8 [n, D], scale float32 [n, D/blk]) of the given table rows."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    nb, ns = head_dim // 4, head_dim // block_size
    W = nb + ns
    n = rows.astype(np.uint64)[:, None] * np.uint64(W) + np.arange(W, dtype=np.uint64)[None, :]
    u = splitmix64(seed, n)
    lut = normal_fp8_lut()
    # the four 16-bit fields of word w, low field first, are its little-endian uint16 pieces 4w .. 4w+3
    idx = np.ascontiguousarray(u[:, :nb]).astype("<u8", copy=False).view("<u2")
    weight = lut[idx].reshape(rows.size, head_dim)
    us = u[:, nb:]
    mant = (us & np.uint64(0x7FFFFF)).astype(np.uint32)
    ex = ((us >> np.uint64(32)) % np.uint64(6)).astype(np.uint32)
    bits = ((np.uint32(127 - 8) + ex) << np.uint32(23)) | mant
    scale = bits.view(np.float32).reshape(rows.size, ns)
    return weight, scale


def full_table(seed: int, n_rows: int, head_dim: int, block_size: int, chunk: int = 1 << 20):
    """Whole table on the host (small tables only)."""
    w = np.empty((n_rows, head_dim), dtype=np.uint8)
    s = np.empty((n_rows, head_dim // block_size), dtype=np.float32)
    for lo in range(0, n_rows, chunk):
        hi = min(n_rows, lo + chunk)
        w[lo:hi], s[lo:hi] = table_rows(seed, np.arange(lo, hi), head_dim, block_size)
    return w, s


class SparseHostTable:
    """A host table of `n_rows` rows of which only requested rows are materialised.

    The backing arrays come from calloc'd (lazily zero-mapped) memory, so a
    384M-row table costs host RAM only for the pages of rows actually filled.
    """

    def __init__(self, seed: int, n_rows: int, head_dim: int, block_size: int):
        self.seed, self.n_rows, self.head_dim, self.block_size = seed, n_rows, head_dim, block_size
        self.weight = np.zeros((n_rows, head_dim), dtype=np.uint8)
        self.scale = np.zeros((n_rows, head_dim // block_size), dtype=np.float32)

    def fill(self, rows) -> None:
        rows = np.unique(np.asarray(rows, dtype=np.int64).reshape(-1))
        rows = rows[(rows >= 0) & (rows < self.n_rows)]
        if rows.size:
            w, s = table_rows(self.seed, rows, self.head_dim, self.block_size)
            self.weight[rows] = w
            self.scale[rows] = s


# ----------------------------------------------------------------------------
# dense operands
# ----------------------------------------------------------------------------
def bf16_normal(seed: int, shape, mean: float = 0.0, std: float = 1.0, device: str = "cpu"):
    """torch bf16 tensor ~ N(mean, std^2), drawn with torch's seeded generator on `device`."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(torch.bfloat16)


@dataclasses.dataclass
class HashInputs:
    input_ids: np.ndarray              # int64 [B, L] (or [B, start_pos + steps] for decode)
    token_mask: Optional[np.ndarray]   # uint8 [B, L] or None
    token_map: np.ndarray              # int64 [vocab]
    multipliers: np.ndarray            # int64 [E, N]
    primes: np.ndarray                 # int64 [E, N-1, H]
    offsets: np.ndarray                # int64 [E, C]


def hash_inputs(cfg: EngramConfig, full_range_multipliers: bool = False) -> HashInputs:
    """All inputs of the hash step for a workload (decode: the whole token history)."""
    L_total = cfg.start_pos + cfg.decode_steps if cfg.decode_steps else cfg.seqlen
    ids = token_ids(cfg.seed(0), (cfg.batch, L_total), cfg.vocab_size, cfg.token_dist, cfg.zipf_s)
    mask = mask_spans(cfg.seed(3), cfg.batch, L_total, cfg.mask_frac) if cfg.mask_frac > 0 else None
    tmap = token_map(cfg.seed(1), cfg.vocab_size, cfg.compressed_vocab_size)
    mult = multipliers(cfg.seed(2), cfg.n_layers, cfg.max_ngram_size, cfg.compressed_vocab_size,
                       full_range_multipliers)
    primes = layout_primes(cfg.prime_base, cfg.n_layers, cfg.max_ngram_size, cfg.n_heads)
    return HashInputs(ids, mask, tmap, mult, primes, layout_offsets(primes))


def table_seed(cfg: EngramConfig, layer: int) -> int:
    return cfg.seed(4 + layer)


def wkv_weight(cfg: EngramConfig, layer: int, device: str = "cpu"):
    """bf16 [dim*(hc+1), C*D] ~ N(0, 0.02^2)."""
    return bf16_normal(cfg.seed(6 + layer), (cfg.n_out, cfg.K), std=0.02, device=device)


def qk_weights(cfg: EngramConfig, layer: int = 0, device: str = "cpu"):
    """(q_weight, k_weight), each bf16 [hc, dim] ~ 1 + N(0, 0.1^2)."""
    q = bf16_normal(cfg.seed(8) * 16 + 2 * layer, (cfg.hc_mult, cfg.dim), mean=1.0, std=0.1, device=device)
    k = bf16_normal(cfg.seed(8) * 16 + 2 * layer + 1, (cfg.hc_mult, cfg.dim), mean=1.0, std=0.1, device=device)
    return q, k


def residual(cfg: EngramConfig, tokens: Optional[int] = None, device: str = "cpu", step: int = 0):
    """bf16 x [T, hc, dim] ~ N(0, 1) (T = B*L unless given)."""
    T = cfg.tokens if tokens is None else tokens
    return bf16_normal(cfg.seed(9) * 1024 + step, (T, cfg.hc_mult, cfg.dim), device=device)


def rows_used(primes: np.ndarray) -> list:
    """Rows each layer's hash ids can reach (sum of its primes)."""
    return [int(x) for x in primes.reshape(primes.shape[0], -1).sum(axis=1)]


def compact_table(ids: np.ndarray, n_rows: int, seed: int, head_dim: int, block_size: int):
    """The rows that `ids` reach in an `n_rows`-row seeded table, as a compact host table.

    Returns (weight [U, D], scale [U, D/blk], remapped ids): in-range ids are
    replaced by their index among the sorted distinct rows, out-of-range ids by
    -1 (still out of range for the compact table).  Lets a host consumer see
    exactly the rows of a table that only exists on the GPU.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    ok = (flat >= 0) & (flat < n_rows)
    uniq = np.unique(flat[ok])
    w, s = table_rows(seed, uniq, head_dim, block_size)
    remap = np.full(flat.shape, -1, dtype=np.int64)
    remap[ok] = np.searchsorted(uniq, flat[ok])
    return w, s, remap.reshape(np.shape(ids))


def scale_bytes(scale_f32: np.ndarray, fmt: str) -> np.ndarray:
    """The one-byte block scales of a table whose scales are stored as E8M0 or float8_e4m3fn, as a bit-level
    function of the seeded float32 scales of the same rows (exponent uniform in {-8..-3}, 23 random mantissa
    bits): E8M0 keeps the float32 exponent byte (a power of two in [2^-8, 2^-3]); E4M3 takes exponent field
    (biased exponent - 117), in 2..7, and the top three mantissa bits: the scale times 8 truncated to E4M3
    (values in [2^-5, 2))."""
    bits = np.ascontiguousarray(scale_f32, dtype=np.float32).view(np.uint32)
    e = (bits >> np.uint32(23)) & np.uint32(0xFF)
    if fmt == "e8m0":
        return e.astype(np.uint8)
    if fmt == "e4m3":
        return (((e - np.uint32(117)) << np.uint32(3)) | ((bits >> np.uint32(20)) & np.uint32(7))).astype(np.uint8)
    raise ValueError(fmt)


def table_rows_alloc(cfg: EngramConfig) -> list:
    return list(cfg.rows_alloc[: cfg.n_layers])


__all__ = [name for name in dir() if not name.startswith("_")] + ["_is_prime"]
del math
