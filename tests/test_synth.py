"""The seeded input generators: determinism, distributions and the
counter-based table generator's definition."""
import numpy as np
import torch

import synth


def test_splitmix64_reference_vector():
    # the first outputs of SplitMix64 seeded with 1234567 (Vigna's reference generator)
    got = synth.splitmix64(1234567, np.arange(3)).tolist()
    assert got[0] == 6457827717110365317
    assert got == [0x599ED017FB08FC85, 0x2C73F08458540FA5, 0x883EBCE5A3F27C77]


def test_table_rows_are_counter_based():
    rows = np.array([0, 5, 123456789, 384006167], dtype=np.int64)
    w, s = synth.table_rows(3004, rows, 64, 32)
    w2, s2 = synth.table_rows(3004, rows[::-1], 64, 32)
    np.testing.assert_array_equal(w, w2[::-1])
    np.testing.assert_array_equal(s, s2[::-1])
    # one row on its own is the same as inside a batch
    w1, s1 = synth.table_rows(3004, rows[2:3], 64, 32)
    np.testing.assert_array_equal(w1[0], w[2])
    # layout of the words: byte 4w+i of a row is LUT[16-bit field i of word w]
    W = synth.words_per_row(64, 32)
    u = synth.splitmix64(3004, np.uint64(5) * np.uint64(W) + np.arange(W, dtype=np.uint64))
    lut = synth.normal_fp8_lut()
    assert w[1, 4 * 3 + 2] == lut[(int(u[3]) >> 32) & 0xFFFF]
    bits = s[1].view(np.uint32)
    assert (bits & 0x7FFFFF).tolist() == [int(x) & 0x7FFFFF for x in u[16:18]]
    assert ((bits >> 23).astype(np.int64) - 127).tolist() == [-8 + ((int(x) >> 32) % 6) for x in u[16:18]]


def test_table_value_distribution():
    w, s = synth.table_rows(1, np.arange(20000), 64, 32)
    v = torch.from_numpy(w).view(torch.float8_e4m3fn).float().numpy()
    assert np.isfinite(v).all()
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1.0) < 0.02
    assert s.min() >= 2.0**-8 and s.max() < 2.0**-2
    e = np.floor(np.log2(s))
    counts = np.array([(e == k).sum() for k in range(-8, -2)])
    assert counts.min() > 0.9 * counts.mean()


def test_lut_is_monotone_quantiles():
    lut = synth.normal_fp8_lut()
    v = torch.from_numpy(lut.copy()).view(torch.float8_e4m3fn).float().numpy()
    assert (np.diff(v) >= 0).all()
    np.testing.assert_array_equal(v, -v[::-1])
    assert v[0] < -3.5 and v[-1] > 3.5


def test_zipf_and_uniform_ids():
    ids = synth.token_ids(7, (200000,), 129280, "zipf", 1.1)
    assert ids.min() >= 0 and ids.max() < 129280
    top1 = (ids == 0).mean()
    assert abs(top1 - 0.133) < 0.005  # P(rank 1) of Zipf(1.1) over 129280 ids
    u = synth.token_ids(7, (200000,), 129280, "uniform")
    assert abs(u.mean() / 129280 - 0.5) < 0.01


def test_mask_spans_hit_the_fraction_exactly():
    m = synth.mask_spans(2003, 4, 2048, 0.10)
    assert ((m == 0).sum(axis=1) == 205).all()
    for row in m:
        z = np.flatnonzero(np.diff(np.concatenate([[1], row, [1]]).astype(int)))
        lengths = z[1::2] - z[0::2]
        assert lengths.max() <= 256 and (lengths >= 1).all()
        assert (lengths >= 16).sum() >= len(lengths) - 1  # only the trimmed last span may be short


def test_configs_are_consistent():
    for c in synth.CONFIGS.values():
        primes = synth.layout_primes(c.prime_base, c.n_layers, c.max_ngram_size, c.n_heads)
        used = synth.rows_used(primes)
        assert all(u <= a for u, a in zip(used, c.rows_alloc))
        assert c.head_dim % c.block_size == 0
        assert c.n_out == c.dim * 5 and c.K == c.n_hash_cols * c.head_dim
    assert synth.CONFIGS[3].K == 1536 and synth.CONFIGS[3].n_out == 25600


def test_scale_bytes_definition():
    """The one-byte scale stand-ins: E8M0 is the float32 scale's exponent byte, E4M3 the scale times 8 truncated
    to three mantissa bits (a normal code in [2^-5, 2))."""
    import torch

    w, s = synth.table_rows(123, np.arange(5000), 64, 16)
    e8 = synth.scale_bytes(s, "e8m0")
    np.testing.assert_array_equal(torch.from_numpy(e8).view(torch.float8_e8m0fnu).float().numpy(),
                                  np.exp2(np.floor(np.log2(s))))
    e4 = synth.scale_bytes(s, "e4m3")
    v = torch.from_numpy(e4).view(torch.float8_e4m3fn).float().numpy()
    assert (v >= 2.0 ** -5).all() and (v < 2.0).all()
    # the scale times 8, truncated to three mantissa bits
    x = s.astype(np.float64) * 8
    q = np.exp2(np.floor(np.log2(x)) - 3)
    np.testing.assert_array_equal(v, np.floor(x / q) * q)
