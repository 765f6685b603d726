"""Pins for the oracle's gather + dequant with the table's block scales in the
one-byte formats the page's `scale_dtype` may name (stack-hashes page,
ParallelEngramEmbedding: `scales.float()`, then the fp32 product and bf16) --
E8M0 (the pages' indexer format, block 32) and float8_e4m3fn (the pages'
compressed-KV format, block 16) -- and with int32 ids.

Each format is checked against torch's own decode of the scale dtype and its
fp32 product and bf16 cast; the float32 format against the original oracle
function bit for bit; closed forms (unit scales, NaN scales, zero rows for ids
outside the share) and int32 ids against int64 ids.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _torch_dequant(w_rows, s_rows, fmt, blk):
    wf = torch.from_numpy(w_rows).view(torch.float8_e4m3fn).float()
    if fmt == "fp32":
        sf = torch.from_numpy(s_rows)
    elif fmt == "e8m0":
        sf = torch.from_numpy(s_rows).view(torch.float8_e8m0fnu).float()
    else:
        sf = torch.from_numpy(s_rows).view(torch.float8_e4m3fn).float()
    prod = wf.unflatten(-1, (-1, blk)) * sf.unsqueeze(-1)
    return prod.flatten(-2).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fmt,blk,D", [("e8m0", 32, 64), ("e4m3", 16, 64), ("e8m0", 32, 256), ("e4m3", 16, 32),
                                       ("fp32", 32, 64)])
def test_formats_against_torch(fmt, blk, D):
    rng = np.random.default_rng(D + blk)
    R, T, C = 500, 40, 7
    w, s32 = synth.table_rows(77 + D, np.arange(R), D, blk)
    if fmt == "e8m0":
        s = rng.integers(1, 255, size=(R, D // blk)).astype(np.uint8)  # every finite code
    elif fmt == "e4m3":
        s = rng.integers(0, 0x7F, size=(R, D // blk)).astype(np.uint8)  # every finite non-negative code
    else:
        s = s32
    ids = rng.integers(0, R, size=(T, C))
    out = oracle.gather_dequant_fmt(ids, w, s, fmt, block_size=blk)
    want = _torch_dequant(w[ids.reshape(-1)], s[ids.reshape(-1)], fmt, blk).reshape(T, C, D)
    nan_g = (out & 0x7FFF) > 0x7F80
    nan_w = (want & 0x7FFF) > 0x7F80
    np.testing.assert_array_equal(nan_g, nan_w)
    np.testing.assert_array_equal(out[~nan_g], want[~nan_w])


def test_fp32_format_equals_the_original_gather():
    rng = np.random.default_rng(3)
    R, D, blk = 999, 64, 32
    w, s = synth.table_rows(5, np.arange(R), D, blk)
    ids = rng.integers(-20, R + 20, size=(50, 11))
    for rs in (0, 7):
        got = oracle.gather_dequant_fmt(ids, w, s, "fp32", row_start=rs, block_size=blk, n_cols=9, want_raw=True)
        want = oracle.gather_dequant(ids, w, s, row_start=rs, block_size=blk, n_cols=9, want_raw=True)
        for g, o in zip(got, want):
            np.testing.assert_array_equal(g, o)


def test_closed_forms_and_int32_ids():
    R, D = 300, 64
    w, _ = synth.table_rows(9, np.arange(R), D, 32)
    plain = torch.from_numpy(w).view(torch.float8_e4m3fn).float().to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ids = np.arange(R).reshape(R, 1)
    # unit scales: E8M0 127 and E4M3 0x38 are 1.0, so the rows are the plain bf16 of their fp8 values
    one8 = np.full((R, 2), 127, np.uint8)
    np.testing.assert_array_equal(oracle.gather_dequant_fmt(ids, w, one8, "e8m0", block_size=32)[:, 0], plain)
    one4 = np.full((R, 4), 0x38, np.uint8)
    np.testing.assert_array_equal(oracle.gather_dequant_fmt(ids, w, one4, "e4m3", block_size=16)[:, 0], plain)
    # E8M0 128 doubles every value (exact), 0xFF is NaN
    two = np.full((R, 2), 128, np.uint8)
    two[3, 1] = 0xFF
    out = oracle.gather_dequant_fmt(ids, w, two, "e8m0", block_size=32)[:, 0]
    dbl = oracle.bf16_bits_to_float(plain) * 2
    assert np.isnan(oracle.bf16_bits_to_float(out[3, 32:])).all()
    keep = np.ones_like(out, dtype=bool)
    keep[3, 32:] = False
    np.testing.assert_array_equal(oracle.bf16_bits_to_float(out)[keep], dbl[keep])
    # ids outside the share give zero rows even with NaN scales; int32 ids equal int64 ids
    rng = np.random.default_rng(4)
    ids64 = rng.integers(-5, R + 5, size=(60, 8))
    for fmt, sc, blk in (("e8m0", two, 32), ("e4m3", one4, 16)):
        a = oracle.gather_dequant_fmt(ids64, w, sc, fmt, block_size=blk, row_start=5, want_raw=True)
        b = oracle.gather_dequant_fmt(ids64.astype(np.int32), w, sc, fmt, block_size=blk, row_start=5, want_raw=True)
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)
        out_of = (ids64 < 5) | (ids64 >= R + 5)
        assert (a[0][out_of] == 0).all()
