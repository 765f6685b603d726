"""Pins for the oracle's gather and block dequant (DeepSeek V4.1 pages,
stack-hashes page: ParallelEngramEmbedding.forward).

The fp8 decode is checked against torch's float8_e4m3fn for all 256 bytes,
the bf16 rounding against torch's cast, and the whole dequant (fp32 product,
then bf16) against torch's casts and numpy's fp32 multiply.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _torch_dequant(wbytes, scales, blk):
    v = torch.from_numpy(np.ascontiguousarray(wbytes)).view(torch.float8_e4m3fn).float()
    s = torch.from_numpy(np.ascontiguousarray(scales)).float()
    shp = v.shape
    v = (v.reshape(*shp[:-1], -1, blk) * s.unsqueeze(-1)).reshape(shp)
    return v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_e4m3fn_decode_all_bytes_match_torch():
    want = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3fn_decode(b) for b in range(256)], dtype=np.float32)
    nan = np.isnan(want)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))  # -0 included


def test_e4m3fn_is_not_fnuz():
    assert oracle.e4m3fn_decode(0x38) == 1.0
    assert oracle.e4m3fn_decode(0x7E) == 448.0
    assert oracle.e4m3fn_decode(0x01) == 2.0**-9
    assert np.float32(oracle.e4m3fn_decode(0x80)).view(np.uint32) == 0x80000000


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2**32, size=4000, dtype=np.uint64).astype(np.uint32)
    # ties and near-ties at both parities, both signs, denormals, max finite
    special = np.array([0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0xBF808000, 0xBF818000,
                        0x00008000, 0x00018000, 0x7F7FFFFF, 0x7F7F8000, 0x80000000, 0x00000000], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne(f)
    np.testing.assert_array_equal(got, want)


def test_two_roundings_regression_vector():
    # 0xED (-104) times a scale whose fp32 product sits just above a bf16 tie:
    # rounding to fp32 first lands exactly on the tie, which then goes to even.
    scale = np.array([0x3D8713B1], dtype=np.uint32).view(np.float32)
    prod32 = np.float32(-104.0) * scale[0]
    assert prod32.view(np.uint32) == 0xC0DB8000
    w = np.full((1, 32), 0xED, dtype=np.uint8)
    s = scale.reshape(1, 1)
    out = oracle.gather_dequant(np.zeros((1, 1), np.int64), w, s, block_size=32)
    assert out[0, 0, 0] == 0xC0DC
    # a single rounding of the exact product would have given 0xC0DB
    exact = -104.0 * float(scale[0])  # exact in double (7-bit times 24-bit significand)
    assert -6.859375 < exact < -6.84375  # between bf16 0xC0DB (-6.84375) and the tie point
    np.testing.assert_array_equal(out[0, 0], _torch_dequant(w, s, 32)[0])


def test_simple_vector():
    w = np.full((1, 32), 0x38, dtype=np.uint8)
    s = np.array([[0.125]], dtype=np.float32)
    out = oracle.gather_dequant(np.zeros((1, 1), np.int64), w, s, block_size=32)
    assert (out == 0x3E00).all()


def test_dequant_matches_torch_on_random_rows():
    w, s = synth.table_rows(77, np.arange(3000), 64, 32)
    # add every byte value, both zero signs and the NaN codes into the rows
    w[0, :] = np.arange(64)
    w[1, :] = np.arange(64, 128)
    w[2, :] = np.arange(128, 192)
    w[3, :] = np.arange(192, 256)
    ids = np.arange(3000, dtype=np.int64).reshape(-1, 6)
    got = oracle.gather_dequant(ids, w, s, block_size=32)
    want = _torch_dequant(w, s, 32).reshape(got.shape)
    gf, wf = oracle.bf16_bits_to_float(got), oracle.bf16_bits_to_float(want)
    np.testing.assert_array_equal(np.isnan(gf), np.isnan(wf))
    ok = ~np.isnan(wf)
    np.testing.assert_array_equal(got[ok], want[ok])


@pytest.mark.parametrize("D,blk", [(32, 32), (64, 32), (128, 32), (64, 16), (256, 128)])
def test_gather_copies_rows_and_zeroes_out_of_range(D, blk):
    R, row_start = 500, 100
    w, s = synth.table_rows(5, np.arange(R), D, blk)
    rng = np.random.default_rng(D + blk)
    ids = rng.integers(row_start - 50, row_start + R + 50, size=(40, 7), dtype=np.int64)
    ids[0, 0], ids[0, 1], ids[0, 2] = -(2**62), 2**62, row_start + R  # far out and the first past the end
    C = 5  # only the first 5 of 7 columns are this layer's
    out, raw, rsc = oracle.gather_dequant(ids, w, s, row_start=row_start, block_size=blk, n_cols=C, want_raw=True)
    used = ids[:, :C]
    bad = (used < row_start) | (used >= row_start + R)
    local = np.where(bad, 0, used - row_start)
    np.testing.assert_array_equal(raw, w[local])
    np.testing.assert_array_equal(rsc.view(np.uint32), s[local].view(np.uint32))
    assert bad.sum() >= 3
    assert (out[bad] == 0).all()
    want = _torch_dequant(w[local], s[local], blk)
    np.testing.assert_array_equal(out[~bad], want[~bad])


def test_negative_zero_survives():
    w = np.zeros((2, 32), dtype=np.uint8)
    w[1, :] = 0x80
    s = np.array([[0.5], [0.5]], dtype=np.float32)
    out = oracle.gather_dequant(np.array([[0, 1]], np.int64), w, s, block_size=32)
    assert (out[0, 0] == 0x0000).all() and (out[0, 1] == 0x8000).all()
