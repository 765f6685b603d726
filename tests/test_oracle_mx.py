"""Pins for the oracle's fp8 block-scaled projection (the `wkv` Linear under the
released config's "dtype": "fp8", stack-hashes page: the config block and
Engram.__init__): OCP MX fp8 operands, E4M3FN elements in blocks of 32 columns
with one E8M0 scale each.

The E8M0 decode is checked on all 256 codes against torch's float8_e8m0fnu;
the E4M3 encoder (round to nearest even, saturating) against its own decoder
on every code, against torch's float8_e4m3fn cast, on ties and around the
saturation point; the quantisation on blocks whose result is known in closed
form (exact round trips, saturation, zero blocks, subnormal maxima) and
against an independent numpy/torch computation of the same rule; the product
on scaled identities, one-hot rows, and against the bf16 projection of the
exactly dequantised operands.
"""
import numpy as np
import pytest
import torch

import oracle


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f(bits):
    return oracle.bf16_bits_to_float(bits).astype(np.float64)


DEC8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def test_e8m0_decode_all_codes_against_torch():
    want = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.e8m0_decode(b) for b in range(256)])
    np.testing.assert_array_equal(got[:255], want[:255])
    assert np.isnan(got[255]) and np.isnan(want[255])
    assert got[127] == 1.0 and got[128] == 2.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_e4m3_encoder_round_trips_every_code():
    for b in range(256):
        if (b & 0x7F) == 0x7F:
            continue  # NaN codes
        assert oracle.e4m3fn_encode_sat(DEC8[b]) == b, hex(b)


def test_e4m3_encoder_ties_saturation_and_torch():
    enc = oracle.e4m3fn_encode_sat
    assert enc(1.0625) == 0x38 and enc(1.1875) == 0x3A  # ties to the even mantissa (1.0, 1.25)
    assert enc(2.0 ** -10) == 0x00 and enc(3 * 2.0 ** -10) == 0x02  # subnormal ties (0 and 2 * 2^-9)
    assert enc(15 * 2.0 ** -10) == 0x08  # the largest subnormal tie rounds up into the smallest normal
    assert enc(448.0) == 0x7E and enc(463.9) == 0x7E and enc(464.0) == 0x7E and enc(1e30) == 0x7E
    assert enc(-500.0) == 0xFE and enc(-0.0) == 0x80 and enc(0.0) == 0x00
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.normal(scale=60, size=4000), rng.uniform(-2.0 ** -5, 2.0 ** -5, 2000),
                        rng.uniform(-448, 448, 2000)])
    want = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([enc(x) for x in v], dtype=np.uint8)
    np.testing.assert_array_equal(got, want)


def test_mx_quant_exact_round_trip_and_scale():
    """A block built from E4M3 codes whose largest magnitude lies in [256, 448], times 2^s, quantises back to
    exactly those codes with scale byte s + 127."""
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 0x7E, size=(6, 64)).astype(np.uint8) | (rng.integers(0, 2, (6, 64)) << 7).astype(np.uint8)
    codes[:, 0] = 0x78  # 256
    codes[:, 32] = 0x7E  # 448
    codes[codes & 0x7F == 0x7F] &= 0xFE
    s = np.array([[-3, 5], [0, 0], [-20, 20], [-100, -60], [90, 60], [7, -7]])
    x = DEC8[codes] * np.exp2(np.repeat(s, 32, axis=1))
    q, sc = oracle.mx_quant(_bf16_bits(x))
    np.testing.assert_array_equal(q, codes)
    np.testing.assert_array_equal(sc, (s + 127).astype(np.uint8))


def test_mx_quant_closed_forms():
    K = 64
    x = np.zeros((5, K), np.float32)
    x[0, :] = 1.0                          # amax 1 -> exponent -8 (byte 119): elements 256 = 0x78
    x[1, 0], x[1, 1] = 480.0, -3.0         # amax 480 -> exponent 0: 480 saturates to 448
    x[1, 32] = 0.75                        # block 1: amax 0.75 -> exponent -9 (byte 118): 384 = 0x7C
    x[2, 5] = -0.0                         # all-zero block -> byte 0, -0 kept
    x[3, :32] = 2.0 ** -133                # the smallest bf16 subnormal: exponent clamped to -127
    x[4, 0], x[4, 1] = 1.0, 2.0 ** -9      # 2^-9 / 2^-8 = 0.5 -> 0x30; the rest of the block is 0
    q, sc = oracle.mx_quant(_bf16_bits(x))
    assert sc[0, 0] == 119 and (q[0, :32] == 0x78).all()
    assert sc[1, 0] == 127 and q[1, 0] == 0x7E and q[1, 1] == oracle.e4m3fn_encode_sat(-3.0) == 0xC4
    assert sc[1, 1] == 118 and q[1, 32] == 0x7C
    assert sc[2, 0] == 0 and q[2, 5] == 0x80 and (np.delete(q[2, :32], 5) == 0).all()
    assert sc[3, 0] == 0 and (q[3, :32] == oracle.e4m3fn_encode_sat(2.0 ** -6)).all()  # 2^-133 * 2^127
    assert sc[4, 0] == 119 and q[4, 0] == 0x78 and q[4, 1] == 0x30


def test_mx_quant_against_an_independent_computation():
    rng = np.random.default_rng(13)
    xb = _bf16_bits(rng.normal(size=(40, 256)) * np.exp2(rng.integers(-30, 30, size=(40, 1))))
    x = _f(xb).reshape(40, 8, 32)
    amax = np.abs(x).max(axis=-1)
    _, e = np.frexp(amax)
    shared = np.clip((e - 1) - 8, -127, 127)
    v = x / np.exp2(shared)[..., None]
    want_q = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    q, sc = oracle.mx_quant(xb)
    np.testing.assert_array_equal(sc, (shared + 127).astype(np.uint8))
    np.testing.assert_array_equal(q, want_q.reshape(40, 256))
    # the dequantised value is within half an E4M3 step of the input (relative 2^-4), except saturated elements
    deq = oracle.mx_dequant(q, sc)
    ok = np.abs(v.reshape(40, 256)) < 448
    rel = np.abs(deq - _f(xb)) / np.maximum(np.abs(_f(xb)), 1e-300)
    assert (rel[ok & (np.abs(v.reshape(40, 256)) >= 2.0 ** -6)] <= 2.0 ** -4 + 1e-12).all()


def test_wkv_mx_scaled_identity_and_one_hot():
    rng = np.random.default_rng(14)
    K = 128
    a_q = rng.integers(0, 0x7E, size=(5, K)).astype(np.uint8)
    a_s = rng.integers(100, 150, size=(5, K // 32)).astype(np.uint8)
    w_q = np.zeros((K + 32, K), np.uint8)
    w_q[np.arange(K), np.arange(K)] = 0x38  # 1.0
    w_s = np.full((K + 32, K // 32), 127, np.uint8)
    got = oracle.wkv_mx(a_q, a_s, w_q, w_s)
    a = oracle.mx_dequant(a_q, a_s)
    np.testing.assert_array_equal(got[:, :K], a)
    assert (got[:, K:] == 0).all()
    w_s[:] = 128  # the weights' scale doubles every output
    np.testing.assert_array_equal(oracle.wkv_mx(a_q, a_s, w_q, w_s)[:, :K], 2 * a)
    w_s[:, 1] = 125  # one block of columns at a quarter
    got = oracle.wkv_mx(a_q, a_s, w_q, w_s)
    np.testing.assert_array_equal(got[:, 32:64], 0.25 * a[:, 32:64])
    np.testing.assert_array_equal(got[:, :32], 2 * a[:, :32])


def test_wkv_mx_equals_the_projection_of_the_dequantised_operands():
    """On operands whose dequantised values are exact in bf16, the block-scaled product equals the bf16
    projection of those values (both accumulated in double), and the float64-matmul form agrees."""
    rng = np.random.default_rng(15)
    T, K, N = 9, 192, 70
    a_q, a_s = oracle.mx_quant(_bf16_bits(rng.normal(size=(T, K))))
    w_q, w_s = oracle.mx_quant(_bf16_bits(rng.normal(scale=0.02, size=(N, K))))
    got = oracle.wkv_mx(a_q, a_s, w_q, w_s)
    a_bits = _bf16_bits(oracle.mx_dequant(a_q, a_s))
    w_bits = _bf16_bits(oracle.mx_dequant(w_q, w_s))
    np.testing.assert_array_equal(_f(a_bits), oracle.mx_dequant(a_q, a_s))  # exact in bf16
    np.testing.assert_allclose(got, oracle.wkv(a_bits, w_bits), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(oracle.wkv_mx_matmul(a_q, a_s, w_q, w_s), got, rtol=1e-12, atol=1e-300)
