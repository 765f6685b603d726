"""Pins for the oracle's gate activation, mask and residual (DeepSeek V4.1
pages, stack-hashes page: the end of Engram.forward, after `dot`).

The gate is the sigmoid of the signed square root of the dot, with |dot|
clamped from below at 1e-6; a masked token's gate is 0; the output adds the
gated value (one per token, shared by the hc copies) to every copy of the
stream.  Expected gates are sigmoid values computed to 40 digits with Python's
decimal module (1 / (1 + exp(-z))), independent of the oracle's C library.
"""
import numpy as np
import pytest
import torch

import oracle

# sigmoid(z) to double precision, from decimal arithmetic at 40 digits
SIG = {
    "0.001": 0.5002499999791666687499997891865292934283,
    "-0.001": 0.4997500000208333312500002108134707065718,
    "2": 0.8807970779778824440597291413023967952061,
    "-3": 0.04742587317756678087884815177175220138617,
    "4": 0.9820137900379084419732068620504615751274,
    "-4": 0.01798620996209155802679313794953842487249,
    "sqrt2": 0.8044296825069569051929726070005621025987,
}


def _bits(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f64(b):
    return oracle.bf16_bits_to_float(b).astype(np.float64)


def _run(x, value, dot, mask=None):
    """x [T,hc,dim], value [T,dim] floats (bf16-exact), dot [T,hc] -> gate, out"""
    T, hc, dim = x.shape
    kv = np.full((T, (hc + 1) * dim + 8), 99.0, dtype=np.float32)  # key columns and padding must be ignored
    kv[:, hc * dim:(hc + 1) * dim] = value
    return oracle.gate_output(_bits(x), _bits(kv), np.asarray(dot, dtype=np.float64), mask)


def test_gate_of_zero_and_tiny_dots_is_clamped_and_keeps_the_sign():
    dots = np.array([[0.0, -0.0, 1e-9, -1e-9, 1e-6, -1e-6]])
    gate, _ = _run(np.zeros((1, 6, 8)), np.zeros((1, 8)), dots)
    want = [SIG["0.001"], SIG["-0.001"], SIG["0.001"], SIG["-0.001"], SIG["0.001"], SIG["-0.001"]]
    np.testing.assert_allclose(gate[0], want, rtol=0, atol=1e-15)


def test_gate_takes_the_signed_square_root_before_the_sigmoid():
    # sqrt(4) = 2, -sqrt(9) = -3, +-sqrt(16) = +-4; a sigmoid of the raw dot would give 0.982, 1.2e-4, ...
    gate, _ = _run(np.zeros((1, 4, 8)), np.zeros((1, 8)), [[4.0, -9.0, 16.0, -16.0]])
    np.testing.assert_allclose(gate[0], [SIG["2"], SIG["-3"], SIG["4"], SIG["-4"]], rtol=0, atol=1e-15)


def test_gate_symmetry_and_range():
    rng = np.random.default_rng(5)
    d = rng.normal(scale=20.0, size=(50, 4))
    g_pos, _ = _run(np.zeros((50, 4, 8)), np.zeros((50, 8)), d)
    g_neg, _ = _run(np.zeros((50, 4, 8)), np.zeros((50, 8)), -d)
    np.testing.assert_allclose(g_pos + g_neg, 1.0, rtol=0, atol=1e-15)
    assert ((g_pos > 0) & (g_pos < 1)).all()
    order = np.argsort(d.ravel())
    assert (np.diff(g_pos.ravel()[order]) >= 0).all()  # monotone in the dot


def test_worked_example_through_the_dot():
    # copy 0: h = key = 1 (dim 4, w = 1) -> dot = 4 * 4^-1/2 = 2 -> gate = sigmoid(sqrt 2)
    # copy 1: h = (1,-1,1,-1) is orthogonal to key = 1 -> dot = 0 -> gate = sigmoid(1e-3)
    x = np.array([[[1, 1, 1, 1], [1, -1, 1, -1]]], dtype=np.float32)
    key = np.ones((1, 2, 4), dtype=np.float32)
    value = np.array([[1.0, -1.0, 0.5, 2.0]], dtype=np.float32)
    kv = np.concatenate([key.reshape(1, 8), value], axis=1)
    dot = oracle.gate_dot(_bits(x), _bits(kv), _bits(np.ones((2, 4))), _bits(np.ones((2, 4))), 1e-20)
    np.testing.assert_allclose(dot, [[2.0, 0.0]], rtol=0, atol=1e-15)
    gate, out = oracle.gate_output(_bits(x), _bits(kv), dot)
    g0, g1 = SIG["sqrt2"], SIG["0.001"]
    np.testing.assert_allclose(gate, [[g0, g1]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 0], [1 + g0, 1 - g0, 1 + 0.5 * g0, 1 + 2 * g0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 1], [1 + g1, -1 - g1, 1 + 0.5 * g1, -1 + 2 * g1], rtol=0, atol=1e-15)


def test_value_is_shared_by_the_copies_and_scaled_by_each_gate():
    rng = np.random.default_rng(6)
    T, hc, dim = 7, 3, 16
    x = _f64(_bits(rng.normal(size=(T, hc, dim))))
    value = _f64(_bits(rng.normal(size=(T, dim)) + 3.0))  # bounded away from zero
    dot = rng.normal(scale=3.0, size=(T, hc))
    gate, out = _run(x, value, dot)
    ratio = (out - x) / value[:, None, :]
    np.testing.assert_allclose(ratio, np.repeat(gate[:, :, None], dim, axis=2), rtol=1e-12, atol=0)


def test_masked_tokens_pass_through_untouched():
    rng = np.random.default_rng(7)
    T, hc, dim = 6, 4, 8
    x = _f64(_bits(rng.normal(size=(T, hc, dim))))
    value = _f64(_bits(rng.normal(size=(T, dim))))
    mask = np.array([1, 0, 1, 0, 0, 1], dtype=np.uint8)
    gate, out = _run(x, value, rng.normal(size=(T, hc)), mask)
    assert (gate[mask == 0] == 0).all() and (gate[mask == 1] > 0).all()
    np.testing.assert_array_equal(out[mask == 0], x[mask == 0])
    # a zero value leaves every token's stream as it was, whatever the gate
    _, out0 = _run(x, np.zeros((T, dim)), rng.normal(size=(T, hc)))
    np.testing.assert_array_equal(out0, x)


@pytest.mark.parametrize("v, want_sign", [(1.5, 0.0), (-1.5, -0.0)])
def test_masked_negative_zero_follows_ieee_addition(v, want_sign):
    # gate 0: out = -0 + (+0 * v); +0 * v is +0 for v > 0 (sum +0) and -0 for v < 0 (sum -0)
    x = np.full((1, 1, 8), -0.0, dtype=np.float32)
    _, out = _run(x, np.full((1, 8), v), [[5.0]], np.array([0], dtype=np.uint8))
    assert (out == 0).all()
    assert (np.signbit(out) == np.signbit(want_sign)).all()


def test_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.gate_output(np.zeros((2, 2, 8), np.uint16), np.zeros((2, 24), np.uint16), np.zeros((2, 3)))
    with pytest.raises(oracle.OracleError):  # kv too narrow to hold the value columns
        oracle.gate_output(np.zeros((2, 2, 8), np.uint16), np.zeros((2, 16), np.uint16), np.zeros((2, 2)))
