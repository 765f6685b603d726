"""Pins for the oracle's wkv projection and gate pre-activation (DeepSeek V4.1
pages, stack-hashes page: Engram.__init__ / Engram.forward up to `dot`).

wkv is a plain matrix product: checked against numpy's float64 matmul and on
operands whose product is known.  The gate dot is checked on hand-built
vectors with closed-form results.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_f64(b):
    return oracle.bf16_bits_to_float(b).astype(np.float64)


def test_wkv_matches_numpy_matmul():
    rng = np.random.default_rng(1)
    a = _bf16_bits(rng.normal(size=(37, 96)))
    w = _bf16_bits(rng.normal(scale=0.02, size=(130, 96)))
    got = oracle.wkv(a, w)
    want = _bits_to_f64(a) @ _bits_to_f64(w).T
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_wkv_identity_and_one_hot():
    rng = np.random.default_rng(2)
    K = 64
    a = _bf16_bits(rng.normal(size=(9, K)))
    eye = np.zeros((K + 16, K), dtype=np.float32)
    eye[:K] = np.eye(K)
    got = oracle.wkv(a, _bf16_bits(eye))
    np.testing.assert_array_equal(got[:, :K], _bits_to_f64(a))
    assert (got[:, K:] == 0).all()
    # one-hot row of A selects a column of W^T (a row of W)
    w = _bf16_bits(rng.normal(size=(20, K)))
    onehot = np.zeros((3, K), dtype=np.float32)
    onehot[0, 5], onehot[1, 0], onehot[2, K - 1] = 1.0, 2.0, -1.0
    got = oracle.wkv(_bf16_bits(onehot), w)
    wf = _bits_to_f64(w)
    np.testing.assert_array_equal(got[0], wf[:, 5])
    np.testing.assert_array_equal(got[1], 2 * wf[:, 0])
    np.testing.assert_array_equal(got[2], -wf[:, K - 1])


def test_wkv_matmul_closed_forms_and_the_c_loop():
    """The library-contraction form of the projection (used for whole-workload parity) on the same closed
    forms as the C loop, and equal to it on random operands up to float64 summation order."""
    rng = np.random.default_rng(5)
    K = 96
    a = _bf16_bits(rng.normal(size=(11, K)))
    eye = np.zeros((K + 8, K), dtype=np.float32)
    eye[:K] = np.eye(K)
    got = oracle.wkv_matmul(a, _bf16_bits(eye), chunk=4)
    np.testing.assert_array_equal(got[:, :K], _bits_to_f64(a))
    assert (got[:, K:] == 0).all()
    w = _bf16_bits(rng.normal(size=(20, K)))
    onehot = np.zeros((2, K), dtype=np.float32)
    onehot[0, 7], onehot[1, K - 1] = -4.0, 0.5
    got = oracle.wkv_matmul(_bf16_bits(onehot), w)
    np.testing.assert_array_equal(got[0], -4 * _bits_to_f64(w)[:, 7])
    np.testing.assert_array_equal(got[1], 0.5 * _bits_to_f64(w)[:, K - 1])
    # a row of ones sums each W row (integers: exact in any order)
    wi = _bf16_bits(rng.integers(-100, 100, size=(13, K)).astype(np.float32))
    got = oracle.wkv_matmul(_bf16_bits(np.ones((1, K), np.float32)), wi)
    np.testing.assert_array_equal(got[0], _bits_to_f64(wi).sum(axis=1))
    a = _bf16_bits(rng.normal(size=(70, 256)))
    w = _bf16_bits(rng.normal(scale=0.02, size=(300, 256)))
    np.testing.assert_allclose(oracle.wkv_matmul(a, w, chunk=16), oracle.wkv(a, w), rtol=1e-12, atol=1e-14)


def _gate(x, key, q=None, k=None, eps=1e-20):
    T, hc, dim = x.shape
    if q is None:
        q = np.ones((hc, dim), np.float32)
    if k is None:
        k = np.ones((hc, dim), np.float32)
    kv = np.zeros((T, hc * dim + 7), dtype=np.float32)  # trailing value columns are ignored
    kv[:, : hc * dim] = key.reshape(T, hc * dim)
    kv[:, hc * dim:] = 99.0
    return oracle.gate_dot(_bf16_bits(x), _bf16_bits(kv), _bf16_bits(q), _bf16_bits(k), eps)


@pytest.mark.parametrize("dim", [256, 5120])
def test_gate_closed_forms(dim):
    rng = np.random.default_rng(dim)
    hc = 4
    h = rng.normal(size=(1, hc, dim)).astype(np.float32)
    h = oracle.bf16_bits_to_float(_bf16_bits(h)).reshape(1, hc, dim)
    # copy 0: key = h -> sqrt(dim); copy 1: key = -h -> -sqrt(dim);
    # copy 2: key orthogonal to h -> 0; copy 3: key = 0 -> 0
    key = np.empty_like(h)
    key[0, 0] = h[0, 0]
    key[0, 1] = -h[0, 1]
    key[0, 2] = 0
    key[0, 2, 0], key[0, 2, 1] = h[0, 2, 1], -h[0, 2, 0]
    ortho_h = np.zeros(dim, np.float32)
    ortho_h[0], ortho_h[1] = h[0, 2, 0], h[0, 2, 1]
    hh = h.copy()
    hh[0, 2] = ortho_h
    key[0, 3] = 0
    got = _gate(hh, key)
    assert got[0, 0] == pytest.approx(math.sqrt(dim), rel=1e-12)
    assert got[0, 1] == pytest.approx(-math.sqrt(dim), rel=1e-12)
    assert got[0, 2] == 0.0
    assert got[0, 3] == 0.0


def test_gate_is_sqrt_dim_times_cosine():
    # with w = 1 and eps negligible, rstd * dim^-1/2 turns the dot into sqrt(dim) * cos(h, key)
    rng = np.random.default_rng(3)
    T, hc, dim = 5, 4, 256
    h = oracle.bf16_bits_to_float(_bf16_bits(rng.normal(size=(T, hc, dim)))).reshape(T, hc, dim).astype(np.float64)
    key = oracle.bf16_bits_to_float(_bf16_bits(rng.normal(size=(T, hc, dim)))).reshape(T, hc, dim).astype(np.float64)
    got = _gate(h, key)
    cos = (h * key).sum(-1) / (np.linalg.norm(h, axis=-1) * np.linalg.norm(key, axis=-1))
    np.testing.assert_allclose(got, math.sqrt(dim) * cos, rtol=1e-10)


def test_gate_weight_product_scales_and_normalisation_is_per_copy():
    rng = np.random.default_rng(4)
    T, hc, dim = 3, 4, 256
    h = rng.normal(size=(T, hc, dim)).astype(np.float32)
    key = rng.normal(size=(T, hc, dim)).astype(np.float32)
    base = _gate(h, key)
    # q*k = 2 on copy 1 only (q = 4, k = 0.5): that copy's dot doubles
    q = np.ones((hc, dim), np.float32)
    k = np.ones((hc, dim), np.float32)
    q[1], k[1] = 4.0, 0.5
    got = _gate(h, key, q, k)
    np.testing.assert_allclose(got[:, 1], 2 * base[:, 1], rtol=1e-12)
    np.testing.assert_array_equal(got[:, [0, 2, 3]], base[:, [0, 2, 3]])
    # scaling one copy's stream or key (by powers of two, exact in bf16) changes no dot
    h2, key2 = h.copy(), key.copy()
    h2[:, 0] *= 8.0
    key2[:, 3] *= 0.25
    np.testing.assert_allclose(_gate(h2, key2), base, rtol=1e-12)
    # permuting the copies permutes the dots
    perm = [2, 0, 3, 1]
    np.testing.assert_array_equal(_gate(h[:, perm], key[:, perm]), base[:, perm])


def test_gate_eps_only_matters_for_tiny_rows():
    h = np.zeros((1, 4, 256), np.float32)
    key = np.zeros((1, 4, 256), np.float32)
    h[0, :, 0] = 1.0
    key[0, :, 0] = 1.0
    got = _gate(h, key, eps=1e-20)
    assert got[0, 0] == pytest.approx(16.0, rel=1e-12)
    # with eps = 1 the rows' mean squares (1/256) are swamped: dot = 1 / (1/256 + 1) / 16
    got = _gate(h, key, eps=1.0)
    assert got[0, 0] == pytest.approx(1.0 / (1.0 / 256 + 1.0) / 16.0, rel=1e-12)
