"""engram_gate_output on the GPU against the oracle: the dot within the gate
tolerance, the output stream within bf16 rounding of the oracle's output
taken from the GPU's own dot, masked tokens bit-exact, on ragged shapes,
every register-tile variant, and closed forms of the gate."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import assert_close, bits

pytestmark = pytest.mark.gpu


def _rand_bf16(rng, shape, std=1.0):
    import torch

    return torch.from_numpy((rng.normal(size=shape) * std).astype(np.float32)).to(torch.bfloat16)


def _f(b):
    return oracle.bf16_bits_to_float(b).astype(np.float64)


# (T, hc, dim, extra kv columns, masked): dim / 512 rounds up to 1, 2, 4, 6, 8, 10, 12 and 16 pieces per lane.
# Launches of fewer than 1,024 (token group, copy) waves with 2048 <= dim <= 6144 split each row over a
# workgroup (the small-T cases at dims 3000-6144 below); the larger T at those dims keep one wave per row.
SHAPES = [(5, 4, 256, 0, False), (3, 7, 520, 8, True), (17, 1, 8, 0, False), (2, 64, 16, 0, True),
          (9, 3, 1024, 0, True), (11, 2, 3000, 16, False), (6, 4, 4096, 0, True), (64, 4, 5120, 5120, True),
          (7, 2, 6144, 0, True), (3, 2, 8192, 8, False), (1, 4, 5120, 0, False),
          (1100, 2, 3000, 16, False), (520, 4, 4096, 0, True), (1030, 2, 6144, 0, True)]


@pytest.mark.parametrize("T,hc,dim,extra,masked", SHAPES)
def test_gate_output_shapes(gpu_device, T, hc, dim, extra, masked):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(T * 131 + hc * 7 + dim)
    x = _rand_bf16(rng, (T, hc, dim))
    kv = _rand_bf16(rng, (T, (hc + 1) * dim + extra), 0.5)
    q = _rand_bf16(rng, (hc, dim), 0.1) + 1
    k = _rand_bf16(rng, (hc, dim), 0.1) + 1
    mask = torch.from_numpy(rng.random(T) < 0.6) if masked else None
    dot = torch.full((T, hc), float("nan"), dtype=torch.float32, device=gpu_device)
    out = g.engram_gate_output(x.to(gpu_device), kv.to(gpu_device), q.to(gpu_device), k.to(gpu_device), 1e-20,
                               None if mask is None else mask.to(gpu_device), dot=dot)
    xb, kvb = bits(x), bits(kv)
    dot_want = oracle.gate_dot(xb, kvb, bits(q), bits(k), 1e-20)
    dot_got = dot.cpu().numpy()
    assert_close(dot_got, dot_want, what="dot")
    m = None if mask is None else mask.numpy().astype(np.uint8)
    ob = bits(out)
    # unit check: the oracle's gate and residual from the GPU's own dot -> bf16 rounding apart
    _, out_unit = oracle.gate_output(xb, kvb, dot_got.astype(np.float64), m)
    assert_close(_f(ob), out_unit, rtol=2.0 ** -8, atol=1e-6, what="out (gpu dot)")
    # end to end: from the oracle's dot
    _, out_want = oracle.gate_output(xb, kvb, dot_want, m)
    assert_close(_f(ob), out_want, what="out")
    if m is not None:
        np.testing.assert_array_equal(ob[m == 0], xb[m == 0])


def test_gate_output_without_dot_and_with_bool_mask_matches(gpu_device):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(11)
    T, hc, dim = 33, 4, 640
    x = _rand_bf16(rng, (T, hc, dim)).to(gpu_device)
    kv = _rand_bf16(rng, (T, (hc + 1) * dim), 0.5).to(gpu_device)
    q = (_rand_bf16(rng, (hc, dim), 0.1) + 1).to(gpu_device)
    k = (_rand_bf16(rng, (hc, dim), 0.1) + 1).to(gpu_device)
    mask = torch.from_numpy(rng.random(T) < 0.5).to(gpu_device)
    dot = torch.empty((T, hc), dtype=torch.float32, device=gpu_device)
    a = g.engram_gate_output(x, kv, q, k, 1e-20, mask.to(torch.uint8), dot=dot)
    b = g.engram_gate_output(x, kv, q, k, 1e-20, mask)
    np.testing.assert_array_equal(bits(a), bits(b))
    # the dot it reports is the one engram_gate_dot computes (same sums, same order)
    assert_close(dot.cpu().numpy(), g.engram_gate_dot(x, kv, q, k, 1e-20).cpu().numpy(), rtol=1e-5, atol=1e-6,
                 what="dot vs engram_gate_dot")
    # [B, L, hc, dim] input with a [B, L] mask is the same call
    c = g.engram_gate_output(x.view(3, 11, hc, dim), kv, q, k, 1e-20, mask.view(3, 11))
    assert c.shape == (3, 11, hc, dim)
    np.testing.assert_array_equal(bits(c).reshape(T, hc, dim), bits(a))


def test_gate_output_closed_forms_on_gpu(gpu_device):
    """dim 256, w = 1: key = h -> dot 16 -> gate sigmoid(4); key = -h -> sigmoid(-4); key = 0 -> dot +0 ->
    gate sigmoid(1e-3) = 0.50025, which with h = -0.5 and value 1 leaves 0.00025 (bf16 0x3983), where an
    unclamped gate of exactly 0.5 would give 0; a masked token passes x through bit for bit."""
    import torch

    import gram_hash_embedding_amd as g

    dim, hc = 256, 4
    rng = np.random.default_rng(4)
    h = _rand_bf16(rng, (2, hc, dim))
    h[:, 2] = -0.5
    key = h.clone()
    key[:, 1] = -h[:, 1]
    key[:, 2] = 0
    value = torch.ones((2, dim), dtype=torch.bfloat16)
    value[:, 1::2] = -2.0
    kv = torch.cat([key.reshape(2, -1), value], dim=1)
    ones = torch.ones((hc, dim), dtype=torch.bfloat16, device=gpu_device)
    mask = torch.tensor([True, False], device=gpu_device)
    dot = torch.empty((2, hc), dtype=torch.float32, device=gpu_device)
    out = g.engram_gate_output(h.to(gpu_device), kv.to(gpu_device), ones, ones, 1e-20, mask, dot=dot)
    d = dot.cpu().numpy()
    assert d[0, 0] == pytest.approx(16.0, rel=1e-5) and d[0, 1] == pytest.approx(-16.0, rel=1e-5)
    assert d[0, 2] == 0.0 and not np.signbit(d[0, 2])
    ob = bits(out)
    s4, s_4 = 0.9820137900379084, 0.01798620996209156
    v = _f(bits(value))[0]
    hf = _f(bits(h))
    assert_close(_f(ob[0, 0]), hf[0, 0] + s4 * v, rtol=2.0 ** -8, atol=1e-6, what="gate sigmoid(4)")
    assert_close(_f(ob[0, 1]), hf[0, 1] + s_4 * v, rtol=2.0 ** -8, atol=1e-6, what="gate sigmoid(-4)")
    assert (ob[0, 2, 0::2] == 0x3983).all()  # -0.5 + 0.50025 * 1 = 0.00025 -> bf16 0x3983
    np.testing.assert_array_equal(ob[1], bits(h)[1])


def test_gate_output_zero_tokens(gpu_device):
    import torch

    import gram_hash_embedding_amd as g

    x = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device=gpu_device)
    kv = torch.zeros((0, 320), dtype=torch.bfloat16, device=gpu_device)
    w = torch.ones((4, 64), dtype=torch.bfloat16, device=gpu_device)
    assert g.engram_gate_output(x, kv, w, w, 1e-20).shape == (0, 4, 64)
