"""engram_wkv_gate (the projection and the gate pre-activation in one pass,
keys never stored) and engram_gate_residual on the GPU.

The fused value columns are the same arithmetic as engram_wkv's (bit-exact);
the fused dot matches engram_gate_dot on engram_wkv's keys up to the order of
the fp32 sums, and the oracle's pipeline within the gate tolerance; the
residual from a dot is bit-exact against engram_gate_output's, and within
bf16 rounding of the oracle's output."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import assert_close, bits

pytestmark = pytest.mark.gpu


def _rand_bf16(rng, shape, std=1.0, mean=0.0):
    import torch

    return torch.from_numpy((rng.normal(size=shape) * std + mean).astype(np.float32)).to(torch.bfloat16)


def _kv_bf16(kv64):
    import torch

    return torch.from_numpy(kv64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _inputs(rng, T, K, hc, dim, dev):
    a = _rand_bf16(rng, (T, K), 0.1).to(dev)
    w = _rand_bf16(rng, ((hc + 1) * dim, K), 0.02).to(dev)
    x = _rand_bf16(rng, (T, hc, dim)).to(dev)
    q = _rand_bf16(rng, (hc, dim), 0.1, 1.0).to(dev)
    k = _rand_bf16(rng, (hc, dim), 0.1, 1.0).to(dev)
    return a, w, x, q, k


# (T, K, hc, dim): ragged token counts (tails of 44, 1, 1, 232 rows), one-copy and many-copy layouts,
# the workload's dim with its 100 column tiles, and grids of 288 and 720 tiles, so that CUs run several
# tiles back to back (key after key, key after value, value after key).  Launches whose 128-token tiles
# fit the 256 CUs in one pass use those (all but the last three here); the decode step's 256 tokens
# (200 tiles of 128 x 256) and a ragged 200 are on that side, 300 tokens of the same layer (3 x 100
# tiles would not fit) on the other.
SHAPES = [(64, 192, 1, 256), (300, 128, 2, 256), (257, 1536, 4, 512), (513, 64, 3, 768), (1, 64, 1, 256),
          (256, 1536, 4, 5120), (200, 1536, 4, 5120), (300, 1536, 4, 5120),
          (1000, 1536, 4, 5120), (6000, 192, 3, 768), (9000, 64, 4, 1024)]


@pytest.mark.parametrize("T,K,hc,dim", SHAPES)
def test_wkv_gate_matches_the_unfused_path_and_the_oracle(gpu_device, T, K, hc, dim):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(T * 7 + K + hc * 1000 + dim)
    a, w, x, q, k = _inputs(rng, T, K, hc, dim, gpu_device)
    value, dot = g.engram_wkv_gate(a, w, x, q, k, 1e-20)
    kv = g.engram_wkv(a, w)
    dot_unfused = g.engram_gate_dot(x, kv, q, k, 1e-20)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(value), bits(kv)[:, hc * dim:], err_msg="value columns")
    assert_close(dot.cpu().numpy(), dot_unfused.cpu().numpy(), rtol=1e-3, atol=1e-4, what="dot vs unfused")
    rows = np.arange(T) if T <= 300 else np.unique(np.r_[0, 255, 256, 511, 512, T - 1, rng.integers(0, T, 60)])
    kv_want = oracle.wkv(bits(a)[rows], bits(w))
    assert_close(oracle.bf16_bits_to_float(bits(value)[rows]), kv_want[:, hc * dim:], what="value vs oracle")
    dot_want = oracle.gate_dot(bits(x)[rows], _kv_bf16(kv_want), bits(q), bits(k), 1e-20)
    assert_close(dot.cpu().numpy()[rows], dot_want, what="dot vs oracle")


def test_wkv_gate_strided_value_deterministic_and_workspace_checked(gpu_device):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(21)
    T, K, hc, dim = 300, 256, 2, 512
    a, w, x, q, k = _inputs(rng, T, K, hc, dim, gpu_device)
    wide = torch.full((T, dim + 64), 7.0, dtype=torch.bfloat16, device=gpu_device)
    value, dot = g.engram_wkv_gate(a, w, x, q, k, 1e-20, value=wide[:, 32:32 + dim])
    v2, dot2 = g.engram_wkv_gate(a, w, x, q, k, 1e-20)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(wide[:, 32:32 + dim]), bits(v2))
    assert (bits(wide[:, :32]) == bits(torch.tensor([7.0], dtype=torch.bfloat16))[0]).all()
    assert (bits(wide[:, 32 + dim:]) == bits(torch.tensor([7.0], dtype=torch.bfloat16))[0]).all()
    np.testing.assert_array_equal(dot.cpu().numpy().view(np.uint32), dot2.cpu().numpy().view(np.uint32))
    small = torch.empty(g.engram_wkv_gate_workspace_bytes(T, hc, dim) - 16, dtype=torch.uint8, device=gpu_device)
    with pytest.raises(g.EngramError, match="workspace"):
        g.engram_wkv_gate(a, w, x, q, k, 1e-20, workspace=small)


def test_wkv_gate_zero_tokens(gpu_device):
    import torch

    import gram_hash_embedding_amd as g

    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device=gpu_device)
    value, dot = g.engram_wkv_gate(z(0, 64), z(512, 64), z(0, 1, 256), z(1, 256), z(1, 256), 1e-20)
    assert value.shape == (0, 256) and dot.shape == (0, 1)


@pytest.mark.parametrize("T,hc,dim,masked", [(5, 4, 256, False), (33, 4, 5120, True), (7, 3, 520, True),
                                             (1, 1, 8, False)])
def test_gate_residual_matches_gate_output_bit_for_bit(gpu_device, T, hc, dim, masked):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(T + hc + dim)
    x = _rand_bf16(rng, (T, hc, dim)).to(gpu_device)
    kv = _rand_bf16(rng, (T, (hc + 1) * dim), 0.5).to(gpu_device)
    q = _rand_bf16(rng, (hc, dim), 0.1, 1.0).to(gpu_device)
    k = _rand_bf16(rng, (hc, dim), 0.1, 1.0).to(gpu_device)
    mask = torch.from_numpy(rng.random(T) < 0.6).to(gpu_device) if masked else None
    dot = torch.empty((T, hc), dtype=torch.float32, device=gpu_device)
    want = g.engram_gate_output(x, kv, q, k, 1e-20, mask, dot=dot)
    got = g.engram_gate_residual(x, kv[:, hc * dim:], dot, mask)
    np.testing.assert_array_equal(bits(got), bits(want))
    m = None if mask is None else mask.cpu().numpy().astype(np.uint8)
    _, out_unit = oracle.gate_output(bits(x), bits(kv), dot.cpu().numpy().astype(np.float64), m)
    assert_close(oracle.bf16_bits_to_float(bits(got)), out_unit, rtol=2.0 ** -8, atol=1e-6, what="residual")
    # in place: out is x
    x2 = x.clone()
    g.engram_gate_residual(x2, kv[:, hc * dim:], dot, mask, out=x2)
    np.testing.assert_array_equal(bits(x2), bits(want))


# (E, T, K, hc, dim): the decode step's two layers (one launch of 2 x 100 tiles of 256 tokens, where one layer
# alone takes 200 tiles of 128), a ragged token count, three layers whose 128-token tiles still fit the CUs
# together, and layers of several tiles per CU.  On 256-token tiles with K a multiple of 64 of at least three
# slabs (the first two, the fourth and the last two) the layers' key and value tiles share one launch of the
# 16 x 16 x 32 kernel: two to eight layers, ragged last tiles, one to several tiles per workgroup.
LAYER_SHAPES = [(2, 256, 1536, 4, 5120), (2, 130, 1536, 4, 5120), (3, 200, 256, 2, 512), (2, 700, 192, 3, 768),
                (4, 64, 64, 1, 256), (8, 40, 256, 1, 256), (3, 1000, 192, 2, 512), (8, 300, 192, 1, 256)]


@pytest.mark.parametrize("E,T,K,hc,dim", LAYER_SHAPES)
def test_wkv_gate_layers_matches_per_layer_calls_and_the_oracle(gpu_device, E, T, K, hc, dim):
    """engram_wkv_gate_layers: every layer's value columns bit for bit as engram_wkv_gate's (the same MFMA
    sums over K), its dot within the fp32 summation-order tolerance of engram_wkv_gate's, and both against
    the oracle on sampled tokens."""
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(E * 1000 + T + K + hc + dim)
    ins = [_inputs(rng, T, K, hc, dim, gpu_device) for _ in range(E)]
    values, dots = g.engram_wkv_gate_layers([i[0] for i in ins], [i[1] for i in ins], [i[2] for i in ins],
                                            [i[3] for i in ins], [i[4] for i in ins], 1e-20)
    singles = [g.engram_wkv_gate(*i, 1e-20) for i in ins]
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 256 else np.unique(np.r_[0, 127, 128, 255, 256, T - 1, rng.integers(0, T, 40)])
    for e, (a, w, x, q, k) in enumerate(ins):
        np.testing.assert_array_equal(bits(values[e]), bits(singles[e][0]), err_msg=f"layer {e} value")
        assert_close(dots[e].cpu().numpy(), singles[e][1].cpu().numpy(), rtol=1e-3, atol=1e-4, what=f"layer {e} dot")
        kv_want = oracle.wkv(bits(a)[rows], bits(w))
        dot_want = oracle.gate_dot(bits(x)[rows], _kv_bf16(kv_want), bits(q), bits(k), 1e-20)
        assert_close(dots[e].cpu().numpy()[rows], dot_want, what=f"layer {e} dot vs oracle")


def test_wkv_gate_layers_workspace_and_layer_count_checked(gpu_device):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(3)
    T, K, hc, dim = 40, 64, 1, 256
    ins = [_inputs(rng, T, K, hc, dim, gpu_device) for _ in range(2)]
    cols = [[i[j] for i in ins] for j in range(5)]
    small = torch.empty(2 * g.engram_wkv_gate_workspace_bytes(T, hc, dim) - 16, dtype=torch.uint8, device=gpu_device)
    with pytest.raises(g.EngramError, match="workspace"):
        g.engram_wkv_gate_layers(*cols, 1e-20, workspace=small)
    with pytest.raises(g.EngramError, match="layers=9"):
        g.engram_wkv_gate_layers(*[[c[0]] * 9 for c in cols], 1e-20)


@pytest.mark.parametrize("K", [128, 192])
def test_wkv_gate_layers_strided_values(gpu_device, K):
    """Row-strided value views (one stride for all layers): only each view's dim columns are written (K = 192:
    the layers' key and value tiles in one 16 x 16 x 32 launch)."""
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(17 + K)
    E, T, hc, dim = 3, 150, 2, 256
    ins = [_inputs(rng, T, K, hc, dim, gpu_device) for _ in range(E)]
    wide = torch.full((E, T, dim + 48), 3.0, dtype=torch.bfloat16, device=gpu_device)
    views = [wide[e, :, 16:16 + dim] for e in range(E)]
    values, dots = g.engram_wkv_gate_layers([i[0] for i in ins], [i[1] for i in ins], [i[2] for i in ins],
                                            [i[3] for i in ins], [i[4] for i in ins], 1e-20, value=views)
    torch.cuda.synchronize()
    three = bits(torch.tensor([3.0], dtype=torch.bfloat16))[0]
    for e in range(E):
        v1, d1 = g.engram_wkv_gate(*ins[e], 1e-20)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(wide[e, :, 16:16 + dim]), bits(v1), err_msg=f"layer {e}")
        assert (bits(wide[e, :, :16]) == three).all() and (bits(wide[e, :, 16 + dim:]) == three).all()
        assert_close(dots[e].cpu().numpy(), d1.cpu().numpy(), rtol=1e-3, atol=1e-4, what=f"layer {e} dot")
