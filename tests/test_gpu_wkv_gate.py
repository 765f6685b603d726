"""engram_wkv and engram_gate_dot on the GPU against the oracle (tolerance
|got - want| <= 1e-3 + 2e-2 |want|), on ragged shapes and at workload sizes."""
import math

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_close, bits

pytestmark = pytest.mark.gpu


def _rand_bf16(rng, shape, std=1.0):
    import torch

    return torch.from_numpy((rng.normal(size=shape) * std).astype(np.float32)).to(torch.bfloat16)


# 128-token tiles where they fit the CUs in one pass (64, 257, 513, 256 and 130 tokens here; 130 leaves a
# 2-row second tile), 256-token tiles above (2600, 1000); K not a multiple of 64 takes the staged kernel
@pytest.mark.parametrize("T,K,N", [(64, 192, 1280), (1, 8, 8), (300, 200, 264), (257, 1536, 520), (513, 64, 256),
                                   (256, 1536, 25600), (130, 1536, 25600), (2600, 1536, 6400), (1000, 1536, 25600)])
def test_wkv_ragged_shapes(gpu_device, T, K, N):
    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(T + K + N)
    a = _rand_bf16(rng, (T, K), 0.1)
    w = _rand_bf16(rng, (N, K), 0.02)
    kv = g.engram_wkv(a.to(gpu_device), w.to(gpu_device))
    rows = np.arange(T) if T <= 600 else np.unique(np.r_[0, 255, 256, 511, 512, T - 1, rng.integers(0, T, 100)])
    want = oracle.wkv(bits(a)[rows], bits(w))
    got = oracle.bf16_bits_to_float(bits(kv)[rows])
    assert_close(got, want, what=f"wkv T={T} K={K} N={N}")


def test_wkv_identity_is_exact(gpu_device):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(7)
    T, K = 300, 192
    a = _rand_bf16(rng, (T, K))
    w = torch.zeros((K + 64, K), dtype=torch.bfloat16)
    w[:K] = torch.eye(K, dtype=torch.bfloat16)
    kv = g.engram_wkv(a.to(gpu_device), w.to(gpu_device))
    np.testing.assert_array_equal(bits(kv)[:, :K], bits(a))
    assert (bits(kv)[:, K:] == 0).all()


def test_wkv_zero_tokens(gpu_device):
    import torch

    import gram_hash_embedding_amd as g

    a = torch.zeros((0, 64), dtype=torch.bfloat16, device=gpu_device)
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device=gpu_device)
    assert g.engram_wkv(a, w).shape == (0, 64)


@pytest.mark.parametrize("T,hc,dim,extra", [(5, 4, 256, 0), (3, 7, 520, 8), (17, 1, 8, 0), (64, 4, 5120, 5120),
                                            (2, 64, 16, 0)])
def test_gate_shapes(gpu_device, T, hc, dim, extra):
    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(T * hc + dim)
    x = _rand_bf16(rng, (T, hc, dim))
    kv = _rand_bf16(rng, (T, hc * dim + extra))
    q = _rand_bf16(rng, (hc, dim), 0.1) + 1
    k = _rand_bf16(rng, (hc, dim), 0.1) + 1
    dot = g.engram_gate_dot(x.to(gpu_device), kv.to(gpu_device), q.to(gpu_device), k.to(gpu_device), 1e-20)
    want = oracle.gate_dot(bits(x), bits(kv), bits(q), bits(k), 1e-20)
    assert_close(dot.cpu().numpy(), want, what="gate")


def test_gate_closed_forms_on_gpu(gpu_device):
    import torch

    import gram_hash_embedding_amd as g

    dim, hc = 5120, 4
    rng = np.random.default_rng(3)
    h = _rand_bf16(rng, (1, hc, dim))
    key = h.clone()
    key[0, 1] = -h[0, 1]
    key[0, 3] = 0
    kv = torch.cat([key.reshape(1, -1), torch.ones((1, dim), dtype=torch.bfloat16)], dim=1)
    ones = torch.ones((hc, dim), dtype=torch.bfloat16, device=gpu_device)
    dot = g.engram_gate_dot(h.to(gpu_device), kv.to(gpu_device), ones, ones, 1e-20).cpu().numpy()
    assert dot[0, 0] == pytest.approx(math.sqrt(dim), rel=1e-4)
    assert dot[0, 1] == pytest.approx(-math.sqrt(dim), rel=1e-4)
    assert dot[0, 2] == pytest.approx(math.sqrt(dim), rel=1e-4)
    assert dot[0, 3] == 0.0


def test_gate_on_gpu_kv_full_config2(gpu_device):
    """Unit check of the gate at config-2 shape: the oracle reads the GPU's own bf16 kv."""
    import gram_hash_embedding_amd as g

    cfg = synth.CONFIGS[2]
    rng = np.random.default_rng(2)
    T = 2048
    x = synth.residual(cfg, tokens=T)
    kv = _rand_bf16(rng, (T, cfg.n_out), 0.08)
    q, k = synth.qk_weights(cfg)
    dot = g.engram_gate_dot(x.to(gpu_device), kv.to(gpu_device), q.to(gpu_device), k.to(gpu_device), cfg.eps)
    want = oracle.gate_dot(bits(x), bits(kv), bits(q), bits(k), cfg.eps)
    assert_close(dot.cpu().numpy(), want, what="gate cfg2")
