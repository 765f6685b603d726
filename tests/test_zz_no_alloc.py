"""engram_wkv_gate_layers_noalloc (the fused projection + gate pre-activation
with the library's own device scratch, for callers that cannot allocate)
against engram_wkv_gate_layers with a caller workspace: the same kernels and
launch shape, so the value columns and the dots agree bit for bit.  Two calls
in a row, the second smaller than the first (the scratch keeps the first
call's partial sums, which the second must not see), each also against the
oracle within the gate tolerance on sampled tokens."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import assert_close, bits

pytestmark = pytest.mark.gpu


def _rand_bf16(rng, shape, std=1.0, mean=0.0):
    import torch

    return torch.from_numpy((rng.normal(size=shape) * std + mean).astype(np.float32)).to(torch.bfloat16)


def _layers(rng, E, T, K, hc, dim, dev):
    mk = lambda shape, std=1.0, mean=0.0: [_rand_bf16(rng, shape, std, mean).to(dev) for _ in range(E)]
    return (mk((T, K), 0.1), mk(((hc + 1) * dim, K), 0.02), mk((T, hc, dim)), mk((hc, dim), 0.1, 1.0),
            mk((hc, dim), 0.1, 1.0))


def _kv_bf16(kv64):
    import torch

    return torch.from_numpy(kv64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _call_both(g, torch, dev, ops, T, hc, dim):
    a, w, x, q, k = ops
    E = len(a)
    val_n = [torch.full((T, dim), 3.0, dtype=torch.bfloat16, device=dev) for _ in range(E)]
    dot_n = [torch.full((T, hc), 7.0, dtype=torch.float32, device=dev) for _ in range(E)]
    g.engram_wkv_gate_layers_noalloc(a, w, x, q, k, 1e-20, val_n, dot_n)
    torch.cuda.synchronize()
    val_w, dot_w = g.engram_wkv_gate_layers(a, w, x, q, k, 1e-20)
    torch.cuda.synchronize()
    return val_n, dot_n, val_w, dot_w


@pytest.mark.parametrize("first,second", [
    ((2, 4096, 1536, 4, 5120), (2, 256, 1536, 4, 5120)),   # a long call, then a decode step of both layers
    ((3, 700, 256, 2, 512), (1, 33, 128, 3, 256)),          # another shape altogether, fewer layers
])
def test_noalloc_matches_the_workspace_entry_point(gpu_device, first, second):
    import torch

    import gram_hash_embedding_amd as g

    for call, (E, T, K, hc, dim) in enumerate((first, second)):
        assert E * g.engram_wkv_gate_workspace_bytes(T, hc, dim) <= g.NOALLOC_SCRATCH_BYTES
        rng = np.random.default_rng(1000 * call + T + K + hc + dim)
        ops = _layers(rng, E, T, K, hc, dim, gpu_device)
        val_n, dot_n, val_w, dot_w = _call_both(g, torch, gpu_device, ops, T, hc, dim)
        rows = np.unique(np.r_[0, T - 1, rng.integers(0, T, min(T, 48))])
        for e in range(E):
            np.testing.assert_array_equal(bits(val_n[e]), bits(val_w[e]), err_msg=f"call {call}, layer {e}: value")
            np.testing.assert_array_equal(dot_n[e].cpu().numpy().view(np.uint32), dot_w[e].cpu().numpy().view(np.uint32),
                                          err_msg=f"call {call}, layer {e}: dot")
            a, w, x, q, k = (t[e] for t in ops)
            kv_want = oracle.wkv_matmul(bits(a)[rows], bits(w))
            dot_want = oracle.gate_dot(bits(x)[rows], _kv_bf16(kv_want), bits(q), bits(k), 1e-20)
            assert_close(dot_n[e].cpu().numpy()[rows], dot_want, what=f"call {call}, layer {e}: dot vs oracle")


def test_noalloc_rejects_more_than_its_scratch(gpu_device):
    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(5)
    E, T, K, hc, dim = 2, 4370, 64, 4, 5120
    ops = _layers(rng, E, T, K, hc, dim, gpu_device)
    import torch

    val = [torch.empty((T, dim), dtype=torch.bfloat16, device=gpu_device) for _ in range(E)]
    dot = [torch.empty((T, hc), dtype=torch.float32, device=gpu_device) for _ in range(E)]
    with pytest.raises(g.EngramError, match="scratch"):
        g.engram_wkv_gate_layers_noalloc(*ops, 1e-20, val, dot)
