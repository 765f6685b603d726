"""The bf16 projection's 16 x 16 x 32 form (wkv16.hip), which engram_wkv and engram_wkv_gate launch for
256-token tiles with three or more 64-column slabs when every launch has at least two waves of tiles: shapes
chosen to take it -- ragged token counts (a last tile of 1 to 255 rows), a ragged last column tile, the
smallest K (three slabs) and long K, one and many copies, dims up to 8,192 -- against the oracle (the bf16
bar), the fused form's value columns bit for bit against the plain launch's, its dot against the unfused
path (fp32 summation order only) and against the oracle fed the device's keys (the tight bar),
run-to-run identity, and a row-strided value output."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import assert_close, bits

pytestmark = pytest.mark.gpu


def _rand_bf16(rng, shape, std=1.0, mean=0.0):
    import torch

    return torch.from_numpy((rng.normal(size=shape) * std + mean).astype(np.float32)).to(torch.bfloat16)


def _rows(rng, T):
    return np.unique(np.r_[0, 1, 255, 256, 511, 512, T - 2, T - 1, rng.integers(0, T, 90)])


# (T, K, N): 9 x 65 tiles with an 8-column last one, 12 x 50, 32 x 16 at K = 6,144, 16 x 32 at an odd slab
# count (25)
@pytest.mark.parametrize("T,K,N", [(2049, 192, 16392), (3000, 1536, 12800), (8191, 6144, 4096), (4096, 1600, 8192)])
def test_wkv16_plain_matches_the_oracle(gpu_device, T, K, N):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(T + 3 * K + 7 * N)
    a = _rand_bf16(rng, (T, K), 0.1).to(gpu_device)
    w = _rand_bf16(rng, (N, K), 0.02).to(gpu_device)
    kv = g.engram_wkv(a, w)
    kv2 = g.engram_wkv(a, w)
    torch.cuda.synchronize()
    assert torch.equal(kv, kv2), "run to run"
    rows = _rows(rng, T)
    want = oracle.wkv(bits(a[torch.from_numpy(rows).to(gpu_device)]), bits(w))
    assert_close(oracle.bf16_bits_to_float(bits(kv)[rows]), want, what=f"wkv16 T={T} K={K} N={N}")


def _kv_bf16(kv64):
    import torch

    return torch.from_numpy(kv64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# (T, K, hc, dim): 33 x 16 value tiles at K = 192 (a 1-row last tile), the workload's layout at a ragged 9,000
# tokens, two copies of dim 8,192, an odd slab count (25) with a ragged last tile, and 12 x 20 value tiles (under
# one wave: the fused launch follows the plain one's choice of kernel, taken on all 12 x 100 tiles)
@pytest.mark.parametrize("T,K,hc,dim", [(8193, 192, 1, 4096), (9000, 1536, 4, 5120), (16384, 384, 2, 8192),
                                        (8300, 1600, 2, 4096), (3000, 1536, 4, 5120)])
def test_wkv16_gate_matches_the_plain_launch_and_the_oracle(gpu_device, T, K, hc, dim):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(T + K + 100 * hc + dim)
    a = _rand_bf16(rng, (T, K), 0.1).to(gpu_device)
    w = _rand_bf16(rng, ((hc + 1) * dim, K), 0.02).to(gpu_device)
    x = _rand_bf16(rng, (T, hc, dim)).to(gpu_device)
    q = _rand_bf16(rng, (hc, dim), 0.1, 1.0).to(gpu_device)
    k = _rand_bf16(rng, (hc, dim), 0.1, 1.0).to(gpu_device)
    value, dot = g.engram_wkv_gate(a, w, x, q, k, 1e-20)
    v2, d2 = g.engram_wkv_gate(a, w, x, q, k, 1e-20)
    kv = g.engram_wkv(a, w)
    dot_unfused = g.engram_gate_dot(x, kv, q, k, 1e-20)
    torch.cuda.synchronize()
    assert torch.equal(value, v2) and torch.equal(dot, d2), "run to run"
    np.testing.assert_array_equal(bits(value), bits(kv)[:, hc * dim:], err_msg="value columns")
    assert_close(dot.cpu().numpy(), dot_unfused.cpu().numpy(), rtol=1e-3, atol=1e-4, what="dot vs unfused")
    rows = _rows(rng, T)
    sel = torch.from_numpy(rows).to(gpu_device)
    x_bits, kv_bits = bits(x[sel]), bits(kv[sel])
    assert_close(dot.cpu().numpy()[rows], oracle.gate_dot(x_bits, kv_bits, bits(q), bits(k), 1e-20), rtol=1e-3,
                 atol=1e-4, what="dot vs the oracle's gate on the device's keys")
    kv_want = oracle.wkv(bits(a[sel]), bits(w))
    assert_close(oracle.bf16_bits_to_float(kv_bits), kv_want, what="kv vs oracle")
    assert_close(dot.cpu().numpy()[rows], oracle.gate_dot(x_bits, _kv_bf16(kv_want), bits(q), bits(k), 1e-20),
                 what="dot vs oracle")


def test_wkv16_gate_strided_value_leaves_the_padding(gpu_device):
    """The fused launch's value columns into a row-strided view (ld = dim + 384): equal to the plain launch's
    bit for bit, and the columns past dim in each row untouched."""
    import torch

    import gram_hash_embedding_amd as g

    T, K, hc, dim, ld = 4099, 768, 2, 8192, 8192 + 384
    rng = np.random.default_rng(41)
    a = _rand_bf16(rng, (T, K), 0.1).to(gpu_device)
    w = _rand_bf16(rng, ((hc + 1) * dim, K), 0.02).to(gpu_device)
    x = _rand_bf16(rng, (T, hc, dim)).to(gpu_device)
    q = _rand_bf16(rng, (hc, dim), 0.1, 1.0).to(gpu_device)
    k = _rand_bf16(rng, (hc, dim), 0.1, 1.0).to(gpu_device)
    buf = torch.full((T, ld), 7.0, dtype=torch.bfloat16, device=gpu_device)
    _, dot = g.engram_wkv_gate(a, w, x, q, k, 1e-20, value=buf[:, :dim])
    kv = g.engram_wkv(a, w)
    dot2 = g.engram_gate_dot(x, kv, q, k, 1e-20)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(buf[:, :dim]), bits(kv)[:, hc * dim:], err_msg="value columns")
    assert bool((buf[:, dim:] == 7.0).all()), "padding columns written"
    assert_close(dot.cpu().numpy(), dot2.cpu().numpy(), rtol=1e-3, atol=1e-4, what="dot vs unfused")
