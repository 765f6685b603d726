"""The fp8 block-scaled (OCP MX) form of the `wkv` Linear on the GPU (released
config's "dtype": "fp8", stack-hashes page), against the oracle:
engram_mx_quant bit for bit (elements and E8M0 scales, in the library's scale
layout); engram_wkv_mx within the projection's bar on ragged shapes, on
extreme scales, and at the workloads' shapes on sampled tokens."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_close, bf16_tensor, bits, compact_rows, mx_scales_rowmajor, sample_tokens

pytestmark = pytest.mark.gpu


_scales_rowmajor = mx_scales_rowmajor


def _scales_tiled(scale_rowmajor, K, device):
    import torch

    rows = scale_rowmajor.shape[0]
    rows4 = (rows + 3) // 4 * 4
    t = np.zeros((rows4, K // 32), np.uint8)
    t[:rows] = scale_rowmajor
    t = np.ascontiguousarray(t.reshape(rows4, K // 128, 4).transpose(1, 0, 2))
    return torch.from_numpy(t).to(device)


def _assert_close_cancelling(kv, a_q, a_s, w_q, w_s, what, kv_bits=None):
    """The projection's bar plus an allowance for operands whose products cancel: the fp8 matrix core sums its
    products more coarsely than IEEE fp32 -- measured on gfx950, |error| <= 2^-13.3 * sum_k |a_k w_k| on uniform
    E4M3 codes of both signs (2^-19.3 on quantised normal rows), about three times the fp32 recursive-summation
    bound K * 2^-24 -- so each output may also differ by 2^-12 times the sum of its products' magnitudes."""
    mag = np.abs(oracle.mx_dequant(a_q, a_s)) @ np.abs(oracle.mx_dequant(w_q, w_s)).T
    want = oracle.wkv_mx_matmul(a_q, a_s, w_q, w_s)
    assert_close(oracle.bf16_bits_to_float(bits(kv) if kv_bits is None else kv_bits), want,
                 atol=1e-3 + 2.0 ** -12 * mag, what=what)
    return want


def _bf16_rows(rng, rows, K, spread=30):
    x = rng.normal(size=(rows, K)) * np.exp2(rng.integers(-spread, spread, size=(rows, 1)))
    return x.astype(np.float32)


@pytest.mark.parametrize("rows,K", [(1, 128), (5, 256), (257, 1536), (1000, 6144), (3, 384)])
def test_mx_quant_matches_the_oracle(gpu_device, rows, K):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(rows * 7 + K)
    x = _bf16_rows(rng, rows, K)
    if rows >= 3:
        x[0, :32] = 0.0                       # an all-zero block
        x[0, 5] = -0.0
        x[1, 32:64] = 480.0 * 2.0 ** -20      # a saturating block
        x[1, 40] = -3.0 * 2.0 ** -20
        x[2, :32] = 2.0 ** -133               # the smallest bf16 subnormal
        x[2, 64:96] = rng.normal(size=32) * 2.0 ** 120
    xb = torch.from_numpy(x).to(torch.bfloat16)
    x_bits = xb.view(torch.int16).numpy().view(np.uint16)
    q, sc = g.engram_mx_quant(xb.to(gpu_device))
    torch.cuda.synchronize()
    want_q, want_s = oracle.mx_quant(x_bits)
    np.testing.assert_array_equal(q.cpu().numpy(), want_q)
    np.testing.assert_array_equal(_scales_rowmajor(sc, rows, K), want_s)


# K < 384: the streaming kernel; K >= 384: the held-back one (one token, ragged T and N, several tiles per
# workgroup in both)
@pytest.mark.parametrize("T,K,N", [(1, 128, 8), (37, 256, 264), (255, 128, 256), (257, 1536, 1280),
                                   (600, 384, 520), (1000, 1536, 25600), (4173, 1536, 2048), (300, 6144, 512),
                                   (1, 384, 8), (3, 512, 264), (700, 256, 25600)])
def test_wkv_mx_matches_the_oracle(gpu_device, T, K, N):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(T + K * 3 + N * 7)
    a_bits = bits(torch.from_numpy(_bf16_rows(rng, T, K, spread=4)).to(torch.bfloat16))
    w_bits = bits(torch.from_numpy((rng.normal(size=(N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16))
    a_q, a_s = oracle.mx_quant(a_bits)
    w_q, w_s = oracle.mx_quant(w_bits)
    kv = g.engram_wkv_mx(torch.from_numpy(a_q).to(gpu_device), _scales_tiled(a_s, K, gpu_device),
                         torch.from_numpy(w_q).to(gpu_device), _scales_tiled(w_s, K, gpu_device))
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 1000 else np.unique(np.r_[0, 255, 256, T - 1, rng.integers(0, T, 300)])
    want = oracle.wkv_mx_matmul(a_q[rows], a_s[rows], w_q, w_s)
    assert_close(oracle.bf16_bits_to_float(bits(kv)[rows]), want, what=f"wkv_mx {T}x{K}x{N}")


def test_wkv_mx_extreme_scales_and_the_quantiser_chain(gpu_device):
    """Scales near both ends of the E8M0 range (products still in fp32 range), and the device quantiser feeding
    the device projection: equal to the oracle's chain."""
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(99)
    T, K, N = 300, 512, 768
    a_q = rng.integers(0, 0x7E, size=(T, K)).astype(np.uint8) | (rng.integers(0, 2, (T, K)) << 7).astype(np.uint8)
    w_q = rng.integers(0, 0x7E, size=(N, K)).astype(np.uint8) | (rng.integers(0, 2, (N, K)) << 7).astype(np.uint8)
    # per block b: every token's scale 2^(c_b - 127) with c_b up to 2^60 away from 1, every weight row's
    # 2^(254 - c_b + d - 127), |d| <= 8: the operands' scales span 2^-60 .. 2^60, their products 2^-8 .. 2^8
    c = rng.integers(127 - 60, 127 + 60, size=K // 32)
    a_s = np.repeat(c[None, :], T, axis=0).astype(np.uint8)
    w_s = (254 - c[None, :] + rng.integers(-8, 9, size=(N, K // 32))).astype(np.uint8)
    kv = g.engram_wkv_mx(torch.from_numpy(a_q).to(gpu_device), _scales_tiled(a_s, K, gpu_device),
                         torch.from_numpy(w_q).to(gpu_device), _scales_tiled(w_s, K, gpu_device))
    torch.cuda.synchronize()
    _assert_close_cancelling(kv, a_q, a_s, w_q, w_s, "wkv_mx codes")
    # the chain: bf16 rows -> device quantiser -> device projection
    x = torch.from_numpy(_bf16_rows(rng, T, K, spread=10)).to(torch.bfloat16)
    wb = torch.from_numpy((rng.normal(size=(N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    aq, asc = g.engram_mx_quant(x.to(gpu_device))
    wq, wsc = g.engram_mx_quant(wb.to(gpu_device))
    kv = g.engram_wkv_mx(aq, asc, wq, wsc)
    torch.cuda.synchronize()
    oa_q, oa_s = oracle.mx_quant(bits(x))
    ow_q, ow_s = oracle.mx_quant(bits(wb))
    np.testing.assert_array_equal(aq.cpu().numpy(), oa_q)
    np.testing.assert_array_equal(_scales_rowmajor(asc, T, K), oa_s)
    _assert_close_cancelling(kv, oa_q, oa_s, ow_q, ow_s, "chain")


@pytest.mark.parametrize("cfg_index,n_sample", [(2, 8192), (3, 4096)])
def test_fp8_pipeline(gpu_device, cfg_index, n_sample):
    """The fp8 path at workload sizes, launched as the benchmark launches it (EngramForward.step(fp8=True):
    the gathered rows quantised by engram_mx_quant, engram_wkv_mx against the layer's MX weights,
    engram_gate_dot): the MX operands bit-exact against the oracle's quantiser (of the oracle's gathered rows
    and of the bf16 weights), kv within the fp8 bar and the dot within the gate bar of the oracle's chain (and
    of the oracle fed the device's kv).  Every token of the mid prefill (both layers); at the long prefill
    4,096 sampled tokens with the first, last and a random token of every 256-token M tile."""
    import torch

    import synth.workload as sw

    cfg = synth.CONFIGS[cfg_index]
    wl = sw.build(cfg, device=gpu_device, packed=True, fp8=True)
    dots = wl.fwd.step(wl.input_ids, 0, wl.x[0], wl.token_mask, packed=True, fp8=True)
    torch.cuda.synchronize()
    hi = wl.host
    B, L = hi.input_ids.shape
    T, C, D, blk, K = cfg.tokens, cfg.n_hash_cols, cfg.head_dim, cfg.block_size, cfg.K
    ids = oracle.hash(hi.input_ids, 0, hi.token_mask, hi.token_map, np.zeros((B, L), np.int64), hi.multipliers,
                      hi.primes, hi.offsets, cfg.pad_id, synth.DEAD)
    sample = sample_tokens(T, n_sample, cfg_index + 100, L=L, mask=hi.token_mask)
    sidx = torch.from_numpy(sample).to(gpu_device)
    x_bits = bits(wl.x[0].view(T, cfg.hc_mult, cfg.dim)[sidx])
    for e in range(cfg.n_layers):
        lw = wl.fwd.layers[e]
        lid = ids.reshape(T, cfg.n_layers, C)[sample, e]
        cw, cs, remap = compact_rows(lid, cfg.rows_alloc[e], synth.table_seed(cfg, e), D, blk)
        a_want = oracle.gather_dequant(remap, cw, cs, block_size=blk).reshape(len(sample), C * D)
        aq_want, as_want = oracle.mx_quant(a_want)
        np.testing.assert_array_equal(wl.fwd._bufs[("a_mx", e)].view(T, K)[sidx].cpu().numpy(), aq_want,
                                      err_msg=f"MX elements of the gathered rows, layer {e}")
        np.testing.assert_array_equal(_scales_rowmajor(wl.fwd._bufs[("a_mx_scale", e)], T, K)[sample], as_want,
                                      err_msg=f"MX scales of the gathered rows, layer {e}")
        wq_want, ws_want = oracle.mx_quant(bits(lw.wkv))
        N = wq_want.shape[0]
        np.testing.assert_array_equal(lw.wkv_mx[0].cpu().numpy(), wq_want, err_msg=f"MX weights, layer {e}")
        np.testing.assert_array_equal(_scales_rowmajor(lw.wkv_mx[1], N, K), ws_want, err_msg=f"MX weight scales {e}")
        kv_got = bits(wl.fwd._bufs[("kv", e)].view(T, -1)[sidx])
        kv_want = _assert_close_cancelling(None, aq_want, as_want, wq_want, ws_want, f"kv (fp8) layer {e}",
                                           kv_bits=kv_got)
        kv_want_bits = torch.from_numpy(kv_want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        q_bits, k_bits = bits(lw.q_weight), bits(lw.k_weight)
        dot_got = dots[e].view(T, -1)[sidx].cpu().numpy()
        assert_close(dot_got, oracle.gate_dot(x_bits, kv_want_bits, q_bits, k_bits, cfg.eps), what=f"dot (fp8) {e}")
        assert_close(dot_got, oracle.gate_dot(x_bits, kv_got, q_bits, k_bits, cfg.eps), rtol=1e-3, atol=1e-4,
                     what=f"dot (fp8, device kv) layer {e}")
        del kv_want, kv_want_bits
    # the fused fp8 projection + gate (engram_wkv_mx_gate) as the benchmark runs it: value columns bit for bit
    # those of the unfused kv above, the dot within the fp32 summation-order bar of the unfused one
    kv_cols = [bits(wl.fwd._bufs[("kv", e)].view(T, -1)[sidx])[:, cfg.hc_mult * cfg.dim:] for e in range(cfg.n_layers)]
    dots_u = [dots[e].view(T, -1)[sidx].cpu().numpy() for e in range(cfg.n_layers)]
    dots_f = wl.fwd.step(wl.input_ids, 0, wl.x[0], wl.token_mask, packed=True, fp8=True, fused=True)
    torch.cuda.synchronize()
    for e in range(cfg.n_layers):
        np.testing.assert_array_equal(bits(wl.fwd._bufs[("value", e)].view(T, -1)[sidx]), kv_cols[e],
                                      err_msg=f"fused fp8 value columns, layer {e}")
        assert_close(dots_f[e].view(T, -1)[sidx].cpu().numpy(), dots_u[e], rtol=1e-3, atol=1e-4,
                     what=f"fused fp8 dot, layer {e}")
    # the same fused step with the gathers writing MX rows directly (engram_gather_mx): the same A operand
    # (every token), hence the same value columns and dots, bit for bit
    keep = {k: [wl.fwd._bufs[(k, e)].clone() for e in range(cfg.n_layers)] for k in ("a_mx", "a_mx_scale", "value")}
    dots_f = [d.clone() for d in dots_f]
    for k in ("a_mx", "a_mx_scale"):
        for e in range(cfg.n_layers):
            wl.fwd._bufs[(k, e)].fill_(0x5A)  # every byte the gather must write is overwritten
    dots_g = wl.fwd.step(wl.input_ids, 0, wl.x[0], wl.token_mask, packed=True, fp8=True, fused=True,
                         gather_mx=True)
    torch.cuda.synchronize()
    for e in range(cfg.n_layers):
        assert torch.equal(wl.fwd._bufs[("a_mx", e)], keep["a_mx"][e]), f"MX rows from the gather, layer {e}"
        np.testing.assert_array_equal(_scales_rowmajor(wl.fwd._bufs[("a_mx_scale", e)], T, K),
                                      _scales_rowmajor(keep["a_mx_scale"][e], T, K),
                                      err_msg=f"MX scales from the gather, layer {e}")
        assert torch.equal(wl.fwd._bufs[("value", e)], keep["value"][e]), f"value columns, layer {e}"
        assert torch.equal(dots_g[e], dots_f[e]), f"dot, layer {e}"


# (T, K, hc, dim): ragged token counts, one token, grids of more tiles than CUs (several key tiles per workgroup,
# so held-back slabs and the next tile's restart run many times), K from the smallest the fused form takes
# (three slabs) to the workloads', the workloads' dim with its 80 key column tiles
MX_GATE_SHAPES = [(300, 384, 2, 256), (257, 1536, 4, 512), (1, 512, 1, 256), (1000, 1536, 4, 5120),
                  (3000, 768, 3, 768), (9000, 384, 4, 1024)]


@pytest.mark.parametrize("T,K,hc,dim", MX_GATE_SHAPES)
def test_wkv_mx_gate_matches_the_unfused_path_and_the_oracle(gpu_device, T, K, hc, dim):
    """engram_wkv_mx_gate against engram_wkv_mx + engram_gate_dot on the same MX operands: the value columns bit
    for bit, the dot within the fp32 summation-order bar; the dot against the oracle's chain (the exact product
    of the dequantised operands, rounded to bf16, then the gate) on sampled tokens; run-to-run identical."""
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(T * 3 + K + hc * 100 + dim)
    N = (hc + 1) * dim
    a = torch.from_numpy(_bf16_rows(rng, T, K, spread=6)).to(torch.bfloat16)
    w = torch.from_numpy((rng.normal(size=(N, K)) * 0.02).astype(np.float32)).to(torch.bfloat16)
    x = torch.from_numpy(rng.normal(size=(T, hc, dim)).astype(np.float32)).to(torch.bfloat16).to(gpu_device)
    q = torch.from_numpy((1 + 0.1 * rng.normal(size=(hc, dim))).astype(np.float32)).to(torch.bfloat16).to(gpu_device)
    k = torch.from_numpy((1 + 0.1 * rng.normal(size=(hc, dim))).astype(np.float32)).to(torch.bfloat16).to(gpu_device)
    eps = 1e-20
    aq, asc = g.engram_mx_quant(a.to(gpu_device))
    wq, wsc = g.engram_mx_quant(w.to(gpu_device))
    value, dot = g.engram_wkv_mx_gate(aq, asc, wq, wsc, x, q, k, eps)
    kv = g.engram_wkv_mx(aq, asc, wq, wsc)
    dot_u = g.engram_gate_dot(x, kv, q, k, eps)
    value2, dot2 = g.engram_wkv_mx_gate(aq, asc, wq, wsc, x, q, k, eps)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(value), bits(kv)[:, hc * dim:], err_msg="value columns")
    assert_close(dot.cpu().numpy(), dot_u.cpu().numpy(), rtol=1e-3, atol=1e-4, what="dot vs the unfused path")
    np.testing.assert_array_equal(bits(value2), bits(value))
    np.testing.assert_array_equal(dot2.cpu().numpy().view(np.uint32), dot.cpu().numpy().view(np.uint32))
    sample = sample_tokens(T, min(T, 384), T + K)
    x_bits = bits(x)[sample]
    q_bits, k_bits = bits(q), bits(k)
    # the fused gate arithmetic against the oracle's, both on the device's keys (engram_wkv_mx's, which the fused
    # kernel forms with the same MFMAs in the same order): the isolating bar
    dot_dev = oracle.gate_dot(x_bits, bits(kv)[sample], q_bits, k_bits, eps)
    assert_close(dot.cpu().numpy()[sample], dot_dev, rtol=1e-3, atol=1e-4, what="dot vs the oracle on the device kv")
    # end to end: the oracle's exact product of the dequantised operands, rounded to bf16, then the gate; the
    # bar adds the fp8 matrix core's accumulation error (2^-12 sum|a w| per key element) carried through the gate
    a_q, a_s = aq.cpu().numpy()[sample], _scales_rowmajor(asc, T, K)[sample]
    w_q, w_s = wq.cpu().numpy(), _scales_rowmajor(wsc, N, K)
    kv_o = oracle.wkv_mx_matmul(a_q, a_s, w_q, w_s)
    kv_o_bits = torch.from_numpy(kv_o).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    dot_o = oracle.gate_dot(x_bits, kv_o_bits, q_bits, k_bits, eps)
    extra = _gate_bound_of_key_error(x_bits, kv_o_bits,
                                     2.0 ** -12 * (np.abs(oracle.mx_dequant(a_q, a_s)) @ np.abs(oracle.mx_dequant(w_q, w_s)).T),
                                     q_bits, k_bits, eps)
    assert_close(dot.cpu().numpy()[sample], dot_o, atol=1e-3 + extra, what="dot vs the oracle")


def _gate_bound_of_key_error(x_bits, kv_bits, key_err, q_bits, k_bits, eps):
    """A bound on how far the gate pre-activation moves when every key element moves by at most key_err
    [n, Nout] (first order): dot = S rh rk dim^-1/2 with S = sum(h w key), rk = (mean key^2 + eps)^-1/2, so
    |d dot| <= dim^-1/2 rh (rk sum|h w| |d key| + |S| rk^3 mean(|key| |d key|))."""
    hc, dim = q_bits.shape
    n = x_bits.shape[0]
    h = oracle.bf16_bits_to_float(x_bits).astype(np.float64).reshape(n, hc, dim)
    key = oracle.bf16_bits_to_float(kv_bits[:, :hc * dim]).astype(np.float64).reshape(n, hc, dim)
    dk = key_err[:, :hc * dim].reshape(n, hc, dim)
    w = (oracle.bf16_bits_to_float(q_bits).astype(np.float64) * oracle.bf16_bits_to_float(k_bits).astype(np.float64))
    rh = 1.0 / np.sqrt((h * h).mean(-1) + eps)
    rk = 1.0 / np.sqrt((key * key).mean(-1) + eps)
    S = (h * w * key).sum(-1)
    return dim ** -0.5 * rh * (rk * (np.abs(h * w) * dk).sum(-1) + np.abs(S) * rk ** 3 * (np.abs(key) * dk).mean(-1))
