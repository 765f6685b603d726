"""The whole path at workload sizes, launched exactly as the benchmark launches
it (gram_hash_embedding_amd.forward.EngramForward), against the oracle's own
pipeline: hash ids in full, gathered rows bit-exact, kv and the gate
pre-activation within tolerance; the fused projection + gate dot (value
columns bit-exact against the unfused kv, dot within tolerance); then the
whole module (gate, mask, residual) unfused and fused, as the benchmark's
loops run them, the output stream within tolerance and masked tokens
bit-exact.  The tiny and mid-prefill workloads are checked on every token;
the long prefill, the gather-stress workload (per layer) and the released
head_dim on sampled tokens that include a token at both edges of, and one at
random inside, every 256-token tile of the projection, every sequence's first
three positions and the three after every masked span.  The projection's
oracle there is the float64 library-matmul form (oracle.wkv_matmul)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_close, assert_output_close, bits, compact_rows, sample_tokens

pytestmark = pytest.mark.gpu


def _oracle_kv_bf16(kv64):
    import torch

    return torch.from_numpy(kv64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("cfg_index,n_sample", [(1, 64), (2, 8192), (3, 4096), (5, 4096), (6, 2048)])
def test_forward_pipeline(gpu_device, cfg_index, n_sample):
    import torch

    import synth.workload as sw

    cfg = synth.CONFIGS[cfg_index]
    wl = sw.build(cfg, device=gpu_device)
    dots = wl.fwd.step(wl.input_ids, 0, wl.x[0], wl.token_mask)
    torch.cuda.synchronize()
    hi = wl.host
    B, L = hi.input_ids.shape
    T, C, D, blk = cfg.tokens, cfg.n_hash_cols, cfg.head_dim, cfg.block_size
    ids = oracle.hash(hi.input_ids, 0, hi.token_mask, hi.token_map, np.zeros((B, L), np.int64), hi.multipliers,
                      hi.primes, hi.offsets, cfg.pad_id, synth.DEAD)
    np.testing.assert_array_equal(wl.fwd._bufs["ids"].view(B, L, cfg.n_layers, C).cpu().numpy(), ids)
    masked = [] if hi.token_mask is None else np.flatnonzero(hi.token_mask.reshape(T) == 0)
    extra = masked[:: max(1, len(masked) // 16)][:16] if len(masked) else ()
    sample = sample_tokens(T, n_sample, cfg_index, L=L, mask=hi.token_mask, extra=extra)
    sidx = torch.from_numpy(sample).to(gpu_device)
    x_bits = bits(wl.x[0].view(T, cfg.hc_mult, cfg.dim)[sidx])
    want = []
    for e in range(cfg.n_layers):
        lw = wl.fwd.layers[e]
        a_gpu, kv_gpu, dot_gpu = wl.fwd._bufs[("a", e)], wl.fwd._bufs[("kv", e)], dots[e]
        lid = ids.reshape(T, cfg.n_layers, C)[sample, e]
        cw, cs, remap = compact_rows(lid, cfg.rows_alloc[e], synth.table_seed(cfg, e), D, blk)
        a_want = oracle.gather_dequant(remap, cw, cs, block_size=blk).reshape(len(sample), C * D)
        a_got = bits(a_gpu.view(T, C * D)[sidx])
        np.testing.assert_array_equal(a_got, a_want, err_msg=f"gathered rows, layer {e}")
        w_bits = bits(lw.wkv)
        kv_want = oracle.wkv_matmul(a_want, w_bits)
        kv_got = bits(kv_gpu.view(T, -1)[sidx])
        assert_close(oracle.bf16_bits_to_float(kv_got), kv_want, what=f"kv layer {e}")
        q_bits, k_bits = bits(lw.q_weight), bits(lw.k_weight)
        # the gate on the oracle's own (bf16-rounded) kv: end to end
        dot_want = oracle.gate_dot(x_bits, _oracle_kv_bf16(kv_want), q_bits, k_bits, cfg.eps)
        assert_close(dot_gpu.view(T, -1)[sidx].cpu().numpy(), dot_want, what=f"dot layer {e}")
        # and on the GPU's kv: isolates the gate kernel
        dot_unit = oracle.gate_dot(x_bits, kv_got, q_bits, k_bits, cfg.eps)
        assert_close(dot_gpu.view(T, -1)[sidx].cpu().numpy(), dot_unit, rtol=1e-3, atol=1e-4,
                     what=f"dot (gpu kv) layer {e}")
        want.append((_oracle_kv_bf16(kv_want), dot_want))

    m = None if hi.token_mask is None else hi.token_mask.reshape(T)[sample].astype(np.uint8)
    hcd = cfg.hc_mult * cfg.dim
    for fused in (False, True):
        # the fused projection + gate dot: same dot, value columns only
        if fused:
            dots_f = wl.fwd.step(wl.input_ids, 0, wl.x[0], wl.token_mask, fused=True)
            torch.cuda.synchronize()
            for e in range(cfg.n_layers):
                kv_o, dot_o = want[e]
                assert_close(dots_f[e].view(T, -1)[sidx].cpu().numpy(), dot_o, what=f"dot (fused) layer {e}")
                v_got = bits(wl.fwd._bufs[("value", e)].view(T, -1)[sidx])
                np.testing.assert_array_equal(v_got, bits(wl.fwd._bufs[("kv", e)].view(T, -1)[sidx])[:, hcd:],
                                              err_msg=f"fused value columns, layer {e}")
            # every layer's fused projection in one launch (engram_wkv_gate_layers)
            dots_l = wl.fwd.step(wl.input_ids, 0, wl.x[0], wl.token_mask, fused=True, all_layers=True)
            torch.cuda.synchronize()
            for e in range(cfg.n_layers):
                kv_o, dot_o = want[e]
                assert_close(dots_l[e].view(T, -1)[sidx].cpu().numpy(), dot_o, what=f"dot (all layers) layer {e}")
                v_got = bits(wl.fwd._bufs[("value", e)].view(T, -1)[sidx])
                np.testing.assert_array_equal(v_got, bits(wl.fwd._bufs[("kv", e)].view(T, -1)[sidx])[:, hcd:],
                                              err_msg=f"value columns (all layers), layer {e}")
        outs = wl.fwd.step(wl.input_ids, 0, wl.x[0], wl.token_mask, output=True, fused=fused)
        torch.cuda.synchronize()
        for e in range(cfg.n_layers):
            kv_o, dot_o = want[e]
            assert_close(wl.fwd._bufs[("dot", e)].view(T, -1)[sidx].cpu().numpy(), dot_o,
                         what=f"dot (output, fused={fused}) layer {e}")
            _, out_want = oracle.gate_output(x_bits, kv_o, dot_o, m)
            out_got = bits(outs[e].view(T, cfg.hc_mult, cfg.dim)[sidx])
            assert_output_close(out_got, out_want, oracle.bf16_bits_to_float(kv_o[:, hcd:]), what=f"out (fused={fused}) layer {e}")
            # the gate, mask and residual alone: the oracle fed the device's own value and dot (only the
            # output's fp32 sum and bf16 rounding differ)
            v_dev = bits(wl.fwd._bufs[("value", e)].view(T, -1)[sidx]) if fused else \
                bits(wl.fwd._bufs[("kv", e)].view(T, -1)[sidx])[:, hcd:]
            kv_dev = np.zeros((len(sample), hcd + cfg.dim), np.uint16)
            kv_dev[:, hcd:] = v_dev[:, :cfg.dim]
            d_dev = wl.fwd._bufs[("dot", e)].view(T, -1)[sidx].cpu().numpy().astype(np.float64)
            _, out_unit = oracle.gate_output(x_bits, kv_dev, d_dev, m)
            assert_close(oracle.bf16_bits_to_float(out_got), out_unit, rtol=2.0 ** -8, atol=1e-5,
                         what=f"out from the device's value and dot (fused={fused}) layer {e}")
            if m is not None:
                np.testing.assert_array_equal(out_got[m == 0], x_bits[m == 0],
                                              err_msg=f"masked tokens (fused={fused}), layer {e}")


def test_decode_pipeline(gpu_device):
    """The decode workload as the benchmark runs it: the hash of the 4,096-token history, then 64 calls of
    one token per sequence through the whole path (through the residual), each with its own stream, the
    fused and the four-entry-point projection in turn, and the hash and gathers as one launch in half the
    calls (steps 0 and 1 of every four), the fused projections of both layers as one launch in a quarter
    (step 0 of every four).  Every step's hash ids and gathered rows are checked bit-exact for all 256
    sequences; sixteen steps (0-7, 28-31, 60-63: every launch arrangement four times, 4,096 tokens) also the
    gate pre-activation and the output stream, within tolerance."""
    import torch

    import synth.workload as sw

    cfg = synth.CONFIGS[4]
    wl = sw.build(cfg, device=gpu_device, packed=True, x_steps=cfg.decode_steps)
    hi = wl.host
    B, Ltot = hi.input_ids.shape
    P, E, C, D, blk = cfg.start_pos, cfg.n_layers, cfg.n_hash_cols, cfg.head_dim, cfg.block_size
    hc, dim = cfg.hc_mult, cfg.dim
    ids_all = oracle.hash(hi.input_ids, 0, None, hi.token_map, np.zeros((B, Ltot), np.int64), hi.multipliers,
                          hi.primes, hi.offsets, cfg.pad_id, synth.DEAD)
    wl.fwd.hash(wl.input_ids[:, :P].contiguous(), 0)
    seqs = np.arange(B)
    sidx = torch.from_numpy(seqs).to(gpu_device)
    n = cfg.decode_steps
    checked = set(range(8)) | set(range(n // 2 - 4, n // 2)) | set(range(n - 4, n))
    for s in range(cfg.decode_steps):
        fused = s % 2 == 0
        outs = wl.fwd.step(wl.input_ids[:, P + s:P + s + 1].contiguous(), P + s, wl.x[s], None, output=True,
                           fused=fused, packed=True, hash_gather=s % 4 < 2, all_layers=s % 4 == 0)
        torch.cuda.synchronize()
        ids_got = wl.fwd._bufs["ids"][:B * E * C].view(B, E, C).cpu().numpy()  # (the buffer held the prefill)
        np.testing.assert_array_equal(ids_got, ids_all[:, P + s], err_msg=f"hash ids, step {s}")
        x_bits = bits(wl.x[s].view(B, hc, dim)[sidx])
        for e in range(E):
            lw = wl.fwd.layers[e]
            cw, cs, remap = compact_rows(ids_all[seqs, P + s, e], cfg.rows_alloc[e], synth.table_seed(cfg, e), D,
                                         blk)
            a_want = oracle.gather_dequant(remap, cw, cs, block_size=blk).reshape(len(seqs), C * D)
            a_got = bits(wl.fwd._bufs[("a", e)][:B * C * D].view(B, C * D)[sidx])
            np.testing.assert_array_equal(a_got, a_want, err_msg=f"gathered rows, step {s}, layer {e}")
            if s not in checked:
                continue
            kv_want = _oracle_kv_bf16(oracle.wkv_matmul(a_want, bits(lw.wkv)))
            dot_want = oracle.gate_dot(x_bits, kv_want, bits(lw.q_weight), bits(lw.k_weight), cfg.eps)
            dot_got = wl.fwd._bufs[("dot", e)][:B * hc].view(B, hc)[sidx].cpu().numpy()
            assert_close(dot_got, dot_want, what=f"dot, step {s}, layer {e}, fused={fused}")
            _, out_want = oracle.gate_output(x_bits, kv_want, dot_want, None)
            out_got = bits(outs[e].view(B, hc, dim)[sidx])
            assert_output_close(out_got, out_want, oracle.bf16_bits_to_float(kv_want[:, hc * dim:]),
                                what=f"out, step {s}, layer {e}, fused={fused}")


def test_decode_step_graph_replays_match_eager(gpu_device):
    """The benchmark replays the decode step as a HIP graph: a graph of 8 one-token calls (fused and
    four-entry-point projections alternating, the hash and gathers fused in half of them, both layers'
    projections in one launch in a quarter) replayed three times, with eager work and synchronisations in
    between, gives every call's dot and output bit for bit as the eager calls do, and leaves the same cache."""
    import torch

    import synth.workload as sw

    cfg = synth.CONFIGS[4]
    steps = 8
    wl = sw.build(cfg, device=gpu_device, packed=True, x_steps=steps)
    P, E, hc = cfg.start_pos, cfg.n_layers, cfg.hc_mult
    B = cfg.batch
    wl.fwd.hash(wl.input_ids[:, :P].contiguous(), 0)
    step_ids = [wl.input_ids[:, P + s:P + s + 1].contiguous() for s in range(steps)]
    hist = torch.zeros((steps, E, B, hc), dtype=torch.float32, device=gpu_device)
    outs_hist = torch.zeros((steps, E) + tuple(wl.x[0].shape), dtype=torch.bfloat16, device=gpu_device)

    def run():
        for s in range(steps):
            outs = wl.fwd.step(step_ids[s], P + s, wl.x[s], None, output=True, fused=s % 2 == 0, packed=True,
                               hash_gather=s % 4 < 2, all_layers=s % 4 == 0)
            for e in range(E):
                hist[s, e].copy_(wl.fwd._bufs[("dot", e)][:B * hc].view(B, hc))
                outs_hist[s, e].copy_(outs[e])

    run()  # eager (also allocates every buffer the step uses)
    torch.cuda.synchronize()
    want_dot, want_out = hist.clone(), outs_hist.clone()
    want_cache = wl.fwd.state.cache.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for r in range(3):
        hist.zero_()
        outs_hist.zero_()
        wl.fwd.state.cache[:, P:P + steps].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(hist, want_dot), f"replay {r}: dots"
        assert torch.equal(outs_hist.view(torch.int16), want_out.view(torch.int16)), f"replay {r}: outputs"
        assert torch.equal(wl.fwd.state.cache, want_cache), f"replay {r}: cache"
        run()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(hist, want_dot), f"eager after replay {r}"
