"""The whole path at workload sizes, launched exactly as the benchmark launches
it (gram_hash_embedding_amd.forward.EngramForward), against the oracle's own
pipeline on sampled tokens: hash ids in full, gathered rows bit-exact, kv and
the gate pre-activation within tolerance."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_close, bits, compact_rows, sample_tokens

pytestmark = pytest.mark.gpu


def _oracle_kv_bf16(kv64):
    import torch

    return torch.from_numpy(kv64).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("cfg_index,n_sample", [(1, 64), (2, 192), (3, 128), (5, 96)])
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
    sample = sample_tokens(T, n_sample, cfg_index, L=L, mask=hi.token_mask)
    sidx = torch.from_numpy(sample).to(gpu_device)
    x_bits = bits(wl.x[0].view(T, cfg.hc_mult, cfg.dim)[sidx])
    for e in range(cfg.n_layers):
        lw = wl.fwd.layers[e]
        a_gpu, kv_gpu, dot_gpu = wl.fwd._bufs[("a", e)], wl.fwd._bufs[("kv", e)], dots[e]
        lid = ids.reshape(T, cfg.n_layers, C)[sample, e]
        cw, cs, remap = compact_rows(lid, cfg.rows_alloc[e], synth.table_seed(cfg, e), D, blk)
        a_want = oracle.gather_dequant(remap, cw, cs, block_size=blk).reshape(len(sample), C * D)
        a_got = bits(a_gpu.view(T, C * D)[sidx])
        np.testing.assert_array_equal(a_got, a_want, err_msg=f"gathered rows, layer {e}")
        w_bits = bits(lw.wkv)
        kv_want = oracle.wkv(a_want, w_bits)
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
