"""engram_gather_mx / engram_gather_mx_packed (the gather writing its rows as MX fp8) on the GPU: bit for bit the
oracle's MX quantiser applied to the oracle's gathered rows -- elements and E8M0 scales, the scales read back
from the library's layout -- on small tables (ragged row counts, ids outside the rank's rows, every finite fp8
code under varied scales, both table layouts); and on a workload's full-size table bit for bit
engram_mx_quant of engram_gather_dequant's rows over every token, and the oracle on sampled tokens."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bits, compact_rows, mx_scales_rowmajor, sample_tokens

pytestmark = pytest.mark.gpu


def _gather_mx(dev, ids, w, s, blk, row_start, C, packed):
    import torch

    import gram_hash_embedding_amd as g

    w_t = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
    s_t = torch.from_numpy(np.ascontiguousarray(s)).to(dev)
    ids_t = torch.from_numpy(np.ascontiguousarray(ids)).to(dev)
    if packed:
        q, sc = g.engram_gather_mx(ids_t, table=g.engram_pack_table(w_t, s_t, blk), block_size=blk,
                                   row_start=row_start, n_cols=C)
    else:
        q, sc = g.engram_gather_mx(ids_t, w_t, s_t, block_size=blk, row_start=row_start, n_cols=C)
    torch.cuda.synchronize()
    T = ids.shape[0]
    return q.cpu().numpy(), mx_scales_rowmajor(sc, T, C * w.shape[1])


def _want(ids, w, s, blk, row_start, C):
    rows = oracle.gather_dequant(ids, w, s, row_start=row_start, block_size=blk, n_cols=C)
    return oracle.mx_quant(rows.reshape(ids.shape[0], -1))


# (D, blk, C): C*D a multiple of 128 (whole 128-column groups of the scale layout), MX blocks of 32 across
# table scale blocks of 16 to 256
@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("D,blk,C", [(32, 32, 4), (32, 16, 12), (64, 32, 10), (64, 16, 2), (128, 32, 5),
                                     (128, 64, 3), (256, 32, 1), (256, 256, 3)])
def test_gather_mx_matches_the_oracle(gpu_device, D, blk, C, packed):
    R, row_start = 2999, 300
    w, s = synth.table_rows(D * 13 + blk, np.arange(R), D, blk)
    s[:40] *= np.float32(2.0 ** 20)   # products past E4M3's range once rounded to bf16: the shared
    s[40:80] *= np.float32(2.0 ** -60)  # exponent follows them (and subnormal bf16 values)
    rng = np.random.default_rng(D * 5 + blk + C)
    T, stride = 301, C + 2  # ragged: 301 tokens fill no 4-row group of the scale layout
    ids = rng.integers(row_start - 30, row_start + R + 30, size=(T, stride), dtype=np.int64)
    ids[0, :min(C, 3)] = [-(2 ** 62), 2 ** 62, row_start + R][:min(C, 3)]  # out of range: zero rows
    ids[1, :] = row_start + np.arange(stride) % 80  # the rows with the extreme scales
    got_q, got_s = _gather_mx(gpu_device, ids, w, s, blk, row_start, C, packed)
    want_q, want_s = _want(ids, w, s, blk, row_start, C)
    np.testing.assert_array_equal(got_q, want_q)
    np.testing.assert_array_equal(got_s, want_s)
    assert (got_q[0, :D] == 0).all() and (got_s[0, :D // 32] == 0).all()  # a zero row: bytes 0, scale code 0


@pytest.mark.parametrize("packed", [False, True])
def test_gather_mx_every_finite_code(gpu_device, packed):
    """Rows holding every finite fp8 code (both zeros, subnormals, +-448) under varied scales, among them
    products in fp32's subnormal range."""
    D, blk = 64, 32
    codes = np.arange(256 * 4, dtype=np.int64).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00  # the NaN codes: outside the quantiser's finite inputs
    w = codes.reshape(16, 64)
    s = np.array([[2.0 ** -8, 0.3], [1.0, 2.0 ** -2], [0.0625, 0.1], [3.0, 7.5]] * 4, dtype=np.float32)
    s[5] = [2.0 ** -126, 1e-30]
    s[6] = [2.0 ** 40, 2.0 ** 100]
    ids = np.arange(16, dtype=np.int64).reshape(8, 2)
    got_q, got_s = _gather_mx(gpu_device, ids, w, s, blk, 0, 2, packed)
    want_q, want_s = _want(ids, w, s, blk, 0, 2)
    np.testing.assert_array_equal(got_q, want_q)
    np.testing.assert_array_equal(got_s, want_s)


@pytest.mark.parametrize("cfg_index", [2, 3])
def test_gather_mx_workload(gpu_device, cfg_index):
    """A workload's full-size table (both layouts): every token bit for bit engram_mx_quant of
    engram_gather_dequant's rows; 4,096 sampled tokens (every 256-token tile) against the oracle."""
    import torch

    import gram_hash_embedding_amd as g
    import synth.device as sd

    cfg = synth.CONFIGS[cfg_index]
    hi = synth.hash_inputs(cfg)
    B, L = hi.input_ids.shape
    ids = oracle.hash(hi.input_ids, 0, hi.token_mask, hi.token_map, np.zeros((B, L), np.int64), hi.multipliers,
                      hi.primes, hi.offsets, cfg.pad_id, synth.DEAD)
    ids_dev = torch.from_numpy(ids).to(gpu_device)
    T, C, D, blk = cfg.tokens, cfg.n_hash_cols, cfg.head_dim, cfg.block_size
    K = C * D
    e = cfg.n_layers - 1
    R = cfg.rows_alloc[e]
    w_dev, s_dev = sd.device_table(synth.table_seed(cfg, e), R, D, blk, gpu_device)
    rows = g.engram_gather_dequant(ids_dev, w_dev, s_dev, blk, layer=e)
    q_chain, s_chain = g.engram_mx_quant(rows.view(T, K))
    del rows
    q, sc = g.engram_gather_mx(ids_dev, w_dev, s_dev, block_size=blk, layer=e)
    torch.cuda.synchronize()
    assert torch.equal(q, q_chain)
    np.testing.assert_array_equal(mx_scales_rowmajor(sc, T, K), mx_scales_rowmajor(s_chain, T, K))
    packed = g.engram_pack_table(w_dev, s_dev, blk)
    del w_dev, s_dev
    torch.cuda.empty_cache()
    qp, scp = g.engram_gather_mx(ids_dev, table=packed, block_size=blk, layer=e)
    torch.cuda.synchronize()
    assert torch.equal(qp, q_chain)
    np.testing.assert_array_equal(mx_scales_rowmajor(scp, T, K), mx_scales_rowmajor(s_chain, T, K))
    sample = sample_tokens(T, 4096, cfg_index + 20, L=L, mask=hi.token_mask)
    lid = ids.reshape(T, cfg.n_layers, C)[sample, e]
    cw, cs, remap = compact_rows(lid, R, synth.table_seed(cfg, e), D, blk)
    want_q, want_s = oracle.mx_quant(oracle.gather_dequant(remap, cw, cs, block_size=blk).reshape(len(sample), K))
    np.testing.assert_array_equal(q[torch.from_numpy(sample).to(gpu_device)].cpu().numpy(), want_q)
    np.testing.assert_array_equal(mx_scales_rowmajor(sc, T, K)[sample], want_s)
    del packed, q, qp, sc, scp, q_chain, s_chain
    torch.cuda.empty_cache()
