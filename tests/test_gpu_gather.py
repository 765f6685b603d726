"""engram_gather_dequant on the GPU against the oracle: gathered fp8 bytes,
scales and dequantised bf16 rows bit-exact."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bits, compact_rows

pytestmark = pytest.mark.gpu


def _run(dev, ids, w, s, blk, row_start=0, n_cols=None):
    import torch

    import gram_hash_embedding_amd as g

    ids_t = torch.from_numpy(np.ascontiguousarray(ids)).to(dev)
    w_t = torch.from_numpy(np.ascontiguousarray(w)).to(dev) if isinstance(w, np.ndarray) else w
    s_t = torch.from_numpy(np.ascontiguousarray(s)).to(dev) if isinstance(s, np.ndarray) else s
    T = ids.shape[0]
    C = ids.shape[1] if n_cols is None else n_cols
    D = w_t.shape[1]
    f8 = torch.empty((T, C, D), dtype=torch.uint8, device=dev)
    sc = torch.empty((T, C, D // blk), dtype=torch.float32, device=dev)
    out = g.engram_gather_dequant(ids_t, w_t, s_t, blk, row_start, n_cols=n_cols, out_fp8=f8, out_scale=sc)
    return bits(out), f8.cpu().numpy(), sc.cpu().numpy()


def _check(got, want):
    gb, g8, gs = got
    wb, w8, ws = want
    np.testing.assert_array_equal(g8, w8)
    np.testing.assert_array_equal(gs.view(np.uint32), ws.view(np.uint32))
    gf, wf = oracle.bf16_bits_to_float(gb), oracle.bf16_bits_to_float(wb)
    np.testing.assert_array_equal(np.isnan(gf), np.isnan(wf))
    ok = ~np.isnan(wf)
    np.testing.assert_array_equal(gb[ok], wb[ok])


@pytest.mark.parametrize("D,blk", [(32, 32), (64, 32), (64, 16), (128, 32), (128, 64), (256, 32), (256, 256)])
def test_gather_shapes_and_out_of_range(gpu_device, D, blk):
    R, row_start = 3001, 500
    w, s = synth.table_rows(D * 7 + blk, np.arange(R), D, blk)
    rng = np.random.default_rng(D + blk)
    T, stride, C = 301, 9, 7  # 301*7 rows: ragged against every block size
    ids = rng.integers(row_start - 40, row_start + R + 40, size=(T, stride), dtype=np.int64)
    ids[0, :3] = [-(2**62), 2**62, row_start + R]
    got = _run(gpu_device, ids, w, s, blk, row_start, n_cols=C)
    want = oracle.gather_dequant(ids, w, s, row_start=row_start, block_size=blk, n_cols=C, want_raw=True)
    _check(got, want)
    assert (got[0][0, :3] == 0).all()


def test_gather_every_byte_value(gpu_device):
    # rows holding all 256 codes (both zeros, subnormals, +-448, the two NaN codes) under varied scales
    D, blk = 64, 32
    w = np.arange(256 * 4, dtype=np.int64).reshape(16, 64).astype(np.uint8)
    s = np.array([[2.0**-8, 0.3], [1.0, 2.0**-2], [0.0625, 0.1], [3.0, 7.5]] * 4, dtype=np.float32)
    s[5] = [2.0**-126, 1e-30]  # products in the fp32 subnormal range
    ids = np.arange(16, dtype=np.int64).reshape(16, 1).repeat(3, axis=1)
    got = _run(gpu_device, ids, w, s, blk)
    want = oracle.gather_dequant(ids, w, s, block_size=blk, want_raw=True)
    _check(got, want)


def test_fill_kernel_matches_host_generator(gpu_device):
    import synth.device as sd

    cfg = synth.CONFIGS[3]
    R = cfg.rows_alloc[0]
    w, s = sd.device_table(synth.table_seed(cfg, 0), R, cfg.head_dim, cfg.block_size, gpu_device)
    rows = np.concatenate([np.arange(4), np.random.default_rng(0).integers(0, R, 20000), [R - 2, R - 1]])
    ww, ss = synth.table_rows(synth.table_seed(cfg, 0), rows, cfg.head_dim, cfg.block_size)
    import torch

    idx = torch.from_numpy(rows).to(gpu_device)
    np.testing.assert_array_equal(w[idx].cpu().numpy(), ww)
    np.testing.assert_array_equal(s[idx].cpu().numpy().view(np.uint32), ss.view(np.uint32))


@pytest.mark.parametrize("cfg_index", [1, 2, 3, 5])
def test_gather_config(gpu_device, cfg_index):
    """Each layer's gather of a workload, every token and column (the gather-stress workload's 131,072
    tokens per layer in chunks of 16,384, so the host copy of the rows they reach stays small)."""
    import torch

    import gram_hash_embedding_amd as g
    import synth.device as sd

    cfg = synth.CONFIGS[cfg_index]
    hi = synth.hash_inputs(cfg)
    B, L = hi.input_ids.shape
    ids = oracle.hash(hi.input_ids, 0, hi.token_mask, hi.token_map, np.zeros((B, L), np.int64), hi.multipliers,
                      hi.primes, hi.offsets, cfg.pad_id, synth.DEAD)
    ids_dev = torch.from_numpy(ids).to(gpu_device)  # the oracle's ids (the GPU hash is checked separately)
    T, C, D, blk = cfg.tokens, cfg.n_hash_cols, cfg.head_dim, cfg.block_size
    chunk = 16384
    for e in range(cfg.n_layers):
        R = cfg.rows_alloc[e]
        w_dev, s_dev = sd.device_table(synth.table_seed(cfg, e), R, D, blk, gpu_device)
        out = g.engram_gather_dequant(ids_dev, w_dev, s_dev, blk, layer=e)
        torch.cuda.synchronize()
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            got = bits(out.view(T, C, D)[t0:t1])
            lid = ids.reshape(T, cfg.n_layers, C)[t0:t1, e]
            cw, cs, remap = compact_rows(lid, R, synth.table_seed(cfg, e), D, blk)
            want = oracle.gather_dequant(remap, cw, cs, block_size=blk)
            np.testing.assert_array_equal(got, want, err_msg=f"layer {e}, tokens [{t0}, {t1})")
        del w_dev, s_dev, out
        torch.cuda.empty_cache()


def _pack_on_host(w, s, D):
    """The packed layout written out on the host: row bytes, then the scales' bytes, then zeros."""
    R = w.shape[0]
    rec = np.zeros((R, 2 * D), dtype=np.uint8)
    rec[:, :D] = w
    sb = np.ascontiguousarray(s.astype("<f4")).view(np.uint8)
    rec[:, D:D + sb.shape[1]] = sb
    return rec


@pytest.mark.parametrize("D,blk", [(32, 32), (32, 16), (64, 32), (64, 16), (128, 32), (256, 32), (256, 256)])
def test_packed_table_and_gather(gpu_device, D, blk):
    """engram_pack_table writes the documented record layout; the packed gather equals the oracle bit for bit."""
    import torch

    import gram_hash_embedding_amd as g

    R, row_start = 2999, 300
    w, s = synth.table_rows(D * 11 + blk, np.arange(R), D, blk)
    w_t = torch.from_numpy(w).to(gpu_device)
    s_t = torch.from_numpy(s).to(gpu_device)
    packed = g.engram_pack_table(w_t, s_t, blk)
    np.testing.assert_array_equal(packed.cpu().numpy(), _pack_on_host(w, s, D))
    rng = np.random.default_rng(D * 3 + blk)
    T, stride, C = 257, 11, 9
    ids = rng.integers(row_start - 30, row_start + R + 30, size=(T, stride), dtype=np.int64)
    ids[0, :3] = [-(2**62), 2**62, row_start + R]
    ids_t = torch.from_numpy(ids).to(gpu_device)
    f8 = torch.empty((T, C, D), dtype=torch.uint8, device=gpu_device)
    sc = torch.empty((T, C, D // blk), dtype=torch.float32, device=gpu_device)
    out = g.engram_gather_dequant_packed(ids_t, packed, blk, row_start, n_cols=C, out_fp8=f8, out_scale=sc)
    want = oracle.gather_dequant(ids, w, s, row_start=row_start, block_size=blk, n_cols=C, want_raw=True)
    _check((bits(out), f8.cpu().numpy(), sc.cpu().numpy()), want)
    unpacked = g.engram_gather_dequant(ids_t, w_t, s_t, blk, row_start, n_cols=C)
    np.testing.assert_array_equal(bits(out), bits(unpacked))


@pytest.mark.parametrize("cfg_index", [2, 3])
def test_packed_gather_config(gpu_device, cfg_index):
    """The packed gather of a workload's full-size table on sampled tokens, against the oracle."""
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
    sample = np.sort(np.random.default_rng(cfg_index + 10).choice(T, min(T, 4096), replace=False))
    e = cfg.n_layers - 1
    R = cfg.rows_alloc[e]
    w_dev, s_dev = sd.device_table(synth.table_seed(cfg, e), R, D, blk, gpu_device)
    packed = g.engram_pack_table(w_dev, s_dev, blk)
    del w_dev, s_dev
    torch.cuda.empty_cache()
    out = g.engram_gather_dequant_packed(ids_dev, packed, blk, layer=e)
    got = bits(out.view(T, C, D)[torch.from_numpy(sample).to(gpu_device)])
    lid = ids.reshape(T, cfg.n_layers, C)[sample, e]
    cw, cs, remap = compact_rows(lid, R, synth.table_seed(cfg, e), D, blk)
    want = oracle.gather_dequant(remap, cw, cs, block_size=blk)
    np.testing.assert_array_equal(got, want)
    del packed, out
    torch.cuda.empty_cache()
