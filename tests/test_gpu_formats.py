"""int32 hash ids (engram_hash_i32) and the table's block scales as E8M0 or
float8_e4m3fn bytes (engram_gather_dequant_fmt) on the GPU, against the
oracle bit for bit: ids, dequantised rows, gathered bytes and gathered scale
elements; on small tables with every scale code and ids on both sides of the
share, and on the workloads' full-size tables (their one-byte scales derived
on the device from the seeded float32 scales, synth.scale_bytes)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bits, compact_rows, sample_tokens

pytestmark = pytest.mark.gpu


def _narrow(ids64):
    """The int32 form of hash ids: ids outside [0, 2^31) become -1."""
    return np.where((ids64 >= 0) & (ids64 < 2 ** 31), ids64, -1).astype(np.int32)


@pytest.mark.parametrize("cfg_index", [1, 2, 3])
def test_hash_i32_matches_the_oracle(gpu_device, cfg_index):
    import torch

    import gram_hash_embedding_amd as g

    cfg = synth.CONFIGS[cfg_index]
    hi = synth.hash_inputs(cfg)
    B, L = hi.input_ids.shape
    want = oracle.hash(hi.input_ids, 0, hi.token_mask, hi.token_map, np.zeros((B, L), np.int64), hi.multipliers,
                       hi.primes, hi.offsets, cfg.pad_id, synth.DEAD)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu_device)
    cache = torch.zeros((B, L), dtype=torch.int64, device=gpu_device)
    got = g.engram_hash(t(hi.input_ids), 0, None if hi.token_mask is None else t(hi.token_mask), t(hi.token_map),
                        cache, t(hi.multipliers), t(hi.primes), t(hi.offsets), cfg.pad_id, synth.DEAD, int32_ids=True)
    torch.cuda.synchronize()
    assert got.dtype == torch.int32
    np.testing.assert_array_equal(got.cpu().numpy(), _narrow(want))
    assert (want < 2 ** 31).all()


def test_hash_i32_ids_outside_int32_become_minus_one(gpu_device):
    import torch

    import gram_hash_embedding_amd as g

    cfg = synth.CONFIGS[1]
    hi = synth.hash_inputs(cfg)
    B, L = hi.input_ids.shape
    offs = hi.offsets.copy()
    offs[0, :2] = [2 ** 31 - 1000, -5000]  # ids past 2^31 - 1, and negative ids
    want = oracle.hash(hi.input_ids, 0, None, hi.token_map, np.zeros((B, L), np.int64), hi.multipliers, hi.primes,
                       offs, cfg.pad_id, synth.DEAD)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu_device)
    cache = torch.zeros((B, L), dtype=torch.int64, device=gpu_device)
    got = g.engram_hash(t(hi.input_ids), 0, None, t(hi.token_map), cache, t(hi.multipliers), t(hi.primes), t(offs),
                        cfg.pad_id, synth.DEAD, int32_ids=True).cpu().numpy()
    np.testing.assert_array_equal(got, _narrow(want))
    assert (got[..., 0, 0] >= 2 ** 31 - 1000).any() or (got[..., 0, 0] == -1).any()
    assert (got[..., 0, 1] == -1).all()


@pytest.mark.parametrize("fmt,blk,D,id_bytes", [("e8m0", 32, 64, 4), ("e8m0", 32, 64, 8), ("e4m3", 16, 64, 4),
                                                ("e4m3", 16, 32, 8), ("e8m0", 32, 256, 4), ("e4m3", 16, 128, 4),
                                                ("fp32", 32, 64, 4), ("e8m0", 64, 128, 8)])
def test_gather_fmt_matches_the_oracle(gpu_device, fmt, blk, D, id_bytes):
    import torch

    import gram_hash_embedding_amd as g

    rng = np.random.default_rng(D * 5 + blk + id_bytes)
    R, row_start, T, stride, C = 2999, 300, 257, 11, 9
    w, s32 = synth.table_rows(D * 13 + blk, np.arange(R), D, blk)
    if fmt == "fp32":
        s = s32
    else:
        s = rng.integers(0, 255 if fmt == "e8m0" else 0x7F, size=(R, D // blk)).astype(np.uint8)  # all finite codes
        s[:3, 0] = [0, 1, 254] if fmt == "e8m0" else [0, 1, 0x7E]
    ids = rng.integers(row_start - 30, row_start + R + 30, size=(T, stride)).astype(np.int64)
    if id_bytes == 8:
        ids[0, :3] = [-(2 ** 62), 2 ** 62, row_start + R]
    else:
        ids = ids.astype(np.int32)
        ids[0, :3] = [-(2 ** 31), 2 ** 31 - 1, row_start + R]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu_device)
    f8 = torch.empty((T, C, D), dtype=torch.uint8, device=gpu_device)
    sc = torch.empty((T, C, D // blk), dtype=torch.float32 if fmt == "fp32" else torch.uint8, device=gpu_device)
    out = g.engram_gather_dequant_fmt(dev(ids), dev(w), dev(s), fmt, blk, row_start, n_cols=C, out_fp8=f8,
                                      out_scale=sc)
    torch.cuda.synchronize()
    want, want8, wants = oracle.gather_dequant_fmt(ids, w, s, fmt, row_start=row_start, block_size=blk, n_cols=C,
                                                   want_raw=True)
    np.testing.assert_array_equal(bits(out), want)
    np.testing.assert_array_equal(f8.cpu().numpy(), want8)
    np.testing.assert_array_equal(sc.cpu().numpy(), wants)


@pytest.mark.parametrize("cfg_index,fmt", [(2, "e8m0"), (3, "e8m0"), (3, "e4m3")])
def test_gather_fmt_workload(gpu_device, cfg_index, fmt):
    """A workload's full-size table with one-byte scales (derived on the device from its seeded float32
    scales), int32 ids from engram_hash_i32: sampled tokens (every 256-token tile) against the oracle."""
    import torch

    import gram_hash_embedding_amd as g
    import synth.device as sd

    cfg = synth.CONFIGS[cfg_index]
    blk = 32 if fmt == "e8m0" else 16
    hi = synth.hash_inputs(cfg)
    B, L = hi.input_ids.shape
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(gpu_device)
    cache = torch.zeros((B, L), dtype=torch.int64, device=gpu_device)
    ids32 = g.engram_hash(t(hi.input_ids), 0, None if hi.token_mask is None else t(hi.token_mask),
                          t(hi.token_map), cache, t(hi.multipliers), t(hi.primes), t(hi.offsets), cfg.pad_id,
                          synth.DEAD, int32_ids=True)
    ids = oracle.hash(hi.input_ids, 0, hi.token_mask, hi.token_map, np.zeros((B, L), np.int64), hi.multipliers,
                      hi.primes, hi.offsets, cfg.pad_id, synth.DEAD)
    T, C, D = cfg.tokens, cfg.n_hash_cols, cfg.head_dim
    e = cfg.n_layers - 1
    R = cfg.rows_alloc[e]
    w_dev, s_dev = sd.device_table(synth.table_seed(cfg, e), R, D, blk, gpu_device)
    sb_dev = sd.device_scale_bytes(s_dev, fmt)
    del s_dev
    torch.cuda.empty_cache()
    out = g.engram_gather_dequant_fmt(ids32, w_dev, sb_dev, fmt, blk, layer=e)
    torch.cuda.synchronize()
    sample = sample_tokens(T, 4096, cfg_index, L=L, mask=hi.token_mask)
    got = bits(out.view(T, C, D)[torch.from_numpy(sample).to(gpu_device)])
    lid = ids.reshape(T, cfg.n_layers, C)[sample, e]
    cw, cs, remap = compact_rows(lid, R, synth.table_seed(cfg, e), D, blk)
    want = oracle.gather_dequant_fmt(remap, cw, synth.scale_bytes(cs, fmt), fmt, block_size=blk)
    np.testing.assert_array_equal(got, want)
    del w_dev, sb_dev, out
    torch.cuda.empty_cache()
