"""engram_hash on the GPU against the oracle: bit-exact ids and cache contents."""
import numpy as np
import pytest

import oracle
import synth
from tests.test_oracle_hash import _case

pytestmark = pytest.mark.gpu


def _gpu_hash(dev, ids, start_pos, mask, tmap, cache, mult, primes, offs, pad=2, dead=-1):
    import torch

    import gram_hash_embedding_amd as g

    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = g.engram_hash(t(ids), start_pos, t(mask), t(tmap), cache, t(mult), t(primes), t(offs), pad, dead)
    return out.cpu().numpy()


@pytest.mark.parametrize("full_range", [False, True])
# ids per token E*(N-1)*H from 1 to 1008: up to 256 a lane keeps one column for the tile (256: one token
# row per step), above that one id per lane and step
@pytest.mark.parametrize("B,L,E,N,H", [(3, 77, 2, 4, 2), (1, 1, 1, 2, 1), (2, 130, 3, 5, 3), (4, 64, 1, 8, 2),
                                       (5, 33, 2, 3, 8), (2, 70, 2, 5, 32), (2, 70, 2, 4, 64), (1, 70, 8, 8, 18)])
def test_hash_small_shapes(gpu_device, full_range, B, L, E, N, H):
    import torch

    ids, mask, tmap, mult, primes, offs = _case(B * 100 + L + N, B=B, L=L, E=E, N=N, H=H, full_range=full_range,
                                                mask_frac=0.15 if L >= 8 else 0.0)
    ids[0, 0] = 10**9  # an out-of-vocabulary id counts as masked
    want = oracle.hash(ids, 0, mask, tmap, np.zeros((B, L + 3), np.int64), mult, primes, offs, 2, -1)
    cache = torch.full((B + 1, L + 3), 5, dtype=torch.int64, device=gpu_device)
    got = _gpu_hash(gpu_device, ids, 0, mask, tmap, cache, mult, primes, offs)
    np.testing.assert_array_equal(got, want)
    comp = np.where(tmap[np.clip(ids, 0, len(tmap) - 1)] >= 0, tmap[np.clip(ids, 0, len(tmap) - 1)], 0)
    live = (ids >= 0) & (ids < len(tmap))
    if mask is not None:
        live &= mask == 1
    np.testing.assert_array_equal(cache[:B, :L].cpu().numpy(), np.where(live, comp, -1))
    assert (cache[B].cpu().numpy() == 5).all() and (cache[:, L:].cpu().numpy() == 5).all()


def test_hash_chunked_on_gpu_equals_one_shot(gpu_device):
    import torch

    ids, mask, tmap, mult, primes, offs = _case(4242, B=3, L=300, E=2, N=4, H=8, full_range=True, mask_frac=0.1)
    want = oracle.hash(ids, 0, mask, tmap, np.zeros((3, 300), np.int64), mult, primes, offs, 2, -1)
    cache = torch.zeros((3, 300), dtype=torch.int64, device=gpu_device)
    parts = []
    cuts = [0, 100, 101, 102, 103, 200, 257, 300]
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        parts.append(_gpu_hash(gpu_device, ids[:, lo:hi], lo, mask[:, lo:hi], tmap, cache, mult, primes, offs))
    np.testing.assert_array_equal(np.concatenate(parts, axis=1), want)


@pytest.mark.parametrize("cfg_index", [1, 2, 3, 5])
def test_hash_config_full_array(gpu_device, cfg_index):
    import torch

    import gram_hash_embedding_amd as g

    cfg = synth.CONFIGS[cfg_index]
    hi = synth.hash_inputs(cfg)
    B, L = hi.input_ids.shape
    want = oracle.hash(hi.input_ids, 0, hi.token_mask, hi.token_map, np.zeros((B, L), np.int64), hi.multipliers,
                       hi.primes, hi.offsets, cfg.pad_id, synth.DEAD)
    cache = torch.zeros((B, L), dtype=torch.int64, device=gpu_device)
    got = _gpu_hash(gpu_device, hi.input_ids, 0, hi.token_mask, hi.token_map, cache, hi.multipliers, hi.primes,
                    hi.offsets, cfg.pad_id, synth.DEAD)
    np.testing.assert_array_equal(got, want)
    assert got.shape == (B, L, cfg.n_layers, cfg.n_hash_cols)
    rows = synth.rows_used(hi.primes)
    for e in range(cfg.n_layers):
        assert got[:, :, e].min() >= 0 and got[:, :, e].max() < rows[e]
    del g


def test_hash_decode_steps_match_oracle(gpu_device):
    """Decode-style workload: prefill 4096 positions of 256 sequences, then 64 steps of one token each."""
    import torch

    cfg = synth.CONFIGS[4]
    hi = synth.hash_inputs(cfg)
    B, Ltot = hi.input_ids.shape
    P = cfg.start_pos
    host_cache = np.zeros((B, Ltot), np.int64)
    dev_cache = torch.zeros((B, Ltot), dtype=torch.int64, device=gpu_device)
    args = (hi.token_map, None, hi.multipliers, hi.primes, hi.offsets)
    want = oracle.hash(hi.input_ids[:, :P], 0, None, hi.token_map, host_cache, hi.multipliers, hi.primes, hi.offsets,
                       cfg.pad_id, synth.DEAD)
    got = _gpu_hash(gpu_device, hi.input_ids[:, :P], 0, None, hi.token_map, dev_cache, hi.multipliers, hi.primes,
                    hi.offsets)
    np.testing.assert_array_equal(got, want)
    for s in range(cfg.decode_steps):
        sl = hi.input_ids[:, P + s:P + s + 1]
        want = oracle.hash(sl, P + s, None, hi.token_map, host_cache, hi.multipliers, hi.primes, hi.offsets,
                           cfg.pad_id, synth.DEAD)
        got = _gpu_hash(gpu_device, sl, P + s, None, hi.token_map, dev_cache, hi.multipliers, hi.primes, hi.offsets)
        np.testing.assert_array_equal(got, want, err_msg=f"decode step {s}")
    np.testing.assert_array_equal(dev_cache.cpu().numpy(), host_cache)
    del args


def test_hash_rejects_small_cache_and_zero_tokens(gpu_device):
    import torch

    import gram_hash_embedding_amd as g

    ids, _, tmap, mult, primes, offs = _case(1, B=2, L=16, E=1, N=4, H=2)
    t = lambda a: torch.from_numpy(a).to(gpu_device)
    cache = torch.zeros((2, 15), dtype=torch.int64, device=gpu_device)
    with pytest.raises(g.EngramError) as ei:
        g.engram_hash(t(ids), 0, None, t(tmap), cache, t(mult), t(primes), t(offs), 2)
    assert ei.value.status == g.ENGRAM_ERANGE
    empty = torch.zeros((2, 0), dtype=torch.int64, device=gpu_device)
    out = g.engram_hash(empty, 0, None, t(tmap), cache, t(mult), t(primes), t(offs), 2)
    assert out.shape == (2, 0, 1, 6)
