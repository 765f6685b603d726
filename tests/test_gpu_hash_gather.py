"""engram_hash_gather_packed on the GPU against the oracle: the cache, the ids (when stored) and every
layer's gathered bf16 rows, bit-exact -- the oracle's hash, then its gather + dequant per layer."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bits
from tests.test_oracle_hash import _case

pytestmark = pytest.mark.gpu


def _same_bits(got, want, what):
    gf, wf = oracle.bf16_bits_to_float(got), oracle.bf16_bits_to_float(want)
    np.testing.assert_array_equal(np.isnan(gf), np.isnan(wf), err_msg=what)
    ok = ~np.isnan(wf)
    np.testing.assert_array_equal(got[ok], want[ok], err_msg=what)


class _Tables:
    """Per layer: a seeded table of R_e rows (generated on the GPU and packed there) standing for rows
    [row_start_e, row_start_e + R_e) of the layer's id range; the oracle sees the rows the ids reach."""

    def __init__(self, dev, primes, D, blk, seed, short=100):
        import synth.device as sd

        import gram_hash_embedding_amd as g

        self.seed, self.D, self.blk = seed, D, blk
        self.packed, self.R, self.row_start = [], [], []
        for e in range(primes.shape[0]):
            span = int(primes[e].sum())  # the layer's ids lie in [0, span)
            R = max(1, span - 2 * short)
            w, s = sd.device_table(seed + e, R, D, blk, dev)
            self.packed.append(g.engram_pack_table(w, s, blk))
            del w, s
            self.R.append(R)
            self.row_start.append(short + 7 * e)  # ids below it, and the top ~short ids, are outside the share

    def want(self, ids):
        """The oracle's rows per layer for ids [B, L, E, C]: a list of bf16 bits [B*L, C, D]."""
        B, L, E, C = ids.shape
        res = []
        for e in range(E):
            local = ids[:, :, e].reshape(B * L, C) - self.row_start[e]
            cw, cs, remap = synth.compact_table(local, self.R[e], self.seed + e, self.D, self.blk)
            res.append(oracle.gather_dequant(remap, cw, cs, block_size=self.blk))
        return res


def _t(dev, a):
    import torch

    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _fused(dev, tabs, ids, start_pos, mask, tmap, cache, mult, primes, offs, blk, store_ids=True, pad=2, dead=-1):
    import torch

    import gram_hash_embedding_amd as g

    B, L = ids.shape
    E, C = offs.shape
    hid = torch.full((B, L, E, C), -7, dtype=torch.int64, device=dev) if store_ids else None
    outs, _ = g.engram_hash_gather_packed(_t(dev, ids), start_pos, _t(dev, mask), _t(dev, tmap), cache, _t(dev, mult),
                                          _t(dev, primes), _t(dev, offs), pad, tabs.packed, blk, tabs.row_start, dead,
                                          hash_ids=hid)
    return [bits(o) for o in outs], (None if hid is None else hid.cpu().numpy())


# ids per token E*C from 1 to 1008 (above 256 the hash's second phase takes one id per lane and step; the
# tile then shrinks so its ids fit the LDS); every row width; masks; bounded and full-range multipliers
@pytest.mark.parametrize("B,L,E,N,H,D,blk,full_range,store", [
    (3, 77, 2, 4, 2, 64, 32, False, True), (1, 1, 1, 2, 1, 32, 32, True, True), (2, 130, 3, 5, 3, 128, 64, True, False),
    (4, 64, 2, 4, 8, 64, 16, False, False), (2, 70, 2, 5, 32, 256, 32, False, True),
    (1, 70, 8, 8, 18, 32, 16, True, True), (300, 1, 2, 4, 8, 64, 32, False, True)])
def test_hash_gather_matches_oracle(gpu_device, B, L, E, N, H, D, blk, full_range, store):
    import torch

    ids, mask, tmap, mult, primes, offs = _case(B * 100 + L + N + D, B=B, L=L, E=E, N=N, H=H, full_range=full_range,
                                                mask_frac=0.15 if L >= 8 else 0.0)
    ids[0, 0] = 10**9  # an out-of-vocabulary id counts as masked
    tabs = _Tables(gpu_device, primes, D, blk, seed=B + L + D)
    want_ids = oracle.hash(ids, 0, mask, tmap, np.zeros((B, L + 3), np.int64), mult, primes, offs, 2, -1)
    cache = torch.full((B + 1, L + 3), 5, dtype=torch.int64, device=gpu_device)
    rows, got_ids = _fused(gpu_device, tabs, ids, 0, mask, tmap, cache, mult, primes, offs, blk, store_ids=store)
    if store:
        np.testing.assert_array_equal(got_ids, want_ids)
    want_rows = tabs.want(want_ids)
    for e in range(E):
        _same_bits(rows[e], want_rows[e], f"layer {e}")
    # both sides of the table share occur, so zero rows are exercised
    local = want_ids - np.array(tabs.row_start)[None, None, :, None]
    outside = (local < 0) | (local >= np.array(tabs.R)[None, None, :, None])
    if B * L * E * (N - 1) * H > 200:
        assert outside.any() and (~outside).any()
    # the cache as engram_hash leaves it
    ref_cache = torch.full((B + 1, L + 3), 5, dtype=torch.int64, device=gpu_device)
    import gram_hash_embedding_amd as g

    g.engram_hash(_t(gpu_device, ids), 0, _t(gpu_device, mask), _t(gpu_device, tmap), ref_cache, _t(gpu_device, mult),
                  _t(gpu_device, primes), _t(gpu_device, offs), 2, -1)
    np.testing.assert_array_equal(cache.cpu().numpy(), ref_cache.cpu().numpy())


def test_hash_gather_chunked_decode_steps(gpu_device):
    """A 50-token prefill, then eight one-token steps per sequence: every call against the oracle's hash
    of the whole sequence and its rows (the cache carries the history between calls)."""
    import torch

    B, Ltot, P, blk, D = 5, 58, 50, 32, 64
    ids, mask, tmap, mult, primes, offs = _case(777, B=B, L=Ltot, E=2, N=4, H=8, full_range=True, mask_frac=0.1)
    tabs = _Tables(gpu_device, primes, D, blk, seed=31)
    want_all = oracle.hash(ids, 0, mask, tmap, np.zeros((B, Ltot), np.int64), mult, primes, offs, 2, -1)
    cache = torch.zeros((B, Ltot), dtype=torch.int64, device=gpu_device)
    cuts = [(0, P)] + [(P + i, P + i + 1) for i in range(Ltot - P)]
    for lo, hi in cuts:
        rows, got_ids = _fused(gpu_device, tabs, ids[:, lo:hi], lo, mask[:, lo:hi], tmap, cache, mult, primes, offs,
                               blk)
        np.testing.assert_array_equal(got_ids, want_all[:, lo:hi], err_msg=f"ids, positions [{lo}, {hi})")
        want_rows = tabs.want(want_all[:, lo:hi])
        for e in range(2):
            _same_bits(rows[e], want_rows[e], f"layer {e}, positions [{lo}, {hi})")


def test_hash_gather_equals_the_two_entry_points(gpu_device):
    """On the decode shape (256 sequences, 2 layers, 24 columns, D = 64): the fused call's rows are those of
    engram_hash followed by engram_gather_dequant_packed, bit for bit, on ids that reach both ends of the
    tables."""
    import torch

    import gram_hash_embedding_amd as g

    B, L, blk, D = 256, 1, 32, 64
    ids, _, tmap, mult, primes, offs = _case(4096, B=B, L=L + 40, E=2, N=4, H=8, full_range=True)
    tabs = _Tables(gpu_device, primes, D, blk, seed=5)
    args = lambda cache: (_t(gpu_device, ids[:, 40:]), 40, None, _t(gpu_device, tmap), cache, _t(gpu_device, mult),
                          _t(gpu_device, primes), _t(gpu_device, offs), 2)
    c1 = torch.zeros((B, 41), dtype=torch.int64, device=gpu_device)
    c2 = torch.zeros((B, 41), dtype=torch.int64, device=gpu_device)
    g.engram_hash(_t(gpu_device, ids[:, :40]), 0, None, _t(gpu_device, tmap), c1, _t(gpu_device, mult),
                  _t(gpu_device, primes), _t(gpu_device, offs), 2)
    c2.copy_(c1)
    hid = g.engram_hash(*args(c1))
    sep = [g.engram_gather_dequant_packed(hid, tabs.packed[e], blk, tabs.row_start[e], layer=e) for e in range(2)]
    outs, _ = g.engram_hash_gather_packed(*args(c2), tabs.packed, blk, tabs.row_start)
    for e in range(2):
        np.testing.assert_array_equal(bits(outs[e]), bits(sep[e]), err_msg=f"layer {e}")
    np.testing.assert_array_equal(c1.cpu().numpy(), c2.cpu().numpy())
