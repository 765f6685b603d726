"""Pins for the oracle's hash (DeepSeek V4.1 pages, stack-hashes page: the
engram hash module's forward, and the engram fields of the model config).

The oracle is checked against a Python big-integer brute force written from
the description, against closed forms, and against invariants the pages
state in comments and docstrings.
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tests import bruteforce

HERE = os.path.dirname(os.path.abspath(__file__))
DEAD = synth.DEAD


def _case(seed, B, L, E, N, H, V=1000, Vc=500, full_range=False, mask_frac=0.0, prime_base=1600):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, V, size=(B, L), dtype=np.int64)
    tmap = rng.integers(0, Vc, size=V, dtype=np.int64)
    mult = synth.multipliers(seed + 1, E, N, Vc, full_range=full_range)
    primes = synth.layout_primes(prime_base, E, N, H)
    offs = synth.layout_offsets(primes)
    mask = None
    if mask_frac > 0:
        mask = synth.mask_spans(seed + 2, B, L, mask_frac, min_len=1, max_len=6)
    return ids, mask, tmap, mult, primes, offs


def _oracle_oneshot(ids, mask, tmap, mult, primes, offs, pad=2, dead=DEAD, cache=None):
    B, L = ids.shape
    if cache is None:
        cache = np.zeros((B, L), dtype=np.int64)
    return oracle.hash(ids, 0, mask, tmap, cache, mult, primes, offs, pad, dead)


def _brute(ids, mask, tmap, mult, primes, offs, pad=2):
    return np.array(bruteforce.hash_all(ids.tolist(), None if mask is None else mask.tolist(), tmap.tolist(),
                                        mult.tolist(), primes.tolist(), offs.tolist(), pad), dtype=np.int64)


@pytest.mark.parametrize("full_range", [False, True])
@pytest.mark.parametrize("N,H,E", [(4, 2, 2), (2, 3, 1), (3, 1, 2), (5, 2, 1)])
def test_hash_matches_bruteforce(full_range, N, H, E):
    case = _case(11 + N * 7 + H, B=3, L=40, E=E, N=N, H=H, full_range=full_range, mask_frac=0.2)
    got = _oracle_oneshot(*case)
    want = _brute(*case)
    assert got.shape == (3, 40, E, (N - 1) * H)
    np.testing.assert_array_equal(got, want)


def test_full_range_multipliers_reach_negative_running_values():
    # the full-range case must actually exercise wrap-around / negative XORs
    ids, mask, tmap, mult, primes, offs = _case(5, B=2, L=32, E=2, N=4, H=2, full_range=True)
    assert (mult < 0).any()
    got = _oracle_oneshot(ids, mask, tmap, mult, primes, offs)
    np.testing.assert_array_equal(got, _brute(ids, mask, tmap, mult, primes, offs))


def test_ids_land_in_their_column_range():
    ids, mask, tmap, mult, primes, offs = _case(3, B=2, L=64, E=2, N=4, H=3, full_range=True, mask_frac=0.1)
    got = _oracle_oneshot(ids, mask, tmap, mult, primes, offs)
    P = primes.reshape(2, -1)
    lo = offs[None, None]
    assert ((got >= lo) & (got < lo + P[None, None])).all()


def test_masked_positions_hash_the_all_pad_window():
    pad = 2
    ids, mask, tmap, mult, primes, offs = _case(7, B=3, L=64, E=2, N=4, H=2, mask_frac=0.25)
    got = _oracle_oneshot(ids, mask, tmap, mult, primes, offs, pad=pad)
    # closed form of the all-pad window: (XOR_s pad*m[e,s] for s < n) mod P + O
    E, N = mult.shape
    H = primes.shape[2]
    allpad = np.empty((E, (N - 1) * H), dtype=np.int64)
    for e in range(E):
        x = 0
        for n in range(2, N + 1):
            x = 0
            for s in range(n):
                x ^= bruteforce.wrap64(pad * int(mult[e, s]))
            for h in range(H):
                allpad[e, (n - 2) * H + h] = x % int(primes[e, n - 2, h]) + offs[e, (n - 2) * H + h]
    where = mask == 0
    assert where.sum() > 10
    np.testing.assert_array_equal(got[where], np.broadcast_to(allpad, got[where].shape))


def test_token_after_span_equals_sequence_start():
    # the first token after a masked span sees only pads behind it, like position 0
    ids, mask, tmap, mult, primes, offs = _case(9, B=2, L=80, E=1, N=4, H=2, mask_frac=0.2)
    got = _oracle_oneshot(ids, mask, tmap, mult, primes, offs)
    checked = 0
    for b in range(2):
        for p in range(1, 80):
            if mask[b, p - 1] == 0 and mask[b, p] == 1:
                ref_ids = ids[b:b + 1, p:p + 1]
                ref = _oracle_oneshot(ref_ids, None, tmap, mult, primes, offs)
                np.testing.assert_array_equal(got[b, p], ref[0, 0])
                checked += 1
    assert checked >= 2


def test_chunked_calls_equal_one_shot():
    ids, mask, tmap, mult, primes, offs = _case(13, B=3, L=50, E=2, N=4, H=2, full_range=True, mask_frac=0.2)
    want = _oracle_oneshot(ids, mask, tmap, mult, primes, offs)
    for cuts in ([0, 17, 18, 19, 50], [0, 1, 2, 3, 4, 5, 50], [0, 45] + list(range(46, 51))):
        cache = np.full((4, 64), 12345, dtype=np.int64)  # larger than needed, junk content
        parts = []
        for lo, hi in zip(cuts[:-1], cuts[1:]):
            parts.append(oracle.hash(ids[:, lo:hi], lo, mask[:, lo:hi], tmap, cache, mult, primes, offs, 2, DEAD))
        np.testing.assert_array_equal(np.concatenate(parts, axis=1), want)


def test_dead_value_and_cache_initial_contents_do_not_matter():
    ids, mask, tmap, mult, primes, offs = _case(17, B=2, L=40, E=2, N=4, H=2, mask_frac=0.2)
    a = _oracle_oneshot(ids, mask, tmap, mult, primes, offs, dead=-1)
    b = _oracle_oneshot(ids, mask, tmap, mult, primes, offs, dead=-(2**62))
    c = _oracle_oneshot(ids, mask, tmap, mult, primes, offs, cache=np.full((2, 40), 777, dtype=np.int64))
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, c)


def test_cache_holds_compressed_ids_and_dead():
    ids, mask, tmap, mult, primes, offs = _case(19, B=2, L=40, E=1, N=4, H=2, mask_frac=0.2)
    cache = np.zeros((3, 48), dtype=np.int64)
    oracle.hash(ids[:, :30], 0, mask[:, :30], tmap, cache, mult, primes, offs, 2, DEAD)
    oracle.hash(ids[:, 30:], 30, mask[:, 30:], tmap, cache, mult, primes, offs, 2, DEAD)
    want = np.where(mask == 1, tmap[ids], DEAD)
    np.testing.assert_array_equal(cache[:2, :40], want)
    assert (cache[2] == 0).all() and (cache[:2, 40:] == 0).all()


def test_out_of_vocab_id_counts_as_masked():
    ids, _, tmap, mult, primes, offs = _case(23, B=1, L=20, E=1, N=4, H=2)
    bad = ids.copy()
    bad[0, 7] = 10**6
    bad[0, 12] = -5
    m = np.ones_like(ids, dtype=np.uint8)
    m[0, 7] = 0
    m[0, 12] = 0
    np.testing.assert_array_equal(_oracle_oneshot(bad, None, tmap, mult, primes, offs),
                                  _oracle_oneshot(ids, m, tmap, mult, primes, offs))


def test_lookback_locality_moves_only_longer_ngrams():
    # changing the token 3 back changes only the 4-gram columns at that position
    ids, _, tmap, mult, primes, offs = _case(29, B=1, L=20, E=2, N=4, H=2)
    tmap = np.arange(1000, dtype=np.int64) % 500
    ids2 = ids.copy()
    ids2[0, 10] = (ids[0, 10] + 1) % 500
    a = _oracle_oneshot(ids, None, tmap, mult, primes, offs)
    b = _oracle_oneshot(ids2, None, tmap, mult, primes, offs)
    H = 2
    # position 13 sees the change at lookback 3: only 4-gram columns (n=4 -> c = 2H..3H-1) differ
    diff = a[0, 13] != b[0, 13]
    assert not diff[:, : 2 * H].any() and diff[:, 2 * H:].all()
    # position 11 sees it at lookback 1: 2-, 3- and 4-gram columns all differ
    assert (a[0, 11] != b[0, 11]).all()
    # positions before 10 and from 14 on are untouched
    np.testing.assert_array_equal(a[0, :10], b[0, :10])
    np.testing.assert_array_equal(a[0, 14:], b[0, 14:])


def test_unit_multipliers_reduce_to_xor_of_ids():
    # closed form with every multiplier 1: the n-gram hash is the XOR of the last n ids
    ids, _, tmap, _, primes, offs = _case(31, B=2, L=30, E=1, N=4, H=2)
    mult = np.ones((1, 4), dtype=np.int64)
    got = _oracle_oneshot(ids, None, tmap, mult, primes, offs)
    comp = tmap[ids]
    pad = 2
    for b in range(2):
        for p in range(30):
            t = [comp[b, p - s] if p - s >= 0 else pad for s in range(4)]
            for n in range(2, 5):
                x = 0
                for s in range(n):
                    x ^= int(t[s])
                for h in range(2):
                    c = (n - 2) * 2 + h
                    assert got[b, p, 0, c] == x % primes[0, n - 2, h] + offs[0, c]


def test_prime_layout_reproduces_released_table_sizes():
    # the released config's engram_num_embeddings are the sums of the layers' prime ranges
    cfg = json.load(open(os.path.join(HERE, "golden", "engram_config.json")))
    E = len(cfg["engram_layer_ids"])
    primes = synth.layout_primes(cfg["engram_vocab_size"], E, cfg["engram_max_ngram_size"], cfg["engram_n_heads"])
    assert synth.rows_used(primes) == cfg["engram_num_embeddings"]
    assert len(np.unique(primes)) == primes.size
    offs = synth.layout_offsets(primes)
    np.testing.assert_array_equal(offs[:, -1] + primes.reshape(E, -1)[:, -1], cfg["engram_num_embeddings"])


def test_tiny_config_layout():
    c = synth.CONFIGS[1]
    primes = synth.layout_primes(c.prime_base, c.n_layers, c.max_ngram_size, c.n_heads)
    assert primes.reshape(-1).tolist() == [1601, 1607, 1609, 1613, 1619, 1621]
    assert synth.layout_offsets(primes).reshape(-1).tolist() == [0, 1601, 3208, 4817, 6430, 8049]
    assert synth.rows_used(primes) == [9670]
