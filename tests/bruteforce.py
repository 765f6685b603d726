"""Brute-force n-gram hash ids with Python integers, for tiny inputs.

Written straight from the description of the hash on the DeepSeek V4.1
stack-hashes page, in a different form from the oracle: every n-gram's hash is
rebuilt from scratch (no running value), blocking is "some position between
the lookback slot and the current token is masked" (not a carried flag), and
the int64 wrap and floor modulo are explicit big-integer arithmetic.
"""
from __future__ import annotations


def wrap64(x: int) -> int:
    """Two's-complement int64 value of the integer x."""
    return ((x + 2**63) % 2**64) - 2**63


def window(comp, live, p, N, pad):
    """Slot s (0..N-1) of the lookback window at position p.

    comp[q]: compressed id at position q; live[q]: False where position q is
    masked.  Slot s holds comp[p-s] unless p-s < 0 or some position in
    [p-s, p] is masked; then it holds the pad id.
    """
    out = []
    for s in range(N):
        q = p - s
        if q < 0 or not all(live[r] for r in range(q, p + 1)):
            out.append(pad)
        else:
            out.append(comp[q])
    return out


def ids_at(comp, live, p, multipliers, primes, offsets, pad):
    """Hash ids [E][C] at position p of one sequence.

    multipliers [E][N], primes [E][N-1][H], offsets [E][C] as nested lists.
    Column (n-2)*H + h holds the n-gram (n = 2..N) hash modulo its prime.
    """
    E, N = len(multipliers), len(multipliers[0])
    H = len(primes[0][0])
    t = window(comp, live, p, N, pad)
    res = []
    for e in range(E):
        row = []
        for n in range(2, N + 1):
            x = 0
            for s in range(n):
                x ^= wrap64(t[s] * multipliers[e][s])
            for h in range(H):
                prime = primes[e][n - 2][h]
                row.append((x % prime) + offsets[e][(n - 2) * H + h])  # Python % is floor modulo
        res.append(row)
    return res


def hash_all(input_ids, token_mask, token_map, multipliers, primes, offsets, pad):
    """Hash ids [B][L][E][C] over whole sequences (positions 0..L-1), nested lists.

    An input id outside the vocabulary counts as masked (the pages would raise;
    this is the library's stated reading).
    """
    B, L = len(input_ids), len(input_ids[0])
    V = len(token_map)
    out = []
    for b in range(B):
        comp, live = [], []
        for l in range(L):
            i = input_ids[b][l]
            ok = 0 <= i < V and (token_mask is None or bool(token_mask[b][l]))
            comp.append(token_map[i] if 0 <= i < V else None)
            live.append(ok)
        out.append([ids_at(comp, live, p, multipliers, primes, offsets, pad) for p in range(L)])
    return out
