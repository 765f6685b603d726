"""Shared helpers of the GPU parity tests (no GPU work at import)."""
from __future__ import annotations

import numpy as np

# floating-point bar for the bf16-MFMA projection and the gate dot: |got - want| <= ATOL + RTOL * |want|
RTOL = 2e-2
ATOL = 1e-3


def assert_close(got, want, rtol=RTOL, atol=ATOL, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    err = np.abs(got - want)
    lim = atol + rtol * np.abs(want)
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: got {got[i]!r} "
                             f"want {want[i]!r}")


def bits(t) -> np.ndarray:
    """uint16 host copy of a bf16 (or uint16/int16) tensor."""
    import torch

    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint16)


def bf16_tensor(bits_arr, device):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits_arr, dtype=np.uint16).view(np.int16)).to(device).view(torch.bfloat16)


def sample_tokens(T: int, n: int, seed: int, L: int = None, mask=None, extra=()) -> np.ndarray:
    """Sorted token indices: the first and last tokens, tile edges of 256, the first three
    positions of each sequence and the three after every masked span, plus random others."""
    rng = np.random.default_rng(seed)
    pick = {0, T - 1, min(255, T - 1), min(256, T - 1), max(0, T - 256), max(0, T - 257)}
    pick.update(int(e) for e in extra if 0 <= e < T)
    if L is not None:
        B = T // L
        for b in range(min(B, 8)):
            pick.update(b * L + i for i in range(min(3, L)))
        if mask is not None:
            m = np.asarray(mask).reshape(B, L)
            ends = np.argwhere((m[:, :-1] == 0) & (m[:, 1:] == 1))
            for b, l in ends[:32]:
                pick.update(int(b * L + l + 1 + i) for i in range(3) if l + 1 + i < L)
    while len(pick) < min(n, T):
        pick.add(int(rng.integers(0, T)))
    return np.array(sorted(pick), dtype=np.int64)


def compact_rows(ids: np.ndarray, R: int, table_seed: int, D: int, blk: int):
    """Host copy of the table rows `ids` reach, with ids remapped into it (synth.compact_table)."""
    import synth

    return synth.compact_table(ids, R, table_seed, D, blk)
