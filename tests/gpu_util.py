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


def bf16_ulp(v) -> np.ndarray:
    """One unit in the last place of bf16 at each |v| (the spacing of bf16 values around it)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(np.maximum(e, -126.0) - 7.0), 2.0 ** -133)


def assert_output_close(got_bits, out_want, value_want, x_bits=None, mask=None, what=""):
    """The output stream h + gate * value against the oracle's pipeline.  The device's bf16 value may sit one
    bf16 ulp from the oracle's (its fp32 sum and the oracle's float64 sum can round to neighbouring bf16
    values), and h + gate * value can cancel, so besides the gate bar (1e-3 + 2e-2 |out|) each element may
    differ by |gate| <= 1 times one ulp of its value element."""
    import oracle

    got = oracle.bf16_bits_to_float(got_bits).astype(np.float64)
    v = np.asarray(value_want, dtype=np.float64)[:, None, :]
    assert_close(got, out_want, atol=ATOL + bf16_ulp(v), what=what)


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


def sample_tokens(T: int, n: int, seed: int, L: int = None, mask=None, extra=(), tile: int = 256) -> np.ndarray:
    """Sorted token indices: the first and last tokens; the first and last token and one random token of
    every `tile`-token block (every M tile of the projection, the ragged last one included); the first three
    positions of every sequence and the three after every masked span; then random others up to n."""
    rng = np.random.default_rng(seed)
    pick = {0, T - 1}
    pick.update(int(e) for e in extra if 0 <= e < T)
    for t0 in range(0, T, tile):
        t1 = min(T, t0 + tile)
        pick.update((t0, t1 - 1, int(rng.integers(t0, t1))))
    if L is not None:
        B = T // L
        for b in range(B):
            pick.update(b * L + i for i in range(min(3, L)))
        if mask is not None:
            m = np.asarray(mask).reshape(B, L)
            ends = np.argwhere((m[:, :-1] == 0) & (m[:, 1:] == 1))
            for b, l in ends:
                pick.update(int(b * L + l + 1 + i) for i in range(3) if l + 1 + i < L)
    while len(pick) < min(n, T):
        pick.add(int(rng.integers(0, T)))
    return np.array(sorted(pick), dtype=np.int64)


def compact_rows(ids: np.ndarray, R: int, table_seed: int, D: int, blk: int):
    """Host copy of the table rows `ids` reach, with ids remapped into it (synth.compact_table)."""
    import synth

    return synth.compact_table(ids, R, table_seed, D, blk)


def mx_scales_rowmajor(scale_dev, rows: int, K: int) -> np.ndarray:
    """An MX scale tensor in the library's layout [K/128, rows4, 4] -> uint8 [rows, K/32] (the oracle's)."""
    s = scale_dev.cpu().numpy().reshape(K // 128, -1, 4)
    return np.ascontiguousarray(s.transpose(1, 0, 2).reshape(-1, K // 32)[:rows])
