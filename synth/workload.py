"""Device-resident synthetic workloads: every input of the Engram forward path
for one configuration, drawn from the seeded generators of this package and
placed in GPU memory (tables filled on the GPU by the counter-based fill
kernel).  Used by the GPU tests and the benchmark."""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from . import (DEAD, EngramConfig, hash_inputs, qk_weights, residual, table_rows_alloc, table_seed, wkv_weight)
from . import device as synth_device


@dataclasses.dataclass
class Workload:
    cfg: EngramConfig
    host: object                    # synth.HashInputs (numpy)
    input_ids: "torch.Tensor"       # int64 [B, L_total] on the GPU
    token_mask: Optional["torch.Tensor"]
    fwd: object                     # gram_hash_embedding_amd.forward.EngramForward
    x: List["torch.Tensor"]         # residual stream(s) [T, hc, dim] bf16 (decode: one per step)
    cache_shape: tuple

    @property
    def T(self) -> int:
        return self.cfg.tokens

    def reset_cache(self):
        self.fwd.state.cache.zero_()


def build(cfg: EngramConfig, device="cuda", x_steps: int = 1, full_range: bool = False,
          n_layers: Optional[int] = None, packed: bool = False, fp8: bool = False) -> Workload:
    """`packed`: also give every layer its table in the packed layout (engram_pack_table); `fp8`: also its wkv
    weight in the fp8 block-scaled form (engram_mx_quant of the bf16 weight: the stand-in for released fp8
    weights)."""
    import torch

    from gram_hash_embedding_amd import engram_mx_quant, engram_pack_table
    from gram_hash_embedding_amd.forward import EngramForward, HashState, LayerWeights

    hi = hash_inputs(cfg, full_range_multipliers=full_range)
    E = cfg.n_layers if n_layers is None else n_layers
    L_total = hi.input_ids.shape[1]
    cache = torch.zeros((cfg.batch, L_total), dtype=torch.int64, device=device)
    state = HashState(
        token_map=torch.from_numpy(hi.token_map).to(device),
        cache=cache,
        multipliers=torch.from_numpy(hi.multipliers[:E].copy()).to(device),
        primes=torch.from_numpy(hi.primes[:E].copy()).to(device),
        offsets=torch.from_numpy(hi.offsets[:E].copy()).to(device),
        pad_id=cfg.pad_id, dead=DEAD)
    layers = []
    rows = table_rows_alloc(cfg)
    for e in range(E):
        w, s = synth_device.device_table(table_seed(cfg, e), rows[e], cfg.head_dim, cfg.block_size, device)
        q, k = qk_weights(cfg, e, device=device)
        pk = engram_pack_table(w, s, cfg.block_size) if packed else None
        wkv = wkv_weight(cfg, e, device=device)
        wmx = engram_mx_quant(wkv) if fp8 and cfg.K % 128 == 0 else None
        layers.append(LayerWeights(weight=w, scale=s, wkv=wkv, q_weight=q, k_weight=k, block_size=cfg.block_size,
                                   packed=pk, wkv_mx=wmx))
    fwd = EngramForward(state, layers, cfg.eps)
    ids = torch.from_numpy(hi.input_ids).to(device)
    mask = None if hi.token_mask is None else torch.from_numpy(hi.token_mask).to(device)
    xs = [residual(cfg, device=device, step=s) for s in range(x_steps)]
    return Workload(cfg, hi, ids, mask, fwd, xs, tuple(cache.shape))


def bf16_bits(t) -> np.ndarray:
    """Host uint16 view of a bf16 tensor."""
    import torch

    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


__all__ = ["Workload", "build", "bf16_bits"]
