"""One Engram forward pass over the HIP entry points, with reusable buffers.

The order of the steps is that of the DeepSeek V4.1 "stack-hashes" page: the
model forward hashes once for all engram layers, then each engram layer
gathers its rows from its own slice of the ids, projects them with `wkv`
and forms the gate pre-activation against the residual stream -- or, with
`output=True`, the whole of Engram.forward: the gate, the token mask and the
residual add, which return the layer's new stream.  With `fused=True` the
projection and the gate pre-activation run as one entry point
(engram_wkv_gate: the keys are reduced inside the projection and never
stored) and the output, if asked for, comes from engram_gate_residual.  This
module only allocates outputs and workspace and calls the HIP entry points in
that order.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

from . import (engram_gate_dot, engram_gate_output, engram_gate_residual, engram_gather_dequant,
               engram_gather_dequant_packed, engram_gather_mx, engram_hash, engram_hash_gather_packed,
               engram_mx_quant, engram_wkv, engram_wkv_gate, engram_wkv_gate_layers,
               engram_wkv_gate_workspace_bytes, engram_wkv_mx, engram_wkv_mx_gate)


@dataclasses.dataclass
class HashState:
    """Device tensors of the hash module (all int64)."""

    token_map: "torch.Tensor"      # [vocab]
    cache: "torch.Tensor"          # [max_batch, max_seq]
    multipliers: "torch.Tensor"    # [E, N]
    primes: "torch.Tensor"         # [E, N-1, H]
    offsets: "torch.Tensor"        # [E, (N-1)*H]
    pad_id: int
    dead: int = -1


@dataclasses.dataclass
class LayerWeights:
    """One engram layer: its fp8 table (this GPU's rows), projection and gate weights."""

    weight: "torch.Tensor"         # uint8 / float8_e4m3fn [R, D]
    scale: "torch.Tensor"          # float32 [R, D/block_size]
    wkv: "torch.Tensor"            # bf16 [dim*(hc+1), C*D]
    q_weight: "torch.Tensor"       # bf16 [hc, dim]
    k_weight: "torch.Tensor"       # bf16 [hc, dim]
    block_size: int
    row_start: int = 0
    packed: "Optional[torch.Tensor]" = None  # uint8 [R, 2*D]: the same table as one record per row (engram_pack_table)
    # the wkv weight in the fp8 block-scaled (OCP MX) form: (E4M3 bytes [Nout, K], E8M0 scales), for fp8=True
    wkv_mx: "Optional[tuple]" = None


class EngramForward:
    """Runs hash -> (gather+dequant -> wkv -> gate dot | gate output) per layer on the current stream
    (or gather+dequant -> fused wkv + gate dot [-> gate residual])."""

    def __init__(self, state: HashState, layers: List[LayerWeights], eps: float):
        self.state = state
        self.layers = layers
        self.eps = eps
        self.E, self.N = state.multipliers.shape
        self.H = state.primes.shape[2]
        self.C = (self.N - 1) * self.H
        if len(layers) != self.E:
            raise ValueError("one LayerWeights per hashed engram layer")
        self._bufs = {}

    def _buf(self, key, shape, dtype, device):
        import torch

        b = self._bufs.get(key)
        if b is None or b.numel() < _numel(shape) or b.dtype != dtype:
            b = torch.empty(_numel(shape), dtype=dtype, device=device)
            self._bufs[key] = b
        return b[: _numel(shape)].view(shape)

    @staticmethod
    def _timed(events, name, fn):
        """Run fn(); if `events` is a dict, bracket the launch with timing events on the current stream."""
        if events is None:
            return fn()
        import torch

        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        r = fn()
        end.record()
        events.setdefault(name, []).append((start, end))
        return r

    def hash(self, input_ids, start_pos: int, token_mask=None, events=None):
        import torch

        B, L = input_ids.shape
        out = self._buf("ids", (B, L, self.E, self.C), torch.int64, input_ids.device)
        s = self.state
        return self._timed(events, "hash", lambda: engram_hash(
            input_ids, start_pos, token_mask, s.token_map, s.cache, s.multipliers, s.primes, s.offsets, s.pad_id,
            s.dead, out=out))

    def hash_gather(self, input_ids, start_pos: int, token_mask=None, events=None):
        """The hash and every layer's gather from its packed table in one launch (engram_hash_gather_packed):
        (ids [B, L, E, C], [a_e bf16 [T, C, D]]), in the buffers `hash` and `layer` use."""
        import torch

        B, L = input_ids.shape
        T = B * L
        dev = input_ids.device
        if any(lw.packed is None for lw in self.layers):
            raise ValueError("every layer needs its packed table")
        D = self.layers[0].weight.shape[1]
        blk = self.layers[0].block_size
        if any(lw.weight.shape[1] != D or lw.block_size != blk for lw in self.layers):
            raise ValueError("the layers' tables differ in row width or block size")
        ids = self._buf("ids", (B, L, self.E, self.C), torch.int64, dev)
        outs = [self._buf(("a", e), (T, self.C, D), torch.bfloat16, dev) for e in range(self.E)]
        s = self.state
        self._timed(events, "hash_gather", lambda: engram_hash_gather_packed(
            input_ids, start_pos, token_mask, s.token_map, s.cache, s.multipliers, s.primes, s.offsets, s.pad_id,
            [lw.packed for lw in self.layers], blk, [lw.row_start for lw in self.layers], s.dead, outs=outs,
            hash_ids=ids))
        return ids, outs

    def gather(self, e: int, hash_ids, events=None, packed=False):
        """Layer e's rows bf16 [T, C, D] (this object's buffer) from its table, or its packed copy."""
        import torch

        lw = self.layers[e]
        T = hash_ids.shape[0] * hash_ids.shape[1]
        a = self._buf(("a", e), (T, self.C, lw.weight.shape[1]), torch.bfloat16, hash_ids.device)
        if packed:
            if lw.packed is None:
                raise ValueError(f"layer {e} has no packed table")
            self._timed(events, "gather_dequant_packed", lambda: engram_gather_dequant_packed(
                hash_ids, lw.packed, lw.block_size, lw.row_start, layer=e, out=a))
        else:
            self._timed(events, "gather_dequant", lambda: engram_gather_dequant(
                hash_ids, lw.weight, lw.scale, lw.block_size, lw.row_start, layer=e, out=a))
        return a

    def layer_fp8(self, e: int, hash_ids, x, events=None, packed=False, a=None, fused=False, gather_mx=False):
        """(a bf16 [T, C*D], kv bf16 [T, Nout], dot fp32 [T, hc]) of layer e with the fp8 block-scaled projection:
        the gathered rows quantised to MX fp8 (engram_mx_quant), engram_wkv_mx against the layer's MX weights,
        then engram_gate_dot; with `fused`, (a, value bf16 [T, dim], dot) from engram_wkv_mx_gate instead.
        With `gather_mx` (and no `a`), the gather writes the MX rows itself (engram_gather_mx) and `a` is None."""
        import torch

        lw = self.layers[e]
        if lw.wkv_mx is None:
            raise ValueError(f"layer {e} has no fp8 (MX) projection weights")
        T = hash_ids.shape[0] * hash_ids.shape[1]
        dev = hash_ids.device
        K = self.C * lw.weight.shape[1]
        aq = self._buf(("a_mx", e), (T, K), torch.uint8, dev)
        asc = self._buf(("a_mx_scale", e), (K // 128, (T + 3) // 4 * 4, 4), torch.uint8, dev)
        if a is None and gather_mx:
            if packed:
                if lw.packed is None:
                    raise ValueError(f"layer {e} has no packed table")
                self._timed(events, "gather_mx_packed", lambda: engram_gather_mx(
                    hash_ids, table=lw.packed, block_size=lw.block_size, row_start=lw.row_start, layer=e, q=aq,
                    q_scale=asc))
            else:
                self._timed(events, "gather_mx", lambda: engram_gather_mx(
                    hash_ids, lw.weight, lw.scale, block_size=lw.block_size, row_start=lw.row_start, layer=e, q=aq,
                    q_scale=asc))
        else:
            if a is None:
                a = self.gather(e, hash_ids, events, packed)
            self._timed(events, "mx_quant", lambda: engram_mx_quant(a.view(T, K), q=aq, scale=asc))
        if fused:
            x3 = x.reshape(T, x.shape[-2], x.shape[-1])
            hc, dim = x3.shape[1], x3.shape[2]
            value = self._buf(("value", e), (T, dim), torch.bfloat16, dev)
            dot = self._buf(("dot", e), (T, hc), torch.float32, dev)
            ws = self._buf("workspace", (engram_wkv_gate_workspace_bytes(T, hc, dim),), torch.uint8, dev)
            self._timed(events, "wkv_mx_gate", lambda: engram_wkv_mx_gate(
                aq, asc, lw.wkv_mx[0], lw.wkv_mx[1], x3, lw.q_weight, lw.k_weight, self.eps, value=value, dot=dot,
                workspace=ws))
            return a, value, dot
        kv = self._buf(("kv", e), (T, lw.wkv.shape[0]), torch.bfloat16, dev)
        self._timed(events, "wkv_mx", lambda: engram_wkv_mx(aq, asc, lw.wkv_mx[0], lw.wkv_mx[1], out=kv))
        x3 = x.reshape(T, x.shape[-2], x.shape[-1])
        dot = self._buf(("dot", e), (T, x3.shape[1]), torch.float32, dev)
        self._timed(events, "gate_dot", lambda: engram_gate_dot(x3, kv, lw.q_weight, lw.k_weight, self.eps, out=dot))
        return a, kv, dot

    def layer(self, e: int, hash_ids, x, events=None, token_mask=None, output=False, fused=False, packed=False,
              a=None):
        """(a bf16 [T, C*D], kv bf16 [T, Nout], dot fp32 [T, hc]) of layer e for x [T, hc, dim]
        (or [B, L, hc, dim]); with `output`, also the layer's output stream bf16 (x's shape), where
        token_mask [B, L] (False = pass through) shuts the gate.  With `fused`, the second tensor is
        the value bf16 [T, dim] alone (the keys are never stored).  With `packed`, the rows come from
        the layer's packed table (same values, one record per row).  With `a` (the layer's rows, already
        gathered by `hash_gather`), no gather is launched.

        The tensors are this object's buffers for layer e: the next call for the same layer
        overwrites them."""
        import torch

        lw = self.layers[e]
        T = hash_ids.shape[0] * hash_ids.shape[1]
        dev = hash_ids.device
        if a is None:
            a = self.gather(e, hash_ids, events, packed)
        x3 = x.reshape(T, x.shape[-2], x.shape[-1])
        dot = self._buf(("dot", e), (T, x3.shape[1]), torch.float32, dev)
        if fused:
            hc, dim = x3.shape[1], x3.shape[2]
            value = self._buf(("value", e), (T, dim), torch.bfloat16, dev)
            ws = self._buf("workspace", (engram_wkv_gate_workspace_bytes(T, hc, dim),), torch.uint8, dev)
            self._timed(events, "wkv_gate", lambda: engram_wkv_gate(
                a.view(T, -1), lw.wkv, x3, lw.q_weight, lw.k_weight, self.eps, value=value, dot=dot, workspace=ws))
            if output:
                out = self._buf(("out", e), tuple(x.shape), torch.bfloat16, dev)
                self._timed(events, "gate_residual", lambda: engram_gate_residual(x, value, dot, token_mask, out=out))
                return a, value, dot, out
            return a, value, dot
        kv = self._buf(("kv", e), (T, lw.wkv.shape[0]), torch.bfloat16, dev)
        self._timed(events, "wkv", lambda: engram_wkv(a.view(T, -1), lw.wkv, out=kv))
        if output:
            out = self._buf(("out", e), tuple(x.shape), torch.bfloat16, dev)
            self._timed(events, "gate_output", lambda: engram_gate_output(
                x, kv, lw.q_weight, lw.k_weight, self.eps, token_mask, out=out, dot=dot))
            return a, kv, dot, out
        self._timed(events, "gate_dot", lambda: engram_gate_dot(x3, kv, lw.q_weight, lw.k_weight, self.eps, out=dot))
        return a, kv, dot

    def step(self, input_ids, start_pos: int, xs, token_mask=None, events=None, output=False, fused=False,
             packed=False, hash_gather=False, all_layers=False, fp8=False, gather_mx=False):
        """One forward over all engram layers; xs[e] is layer e's residual stream [B, L, hc, dim]
        (or one tensor shared by all layers).  Returns the per-layer gate pre-activations, or with
        `output` the per-layer output streams (the pre-activations are then in the "dot" buffers).
        With `hash_gather`, the hash and every layer's packed gather are one launch; with `all_layers`
        (fused only), every layer's projection and gate pre-activation are one launch (their tiles share
        the CUs); with `fp8`, the projection is the fp8 block-scaled form (layer_fp8, fused or not; pre-activations
        only), and with `gather_mx` its gathers write MX fp8 rows directly.
        `events`: optional dict that collects (start, end) timing events per entry point."""
        if hash_gather:
            ids, rows = self.hash_gather(input_ids, start_pos, token_mask, events)
        else:
            ids, rows = self.hash(input_ids, start_pos, token_mask, events), [None] * self.E
        if fp8:
            if output or all_layers:
                raise ValueError("the fp8 projection runs up to the pre-activation, one launch per layer")
            return [self.layer_fp8(e, ids, xs[e] if isinstance(xs, (list, tuple)) else xs, events, packed,
                                   rows[e], fused=fused, gather_mx=gather_mx)[-1] for e in range(self.E)]
        if all_layers:
            if not fused:
                raise ValueError("all_layers needs the fused projection")
            return self._fused_all_layers(ids, rows, xs, events, token_mask, output, packed)
        res = []
        for e in range(self.E):
            x = xs[e] if isinstance(xs, (list, tuple)) else xs
            res.append(self.layer(e, ids, x, events, token_mask=token_mask, output=output, fused=fused,
                                  packed=packed, a=rows[e])[-1])
        return res


    def _fused_all_layers(self, ids, rows, xs, events, token_mask, output, packed):
        import torch

        dev = ids.device
        T = ids.shape[0] * ids.shape[1]
        rows = [r if r is not None else self.gather(e, ids, events, packed) for e, r in enumerate(rows)]
        x_of = [xs[e] if isinstance(xs, (list, tuple)) else xs for e in range(self.E)]
        x3 = [x.reshape(T, x.shape[-2], x.shape[-1]) for x in x_of]
        hc, dim = x3[0].shape[1], x3[0].shape[2]
        values = [self._buf(("value", e), (T, dim), torch.bfloat16, dev) for e in range(self.E)]
        dots = [self._buf(("dot", e), (T, hc), torch.float32, dev) for e in range(self.E)]
        ws = self._buf("workspace", (self.E * engram_wkv_gate_workspace_bytes(T, hc, dim),), torch.uint8, dev)
        L = self.layers
        self._timed(events, "wkv_gate_layers", lambda: engram_wkv_gate_layers(
            [r.view(T, -1) for r in rows], [lw.wkv for lw in L], x3, [lw.q_weight for lw in L],
            [lw.k_weight for lw in L], self.eps, value=values, dot=dots, workspace=ws))
        if not output:
            return dots
        res = []
        for e in range(self.E):
            out = self._buf(("out", e), tuple(x_of[e].shape), torch.bfloat16, dev)
            self._timed(events, "gate_residual", lambda: engram_gate_residual(x_of[e], values[e], dots[e], token_mask,
                                                                              out=out))
            res.append(out)
        return res


def _numel(shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


__all__ = ["HashState", "LayerWeights", "EngramForward"]
