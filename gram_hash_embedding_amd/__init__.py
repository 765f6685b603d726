"""Engram forward hot path on AMD Instinct MI355X (gfx950).

A thin ctypes binding over libengram.so (include/engram.h).  Each function
has the name of its C entry point, takes torch tensors that already live on
the GPU, checks dtype/shape/contiguity, and passes raw device pointers plus
the current HIP stream.  Every step of the path runs in the library's HIP
kernels; there is no fallback: if libengram.so is missing or a call fails,
an exception is raised.

    engram_hash            -- n-gram hash ids (+ compressed-id cache update)
    engram_hash_gather_packed -- engram_hash and every layer's packed gather + dequant in one launch
    engram_gather_dequant  -- fp8 row gather + block-scale dequant -> bf16
    engram_gather_dequant_fmt -- the same with E8M0 / E4M3 block scales and int32 or int64 ids
    engram_pack_table      -- the table's rows and scales in one record per row (one-off layout conversion)
    engram_gather_dequant_packed -- engram_gather_dequant on a packed table (same output, fewer lines fetched)
    engram_wkv             -- kv = A @ W^T on bf16 matrix cores
    engram_gate_dot        -- per-(token, copy) RMS-normalised gate pre-activation
    engram_gate_output     -- the dot, the sigmoid gate, the token mask and the residual add
    engram_wkv_gate        -- wkv + gate dot fused: value columns and dot out, keys never stored
    engram_wkv_gate_layers -- engram_wkv_gate for several engram layers in one launch
    engram_wkv_gate_layers_noalloc -- the same with the library's own device scratch (allocates nothing)
    engram_gate_residual   -- gate, token mask and residual add from a given dot
    engram_mx_quant        -- bf16 rows -> OCP MX fp8 (E4M3 + E8M0 scale per 32 columns)
    engram_gather_mx       -- the gather + dequant writing its rows as MX fp8 (no bf16 tensor)
    engram_wkv_mx          -- the wkv projection on MX fp8 operands (fp8 matrix cores with block scales)
    engram_wkv_mx_gate     -- engram_wkv_mx fused with the gate dot (keys reduced in the projection)
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libengram.so")

ENGRAM_OK, ENGRAM_EINVAL, ENGRAM_ERANGE, ENGRAM_EHIP = 0, 1, 2, 3

_lib = None


class EngramError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libengram.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not found: build it with `python -m gram_hash_embedding_amd.build` "
                              "(there is no non-HIP fallback)")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, p, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
        L.engram_hash.argtypes = [p, i64, i64, i64, p, p, i64, p, i64, i64, p, p, p, i32, i32, i32, i64, i64, p, p]
        L.engram_hash_i32.argtypes = [p, i64, i64, i64, p, p, i64, p, i64, i64, p, p, p, i32, i32, i32, i64, i64, p, p]
        L.engram_gather_dequant_fmt.argtypes = [p, i32, i64, i64, i32, p, p, i32, i64, i64, i32, i32, p, p, p, p]
        L.engram_hash_gather_packed.argtypes = [p, i64, i64, i64, p, p, i64, p, i64, i64, p, p, p, i32, i32, i32,
                                                i64, i64, p, p, p, p, i32, i32, p, p]
        L.engram_gather_dequant.argtypes = [p, i64, i64, i32, p, p, i64, i64, i32, i32, p, p, p, p]
        L.engram_gather_dequant_packed.argtypes = [p, i64, i64, i32, p, i64, i64, i32, i32, p, p, p, p]
        L.engram_pack_table.argtypes = [p, p, i64, i32, i32, p, p]
        L.engram_wkv.argtypes = [p, p, p, i64, i32, i32, p]
        L.engram_gate_dot.argtypes = [p, p, i64, p, p, f32, p, i64, i32, i32, p]
        L.engram_gate_output.argtypes = [p, p, i64, p, p, f32, p, p, p, i64, i32, i32, p]
        L.engram_wkv_gate.argtypes = [p, p, p, p, p, f32, p, i64, p, p, i64, i64, i32, i32, i32, p]
        L.engram_gate_residual.argtypes = [p, p, i64, p, p, p, i64, i32, i32, p]
        L.engram_wkv_gate_layers.argtypes = [i32, p, p, p, p, p, f32, p, i64, p, p, i64, i64, i32, i32, i32, p]
        L.engram_wkv_gate_layers_noalloc.argtypes = [i32, p, p, p, p, p, f32, p, i64, p, i64, i32, i32, i32, p]
        L.engram_mx_scale_bytes.argtypes = [i64, i32]
        L.engram_mx_scale_bytes.restype = i64
        L.engram_mx_quant.argtypes = [p, i64, i32, p, p, p]
        L.engram_gather_mx.argtypes = [p, i64, i64, i32, p, p, i64, i64, i32, i32, p, p, p]
        L.engram_gather_mx_packed.argtypes = [p, i64, i64, i32, p, i64, i64, i32, i32, p, p, p]
        L.engram_wkv_mx.argtypes = [p, p, p, p, p, i64, i32, i32, p]
        L.engram_wkv_mx_gate.argtypes = [p, p, p, p, p, p, p, f32, p, i64, p, p, i64, i64, i32, i32, i32, p]
        L.engram_wkv_gate_workspace_bytes.argtypes = [i64, i32, i32]
        L.engram_wkv_gate_workspace_bytes.restype = i64
        for f in (L.engram_hash, L.engram_hash_i32, L.engram_gather_dequant_fmt, L.engram_hash_gather_packed, L.engram_gather_dequant, L.engram_gather_dequant_packed, L.engram_pack_table,
                  L.engram_wkv, L.engram_gate_dot, L.engram_gate_output, L.engram_wkv_gate, L.engram_gate_residual,
                  L.engram_wkv_gate_layers, L.engram_wkv_gate_layers_noalloc, L.engram_mx_quant, L.engram_wkv_mx,
                  L.engram_wkv_mx_gate, L.engram_abi_version):
            f.restype = ctypes.c_int
        L.engram_status_string.argtypes = [ctypes.c_int]
        L.engram_status_string.restype = ctypes.c_char_p
        L.engram_last_error.argtypes = []
        L.engram_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != ENGRAM_OK:
        raise EngramError(status, lib().engram_last_error().decode())


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name, dtype, ndim=None):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def engram_hash(input_ids, start_pos, token_mask, token_map, cache, multipliers, primes, offsets, pad_id,
                dead=-1, out=None, stream=None, int32_ids=False):
    """Hash ids int64 [B, L, E, (N-1)*H] (int32 with `int32_ids`: engram_hash_i32, ids outside [0, 2^31) as -1);
    `cache` (int64 [cache_B, cache_L]) is updated in place."""
    import torch

    B, L = input_ids.shape
    E, N = multipliers.shape
    H = primes.shape[2]
    C = (N - 1) * H
    id_dtype = torch.int32 if int32_ids else torch.int64
    if out is None:
        out = torch.empty((B, L, E, C), dtype=id_dtype, device=input_ids.device)
    if tuple(out.shape) != (B, L, E, C):
        raise ValueError("out has the wrong shape")
    if tuple(primes.shape) != (E, N - 1, H) or tuple(offsets.shape) != (E, C):
        raise ValueError("primes must be [E, N-1, H] and offsets [E, (N-1)*H]")
    mask_p = None
    if token_mask is not None:
        if tuple(token_mask.shape) != (B, L):
            raise ValueError("token_mask must be [B, L]")
        if token_mask.dtype == torch.bool:
            token_mask = token_mask.view(torch.uint8)
        mask_p = _dev(token_mask, "token_mask", torch.uint8, 2)
    fn = lib().engram_hash_i32 if int32_ids else lib().engram_hash
    _check(fn(
        _dev(input_ids, "input_ids", torch.int64, 2), B, L, int(start_pos), mask_p,
        _dev(token_map, "token_map", torch.int64, 1), token_map.numel(),
        _dev(cache, "cache", torch.int64, 2), cache.shape[0], cache.shape[1],
        _dev(multipliers, "multipliers", torch.int64, 2), _dev(primes, "primes", torch.int64, 3),
        _dev(offsets, "offsets", torch.int64, 2), E, N, H, int(pad_id), int(dead),
        _dev(out, "out", id_dtype, 4), _stream(stream)))
    return out


def engram_hash_gather_packed(input_ids, start_pos, token_mask, token_map, cache, multipliers, primes, offsets, pad_id,
                              tables, block_size=32, row_starts=None, dead=-1, outs=None, hash_ids=None,
                              stream=None):
    """engram_hash, then for every layer e engram_gather_dequant_packed of its ids on tables[e], in one launch.

    tables: E packed tables (uint8 [R_e, 2*D], engram_pack_table's layout); row_starts: E ints or None (0).
    Returns (outs, hash_ids): outs[e] is bf16 [B*L, C, D]; hash_ids (int64 [B, L, E, C]) is written only if given.
    `cache` is updated in place as by engram_hash."""
    import torch

    B, L = input_ids.shape
    E, N = multipliers.shape
    H = primes.shape[2]
    C = (N - 1) * H
    if len(tables) != E:
        raise ValueError("one packed table per layer")
    D = tables[0].shape[1] // 2
    if tuple(primes.shape) != (E, N - 1, H) or tuple(offsets.shape) != (E, C):
        raise ValueError("primes must be [E, N-1, H] and offsets [E, (N-1)*H]")
    for t in tables:
        if t.dim() != 2 or t.shape[1] != 2 * D:
            raise ValueError("every packed table must be [R, 2*D] with the same D")
    if outs is None:
        outs = [torch.empty((B * L, C, D), dtype=torch.bfloat16, device=input_ids.device) for _ in range(E)]
    if len(outs) != E or any(o.numel() != B * L * C * D for o in outs):
        raise ValueError("outs must hold E tensors of B*L*C*D elements")
    if hash_ids is not None and tuple(hash_ids.shape) != (B, L, E, C):
        raise ValueError("hash_ids has the wrong shape")
    mask_p = None
    if token_mask is not None:
        if tuple(token_mask.shape) != (B, L):
            raise ValueError("token_mask must be [B, L]")
        if token_mask.dtype == torch.bool:
            token_mask = token_mask.view(torch.uint8)
        mask_p = _dev(token_mask, "token_mask", torch.uint8, 2)
    tab_arr = (ctypes.c_void_p * E)(*[_dev(t, "tables[%d]" % e, torch.uint8, 2).value for e, t in enumerate(tables)])
    row_arr = (ctypes.c_int64 * E)(*[t.shape[0] for t in tables])
    rs_arr = None if row_starts is None else (ctypes.c_int64 * E)(*[int(r) for r in row_starts])
    out_arr = (ctypes.c_void_p * E)(*[_dev(o, "outs[%d]" % e, torch.bfloat16).value for e, o in enumerate(outs)])
    ids_p = None if hash_ids is None else _dev(hash_ids, "hash_ids", torch.int64, 4)
    _check(lib().engram_hash_gather_packed(
        _dev(input_ids, "input_ids", torch.int64, 2), B, L, int(start_pos), mask_p,
        _dev(token_map, "token_map", torch.int64, 1), token_map.numel(),
        _dev(cache, "cache", torch.int64, 2), cache.shape[0], cache.shape[1],
        _dev(multipliers, "multipliers", torch.int64, 2), _dev(primes, "primes", torch.int64, 3),
        _dev(offsets, "offsets", torch.int64, 2), E, N, H, int(pad_id), int(dead), ids_p,
        tab_arr, row_arr, rs_arr, D, int(block_size), out_arr, _stream(stream)))
    return outs, hash_ids


def _gather_ids(hash_ids, n_cols, layer):
    """(T, C, id stride, pointer to the layer's first id) of [B, L, E, C] or [T, C] ids."""
    import torch

    if hash_ids.dim() == 4:
        B, L, E, C = hash_ids.shape
        T, stride, base = B * L, E * C, layer * C
    elif hash_ids.dim() == 2:
        T, C = hash_ids.shape
        stride, base = C, 0
    else:
        raise ValueError("hash_ids must be [B, L, E, C] or [T, C]")
    if n_cols is not None:
        C = n_cols
    if not hash_ids.is_contiguous() or hash_ids.dtype not in (torch.int64, torch.int32) or not hash_ids.is_cuda:
        raise ValueError("hash_ids must be a contiguous int64 (or int32) GPU tensor")
    return T, C, stride, ctypes.c_void_p(hash_ids.data_ptr() + hash_ids.element_size() * base)


def _raw_outputs(out_fp8, out_scale, T, C, D, block_size):
    """Pointers of the optional raw-gather outputs, after checking that each holds exactly what the kernel
    writes (T*C*D bytes; T*C*(D/blk) floats)."""
    import torch

    p8 = ps = None
    if out_fp8 is not None:
        if out_fp8.numel() != T * C * D:
            raise ValueError(f"out_fp8 must hold T*C*D = {T * C * D} bytes, has {out_fp8.numel()}")
        p8 = _dev(out_fp8, "out_fp8", torch.uint8)
    if out_scale is not None:
        if block_size <= 0 or out_scale.numel() != T * C * (D // block_size):
            raise ValueError(f"out_scale must hold T*C*(D/block_size) floats, has {out_scale.numel()}")
        ps = _dev(out_scale, "out_scale", torch.float32)
    return p8, ps


def engram_pack_table(weight, scale, block_size=32, out=None, stream=None):
    """uint8 [R, 2*D]: record r = weight[r] (D fp8 bytes), then scale[r] (fp32), then zeros."""
    import torch

    if weight.dtype == torch.float8_e4m3fn:
        weight = weight.view(torch.uint8)
    R, D = weight.shape
    if tuple(scale.shape) != (R, D // block_size):
        raise ValueError("scale must be [R, D/block_size]")
    if out is None:
        out = torch.empty((R, 2 * D), dtype=torch.uint8, device=weight.device)
    if tuple(out.shape) != (R, 2 * D):
        raise ValueError("out must be [R, 2*D]")
    _check(lib().engram_pack_table(_dev(weight, "weight", torch.uint8, 2), _dev(scale, "scale", torch.float32, 2),
                                   R, D, int(block_size), _dev(out, "out", torch.uint8, 2), _stream(stream)))
    return out


def engram_gather_dequant_packed(hash_ids, table, block_size=32, row_start=0, n_cols=None, layer=0, out=None,
                                 out_fp8=None, out_scale=None, stream=None):
    """engram_gather_dequant on a packed table (uint8 [R, 2*D], engram_pack_table's layout)."""
    import torch

    T, C, stride, ids_ptr = _gather_ids(hash_ids, n_cols, layer)
    R, D2 = table.shape
    D = D2 // 2
    if out is None:
        out = torch.empty((T, C, D), dtype=torch.bfloat16, device=hash_ids.device)
    if out.numel() != T * C * D:
        raise ValueError("out has the wrong size")
    p8, ps = _raw_outputs(out_fp8, out_scale, T, C, D, int(block_size))
    _check(lib().engram_gather_dequant_packed(
        ids_ptr, T, stride, C, _dev(table, "table", torch.uint8, 2), R, int(row_start), D, int(block_size),
        _dev(out, "out", torch.bfloat16), p8, ps, _stream(stream)))
    return out


def engram_gather_dequant(hash_ids, weight, scale, block_size=32, row_start=0, n_cols=None, layer=0,
                          out=None, out_fp8=None, out_scale=None, stream=None):
    """bf16 [T, C, D] rows for one layer's ids.

    hash_ids: int64 [B, L, E, C] (engram_hash's output; `layer` picks e) or [T, C].
    weight: float8_e4m3fn or uint8 [R, D]; scale: float32 [R, D/block_size].
    Optional out_fp8 (uint8 [T, C, D]) and out_scale (float32 [T, C, D/blk]) receive the raw gathered bytes/scales.
    """
    import torch

    T, C, stride, ids_ptr = _gather_ids(hash_ids, n_cols, layer)
    if weight.dtype == torch.float8_e4m3fn:
        weight = weight.view(torch.uint8)
    R, D = weight.shape
    if out is None:
        out = torch.empty((T, C, D), dtype=torch.bfloat16, device=hash_ids.device)
    if out.numel() != T * C * D:
        raise ValueError("out has the wrong size")
    if tuple(scale.shape) != (R, D // block_size):
        raise ValueError("scale must be [R, D/block_size]")
    p8, ps = _raw_outputs(out_fp8, out_scale, T, C, D, int(block_size))
    _check(lib().engram_gather_dequant(
        ids_ptr, T, stride, C, _dev(weight, "weight", torch.uint8, 2), _dev(scale, "scale", torch.float32, 2),
        R, int(row_start), D, int(block_size), _dev(out, "out", torch.bfloat16), p8, ps, _stream(stream)))
    return out


SCALE_FORMATS = {"fp32": 0, "e8m0": 1, "e4m3": 2}


def engram_gather_dequant_fmt(hash_ids, weight, scale, scale_format="fp32", block_size=32, row_start=0, n_cols=None,
                              layer=0, out=None, out_fp8=None, out_scale=None, stream=None):
    """engram_gather_dequant with int64 or int32 ids and the block scales as float32 (`scale` float32 [R, D/blk])
    or one-byte E8M0 / float8_e4m3fn (`scale` uint8, float8_e8m0fnu or float8_e4m3fn [R, D/blk])."""
    import torch

    fmt = SCALE_FORMATS[scale_format]
    T, C, stride, ids_ptr = _gather_ids(hash_ids, n_cols, layer)
    if weight.dtype == torch.float8_e4m3fn:
        weight = weight.view(torch.uint8)
    if scale.dtype in (torch.float8_e4m3fn, torch.float8_e8m0fnu):
        scale = scale.view(torch.uint8)
    R, D = weight.shape
    if tuple(scale.shape) != (R, D // block_size):
        raise ValueError("scale must be [R, D/block_size]")
    sdt = torch.float32 if fmt == 0 else torch.uint8
    if out is None:
        out = torch.empty((T, C, D), dtype=torch.bfloat16, device=hash_ids.device)
    if out.numel() != T * C * D:
        raise ValueError("out has the wrong size")
    p8 = ps = None
    if out_fp8 is not None:
        if out_fp8.numel() != T * C * D:
            raise ValueError("out_fp8 must hold T*C*D bytes")
        p8 = _dev(out_fp8, "out_fp8", torch.uint8)
    if out_scale is not None:
        if out_scale.numel() != T * C * (D // block_size):
            raise ValueError("out_scale must hold T*C*(D/block_size) elements")
        ps = _dev(out_scale, "out_scale", sdt)
    _check(lib().engram_gather_dequant_fmt(
        ids_ptr, hash_ids.element_size(), T, stride, C, _dev(weight, "weight", torch.uint8, 2),
        _dev(scale, "scale", sdt, 2), fmt, R, int(row_start), D, int(block_size), _dev(out, "out", torch.bfloat16),
        p8, ps, _stream(stream)))
    return out


def engram_wkv(a, w, out=None, stream=None):
    """kv bf16 [T, Nout] = a [T, K] @ w[Nout, K]^T (bf16 in, fp32 accumulation)."""
    import torch

    a2 = a.reshape(a.shape[0], -1) if a.dim() == 3 else a
    T, K = a2.shape
    Nout, K2 = w.shape
    if K2 != K:
        raise ValueError(f"K mismatch: a has {K}, w has {K2}")
    if out is None:
        out = torch.empty((T, Nout), dtype=torch.bfloat16, device=a.device)
    if tuple(out.shape) != (T, Nout):
        raise ValueError("out must be [T, Nout]")
    _check(lib().engram_wkv(_dev(a2, "a", torch.bfloat16, 2), _dev(w, "w", torch.bfloat16, 2),
                            _dev(out, "out", torch.bfloat16, 2), T, K, Nout, _stream(stream)))
    return out


def engram_gate_dot(x, kv, q_weight, k_weight, eps, out=None, stream=None):
    """dot float32 [T, hc] from x bf16 [T, hc, dim] (or [B, L, hc, dim]) and the keys in kv [T, >= hc*dim]."""
    import torch

    x3 = x.reshape(-1, x.shape[-2], x.shape[-1])
    T, hc, dim = x3.shape
    if kv.dim() != 2 or kv.shape[0] != T:
        raise ValueError("kv must be [T, ld]")
    if tuple(q_weight.shape) != (hc, dim) or tuple(k_weight.shape) != (hc, dim):
        raise ValueError("q_weight and k_weight must be [hc, dim]")
    if out is None:
        out = torch.empty((T, hc), dtype=torch.float32, device=x.device)
    if tuple(out.shape) != (T, hc):
        raise ValueError("out must be [T, hc]")
    _check(lib().engram_gate_dot(
        _dev(x3, "x", torch.bfloat16, 3), _dev(kv, "kv", torch.bfloat16, 2), kv.shape[1],
        _dev(q_weight, "q_weight", torch.bfloat16, 2), _dev(k_weight, "k_weight", torch.bfloat16, 2),
        float(eps), _dev(out, "out", torch.float32), T, hc, dim, _stream(stream)))
    return out


def engram_gate_output(x, kv, q_weight, k_weight, eps, token_mask=None, out=None, dot=None, stream=None):
    """out bf16 [T, hc, dim] (x's shape) = x + gate * value, the gate from the dot of x with the keys in
    kv [T, >= (hc+1)*dim]; token_mask [T] (or x's leading [B, L]) bool/uint8, False shuts the gate.
    `dot` (float32 [T, hc]), if given, receives the pre-activation."""
    import torch

    x3 = x.reshape(-1, x.shape[-2], x.shape[-1])
    T, hc, dim = x3.shape
    if kv.dim() != 2 or kv.shape[0] != T:
        raise ValueError("kv must be [T, ld]")
    if tuple(q_weight.shape) != (hc, dim) or tuple(k_weight.shape) != (hc, dim):
        raise ValueError("q_weight and k_weight must be [hc, dim]")
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    mask_p = None
    if token_mask is not None:
        if token_mask.numel() != T:
            raise ValueError("token_mask must hold one entry per token")
        if token_mask.dtype == torch.bool:
            token_mask = token_mask.view(torch.uint8)
        mask_p = _dev(token_mask.reshape(T), "token_mask", torch.uint8, 1)
    dot_p = None
    if dot is not None:
        if tuple(dot.shape) != (T, hc):
            raise ValueError("dot must be [T, hc]")
        dot_p = _dev(dot, "dot", torch.float32)
    _check(lib().engram_gate_output(
        _dev(x3, "x", torch.bfloat16, 3), _dev(kv, "kv", torch.bfloat16, 2), kv.shape[1],
        _dev(q_weight, "q_weight", torch.bfloat16, 2), _dev(k_weight, "k_weight", torch.bfloat16, 2),
        float(eps), mask_p, _dev(out, "out", torch.bfloat16), dot_p, T, hc, dim, _stream(stream)))
    return out


def engram_mx_scale_bytes(rows: int, K: int) -> int:
    n = lib().engram_mx_scale_bytes(int(rows), int(K))
    if n < 0:
        raise ValueError(f"MX operands need K a positive multiple of 128, got {K}")
    return n


def engram_mx_quant(x, q=None, scale=None, stream=None):
    """bf16 x [rows, K] -> (q uint8 [rows, K] E4M3FN bytes, scale uint8 [K/128, rows4, 4] E8M0 bytes), the OCP MX
    quantisation (include/engram.h for the scale layout)."""
    import torch

    x2 = x.reshape(x.shape[0], -1) if x.dim() == 3 else x
    rows, K = x2.shape
    nbytes = engram_mx_scale_bytes(rows, K)
    if q is None:
        q = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((K // 128, (rows + 3) // 4 * 4, 4), dtype=torch.uint8, device=x.device)
    if tuple(q.shape) != (rows, K):
        raise ValueError("q must be [rows, K]")
    if scale.numel() != nbytes:
        raise ValueError(f"scale must hold {nbytes} bytes")
    _check(lib().engram_mx_quant(_dev(x2, "x", torch.bfloat16, 2), rows, K, _dev(q, "q", torch.uint8, 2),
                                 _dev(scale, "scale", torch.uint8), _stream(stream)))
    return q, scale


def engram_gather_mx(hash_ids, weight=None, scale=None, table=None, block_size=32, row_start=0, n_cols=None, layer=0,
                     q=None, q_scale=None, stream=None):
    """One layer's gathered rows as MX fp8: (q uint8 [T, C*D], q_scale uint8 [C*D/128, rows4, 4]) =
    engram_mx_quant(engram_gather_dequant(...)) bit for bit, without the bf16 tensor.  The table is `weight`
    (float8_e4m3fn or uint8 [R, D]) with `scale` (float32 [R, D/block_size]), or the packed `table`
    (uint8 [R, 2*D]).  int64 ids as engram_gather_dequant's."""
    import torch

    if hash_ids.dtype != torch.int64:
        raise ValueError("hash_ids must be int64")
    T, C, stride, ids_ptr = _gather_ids(hash_ids, n_cols, layer)
    if (table is None) == (weight is None):
        raise ValueError("give either weight and scale or the packed table")
    if table is not None:
        R, D2 = table.shape
        D = D2 // 2
    else:
        if weight.dtype == torch.float8_e4m3fn:
            weight = weight.view(torch.uint8)
        R, D = weight.shape
        if scale is None or tuple(scale.shape) != (R, D // block_size):
            raise ValueError("scale must be [R, D/block_size]")
    K = C * D
    nbytes = engram_mx_scale_bytes(T, K)
    if q is None:
        q = torch.empty((T, K), dtype=torch.uint8, device=hash_ids.device)
    if q_scale is None:
        q_scale = torch.empty((K // 128, (T + 3) // 4 * 4, 4), dtype=torch.uint8, device=hash_ids.device)
    if q.numel() != T * K:
        raise ValueError("q must hold T * C * D bytes")
    if q_scale.numel() != nbytes:
        raise ValueError(f"q_scale must hold {nbytes} bytes")
    if table is not None:
        _check(lib().engram_gather_mx_packed(
            ids_ptr, T, stride, C, _dev(table, "table", torch.uint8, 2), R, int(row_start), D, int(block_size),
            _dev(q, "q", torch.uint8), _dev(q_scale, "q_scale", torch.uint8), _stream(stream)))
    else:
        _check(lib().engram_gather_mx(
            ids_ptr, T, stride, C, _dev(weight, "weight", torch.uint8, 2), _dev(scale, "scale", torch.float32, 2),
            R, int(row_start), D, int(block_size), _dev(q, "q", torch.uint8), _dev(q_scale, "q_scale", torch.uint8),
            _stream(stream)))
    return q, q_scale


def engram_wkv_mx(a, a_scale, w, w_scale, out=None, stream=None):
    """kv bf16 [T, Nout] from MX fp8 operands a (uint8 [T, K]) and w (uint8 [Nout, K]) with their scales."""
    import torch

    if a.dtype == torch.float8_e4m3fn:
        a = a.view(torch.uint8)
    if w.dtype == torch.float8_e4m3fn:
        w = w.view(torch.uint8)
    T, K = a.shape
    Nout, K2 = w.shape
    if K2 != K:
        raise ValueError(f"K mismatch: a has {K}, w has {K2}")
    if a_scale.numel() != engram_mx_scale_bytes(T, K) or w_scale.numel() != engram_mx_scale_bytes(Nout, K):
        raise ValueError("a_scale / w_scale must be MX scale arrays of a and w")
    if out is None:
        out = torch.empty((T, Nout), dtype=torch.bfloat16, device=a.device)
    if tuple(out.shape) != (T, Nout):
        raise ValueError("out must be [T, Nout]")
    _check(lib().engram_wkv_mx(_dev(a, "a", torch.uint8, 2), _dev(a_scale, "a_scale", torch.uint8),
                               _dev(w, "w", torch.uint8, 2), _dev(w_scale, "w_scale", torch.uint8),
                               _dev(out, "out", torch.bfloat16, 2), T, K, Nout, _stream(stream)))
    return out


def engram_wkv_gate_workspace_bytes(T: int, hc: int, dim: int) -> int:
    n = lib().engram_wkv_gate_workspace_bytes(int(T), int(hc), int(dim))
    if n < 0:
        raise ValueError(f"engram_wkv_gate: hc={hc} dim={dim} outside the limits")
    return n


def engram_wkv_mx_gate(a, a_scale, w, w_scale, x, q_weight, k_weight, eps, value=None, dot=None, workspace=None,
                       stream=None):
    """(value bf16 [T, dim], dot float32 [T, hc]) from MX fp8 operands a (uint8 [T, K]) and w (uint8
    [(hc+1)*dim, K]) with their scales, and the stream x bf16 [T, hc, dim] (or [B, L, hc, dim]); `value`,
    `dot` and `workspace` as engram_wkv_gate."""
    import torch

    if a.dtype == torch.float8_e4m3fn:
        a = a.view(torch.uint8)
    if w.dtype == torch.float8_e4m3fn:
        w = w.view(torch.uint8)
    x3 = x.reshape(-1, x.shape[-2], x.shape[-1])
    T, hc, dim = x3.shape
    if a.dim() != 2 or a.shape[0] != T:
        raise ValueError("a must be [T, K]")
    K = a.shape[1]
    if tuple(w.shape) != ((hc + 1) * dim, K):
        raise ValueError("w must be [(hc+1)*dim, K]")
    if a_scale.numel() != engram_mx_scale_bytes(T, K) or w_scale.numel() != engram_mx_scale_bytes(w.shape[0], K):
        raise ValueError("a_scale / w_scale must be MX scale arrays of a and w")
    if tuple(q_weight.shape) != (hc, dim) or tuple(k_weight.shape) != (hc, dim):
        raise ValueError("q_weight and k_weight must be [hc, dim]")
    if value is None:
        value = torch.empty((T, dim), dtype=torch.bfloat16, device=a.device)
    if value.dim() != 2 or value.shape[0] != T or value.shape[1] < dim or value.stride(1) != 1:
        raise ValueError("value must be [T, >= dim] with unit column stride")
    if value.dtype != torch.bfloat16 or not value.is_cuda:
        raise TypeError("value must be a bf16 GPU tensor")
    if dot is None:
        dot = torch.empty((T, hc), dtype=torch.float32, device=a.device)
    if tuple(dot.shape) != (T, hc):
        raise ValueError("dot must be [T, hc]")
    need = engram_wkv_gate_workspace_bytes(T, hc, dim)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    _check(lib().engram_wkv_mx_gate(
        _dev(a, "a", torch.uint8, 2), _dev(a_scale, "a_scale", torch.uint8), _dev(w, "w", torch.uint8, 2),
        _dev(w_scale, "w_scale", torch.uint8), _dev(x3, "x", torch.bfloat16, 3),
        _dev(q_weight, "q_weight", torch.bfloat16, 2), _dev(k_weight, "k_weight", torch.bfloat16, 2), float(eps),
        ctypes.c_void_p(value.data_ptr()), value.stride(0), _dev(dot, "dot", torch.float32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), T, K, hc, dim, _stream(stream)))
    return value, dot


def engram_wkv_gate(a, w, x, q_weight, k_weight, eps, value=None, dot=None, workspace=None, stream=None):
    """(value bf16 [T, dim], dot float32 [T, hc]) from a bf16 [T, K], w bf16 [(hc+1)*dim, K] and the stream
    x bf16 [T, hc, dim] (or [B, L, hc, dim]).  `value` may be a [T, ld >= dim] row-strided view whose first
    dim columns are written; `workspace` a uint8 device tensor of engram_wkv_gate_workspace_bytes bytes
    (allocated here if not given)."""
    import torch

    x3 = x.reshape(-1, x.shape[-2], x.shape[-1])
    T, hc, dim = x3.shape
    if a.dim() != 2 or a.shape[0] != T:
        raise ValueError("a must be [T, K]")
    K = a.shape[1]
    if tuple(w.shape) != ((hc + 1) * dim, K):
        raise ValueError("w must be [(hc+1)*dim, K]")
    if tuple(q_weight.shape) != (hc, dim) or tuple(k_weight.shape) != (hc, dim):
        raise ValueError("q_weight and k_weight must be [hc, dim]")
    if value is None:
        value = torch.empty((T, dim), dtype=torch.bfloat16, device=a.device)
    if value.dim() != 2 or value.shape[0] != T or value.shape[1] < dim or value.stride(1) != 1:
        raise ValueError("value must be [T, >= dim] with unit column stride")
    if value.dtype != torch.bfloat16 or not value.is_cuda:
        raise TypeError("value must be a bf16 GPU tensor")
    if dot is None:
        dot = torch.empty((T, hc), dtype=torch.float32, device=a.device)
    if tuple(dot.shape) != (T, hc):
        raise ValueError("dot must be [T, hc]")
    need = engram_wkv_gate_workspace_bytes(T, hc, dim)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    _check(lib().engram_wkv_gate(
        _dev(a, "a", torch.bfloat16, 2), _dev(w, "w", torch.bfloat16, 2), _dev(x3, "x", torch.bfloat16, 3),
        _dev(q_weight, "q_weight", torch.bfloat16, 2), _dev(k_weight, "k_weight", torch.bfloat16, 2), float(eps),
        ctypes.c_void_p(value.data_ptr()), value.stride(0), _dev(dot, "dot", torch.float32),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), T, K, hc, dim, _stream(stream)))
    return value, dot


def _layers_args(a, w, x, q_weight, k_weight, value, dot):
    """Checked shapes and host pointer arrays of the per-layer operands of engram_wkv_gate_layers(_noalloc)."""
    import torch

    E = len(a)
    if not (len(w) == len(x) == len(q_weight) == len(k_weight) == E) or E < 1:
        raise ValueError("one a, w, x, q_weight and k_weight per layer")
    x3 = [t.reshape(-1, t.shape[-2], t.shape[-1]) for t in x]
    T, hc, dim = x3[0].shape
    K = a[0].shape[1] if a[0].dim() == 2 else -1
    for e in range(E):
        if a[e].dim() != 2 or tuple(a[e].shape) != (T, K):
            raise ValueError("every a must be [T, K] with one T and K")
        if tuple(x3[e].shape) != (T, hc, dim):
            raise ValueError("every x must be [T, hc, dim] with one T, hc and dim")
        if tuple(w[e].shape) != ((hc + 1) * dim, K):
            raise ValueError("every w must be [(hc+1)*dim, K]")
        if tuple(q_weight[e].shape) != (hc, dim) or tuple(k_weight[e].shape) != (hc, dim):
            raise ValueError("q_weight and k_weight must be [hc, dim]")
    if value is None:
        value = [torch.empty((T, dim), dtype=torch.bfloat16, device=a[0].device) for _ in range(E)]
    if dot is None:
        dot = [torch.empty((T, hc), dtype=torch.float32, device=a[0].device) for _ in range(E)]
    if len(value) != E or len(dot) != E:
        raise ValueError("one value and one dot per layer")
    ld = value[0].stride(0)
    for v in value:
        if v.dim() != 2 or v.shape[0] != T or v.shape[1] < dim or v.stride(1) != 1 or v.stride(0) != ld:
            raise ValueError("every value must be [T, >= dim] with unit column stride and one row stride")
        if v.dtype != torch.bfloat16 or not v.is_cuda:
            raise TypeError("value must be a bf16 GPU tensor")
    for d in dot:
        if tuple(d.shape) != (T, hc):
            raise ValueError("dot must be [T, hc]")
    arr = lambda ts, name, dt, nd: (ctypes.c_void_p * E)(*[_dev(t, f"{name}[{i}]", dt, nd).value
                                                          for i, t in enumerate(ts)])
    ptrs = (arr(a, "a", torch.bfloat16, 2), arr(w, "w", torch.bfloat16, 2), arr(x3, "x", torch.bfloat16, 3),
            arr(q_weight, "q_weight", torch.bfloat16, 2), arr(k_weight, "k_weight", torch.bfloat16, 2))
    vals = (ctypes.c_void_p * E)(*[v.data_ptr() for v in value])
    return E, T, K, hc, dim, value, dot, ptrs, vals, ld, arr(dot, "dot", torch.float32, 2)


def engram_wkv_gate_layers(a, w, x, q_weight, k_weight, eps, value=None, dot=None, workspace=None, stream=None):
    """engram_wkv_gate for E layers in one launch: a, w, x, q_weight, k_weight are lists of E tensors shaped as
    engram_wkv_gate takes them (one T, K, hc and dim for all); returns (values, dots), lists of E tensors.
    `value` (list) entries may be [T, ld >= dim] row-strided views, all with one row stride; `workspace` a uint8
    device tensor of E * engram_wkv_gate_workspace_bytes bytes (allocated here if not given)."""
    import torch

    E, T, K, hc, dim, value, dot, ptrs, vals, ld, dots = _layers_args(a, w, x, q_weight, k_weight, value, dot)
    need = E * engram_wkv_gate_workspace_bytes(T, hc, dim)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=a[0].device)
    _check(lib().engram_wkv_gate_layers(
        E, *ptrs, float(eps), vals, ld, dots, _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        T, K, hc, dim, _stream(stream)))
    return value, dot


NOALLOC_SCRATCH_BYTES = 16 << 20  # ENGRAM_NOALLOC_SCRATCH_BYTES of include/engram.h


def engram_wkv_gate_layers_noalloc(a, w, x, q_weight, k_weight, eps, value, dot, stream=None):
    """engram_wkv_gate_layers with the partial sums in the library's own device scratch (no workspace, nothing
    allocated by the call): for callers that cannot allocate.  `value` and `dot` (lists of E tensors) must be
    given.  At most NOALLOC_SCRATCH_BYTES of partial sums (E * engram_wkv_gate_workspace_bytes); calls that
    overlap in time on one GPU share that scratch and race."""
    if value is None or dot is None:
        raise ValueError("engram_wkv_gate_layers_noalloc writes into caller-provided value and dot tensors")
    E, T, K, hc, dim, value, dot, ptrs, vals, ld, dots = _layers_args(a, w, x, q_weight, k_weight, value, dot)
    _check(lib().engram_wkv_gate_layers_noalloc(E, *ptrs, float(eps), vals, ld, dots, T, K, hc, dim,
                                                _stream(stream)))
    return value, dot


def engram_gate_residual(x, value, dot, token_mask=None, out=None, stream=None):
    """out bf16 (x's shape: [T, hc, dim] or [B, L, hc, dim]) = x + gate(dot) * value, from value bf16
    [T, >= dim] (row-strided view allowed) and dot float32 [T, hc]; token_mask [T] or [B, L]
    (False shuts the gate).  `out` may be x itself."""
    import torch

    x3 = x.reshape(-1, x.shape[-2], x.shape[-1])
    T, hc, dim = x3.shape
    if value.dim() != 2 or value.shape[0] != T or value.shape[1] < dim or value.stride(1) != 1:
        raise ValueError("value must be [T, >= dim] with unit column stride")
    if value.dtype != torch.bfloat16 or not value.is_cuda:
        raise TypeError("value must be a bf16 GPU tensor")
    if tuple(dot.shape) != (T, hc):
        raise ValueError("dot must be [T, hc]")
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    mask_p = None
    if token_mask is not None:
        if token_mask.numel() != T:
            raise ValueError("token_mask must hold one entry per token")
        if token_mask.dtype == torch.bool:
            token_mask = token_mask.view(torch.uint8)
        mask_p = _dev(token_mask.reshape(T), "token_mask", torch.uint8, 1)
    _check(lib().engram_gate_residual(
        _dev(x3, "x", torch.bfloat16, 3), ctypes.c_void_p(value.data_ptr()), value.stride(0),
        _dev(dot, "dot", torch.float32), mask_p, _dev(out, "out", torch.bfloat16), T, hc, dim, _stream(stream)))
    return out


__all__ = ["engram_hash", "engram_hash_gather_packed", "engram_gather_dequant", "engram_wkv", "engram_gate_dot", "engram_gate_output",
           "engram_wkv_gate", "engram_wkv_gate_layers", "engram_wkv_gate_layers_noalloc", "NOALLOC_SCRATCH_BYTES",
           "engram_wkv_gate_workspace_bytes", "engram_gather_dequant_fmt", "SCALE_FORMATS", "engram_mx_quant", "engram_gather_mx", "engram_wkv_mx", "engram_wkv_mx_gate", "engram_mx_scale_bytes", "engram_gate_residual", "engram_pack_table",
           "engram_gather_dequant_packed", "EngramError", "lib",
           "LIB_PATH"]
