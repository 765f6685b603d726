"""CPU oracle for the Engram forward path -- TEST INFRASTRUCTURE ONLY.

Python loader for `liboracle.so` (plain C, `engram_oracle.c`).  Only `tests/`,
`__graft_entry__.smoke()` and the CPU-baseline leg of `bench.py` may import
this package; the product (`gram_hash_embedding_amd`) never does.

Every wrapper takes and returns numpy arrays.  bf16 values travel as their
uint16 bit patterns.  The hash, gather and dequant are exact; the projection,
gate and output return float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SOURCES = [os.path.join(_HERE, "engram_oracle.c")]

_lib = None


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (no GPU toolchain involved)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp", *SOURCES, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.oracle_hash.argtypes = [p, i64, i64, i64, p, p, i64, p, i64, i64, p, p, p, i32, i32, i32, i64, i64, p]
        L.oracle_gather_dequant.argtypes = [p, i64, i64, i32, p, p, i64, i64, i32, i32, p, p, p]
        L.oracle_wkv.argtypes = [p, p, p, i64, i32, i32]
        L.oracle_gate_dot.argtypes = [p, p, i64, p, p, ctypes.c_double, p, i64, i32, i32]
        L.oracle_gate_output.argtypes = [p, p, i64, p, p, p, p, i64, i32, i32]
        L.oracle_gather_dequant_fmt.argtypes = [p, i32, i64, i64, i32, p, p, i32, i64, i64, i32, i32, p, p, p]
        L.oracle_mx_quant.argtypes = [p, i64, i32, i32, p, p]
        L.oracle_wkv_mx.argtypes = [p, p, p, p, p, i64, i32, i32, i32]
        L.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_decode.restype = ctypes.c_double
        L.oracle_e4m3fn_encode_sat.argtypes = [ctypes.c_double]
        L.oracle_e4m3fn_encode_sat.restype = ctypes.c_uint8
        L.oracle_e4m3fn_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3fn_decode.restype = ctypes.c_float
        L.oracle_bf16_rne.argtypes = [ctypes.c_float]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        for f in (L.oracle_hash, L.oracle_gather_dequant, L.oracle_wkv, L.oracle_gate_dot, L.oracle_gate_output,
                  L.oracle_mx_quant, L.oracle_wkv_mx, L.oracle_gather_dequant_fmt):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, name):
    if rc != 0:
        raise OracleError(f"{name} returned {rc}")


def hash(input_ids, start_pos, token_mask, token_map, cache, multipliers, primes, offsets, pad_id,
         dead=-1):
    """ids int64 [B, L, E, C]; `cache` (int64 [cache_B, cache_L], C-contiguous) is updated in place."""
    ids = _c(input_ids, np.int64)
    B, L = ids.shape
    mask = _c(token_mask, np.uint8)
    tmap = _c(token_map, np.int64)
    mult = _c(multipliers, np.int64)
    pr = _c(primes, np.int64)
    off = _c(offsets, np.int64)
    if not (cache.flags.c_contiguous and cache.dtype == np.int64):
        raise ValueError("cache must be a C-contiguous int64 array")
    E, N = mult.shape
    H = pr.shape[2]
    out = np.empty((B, L, E, (N - 1) * H), dtype=np.int64)
    rc = lib().oracle_hash(_ptr(ids), B, L, start_pos, _ptr(mask), _ptr(tmap), tmap.size, _ptr(cache),
                           cache.shape[0], cache.shape[1], _ptr(mult), _ptr(pr), _ptr(off), E, N, H,
                           pad_id, dead, _ptr(out))
    _check(rc, "oracle_hash")
    return out


def gather_dequant(hash_ids, weight, scale, row_start=0, block_size=32, n_cols=None, want_raw=False):
    """hash_ids int64 [T, stride] (first `n_cols` columns used) -> bf16 bits uint16 [T, C, D]
    (and, if want_raw, the gathered bytes [T, C, D] and scales [T, C, D/blk])."""
    ids = _c(hash_ids, np.int64)
    T, stride = ids.shape
    C = stride if n_cols is None else n_cols
    w = _c(weight, np.uint8)
    s = _c(scale, np.float32)
    R, D = w.shape
    out = np.empty((T, C, D), dtype=np.uint16)
    raw = np.empty((T, C, D), dtype=np.uint8) if want_raw else None
    rsc = np.empty((T, C, D // block_size), dtype=np.float32) if want_raw else None
    rc = lib().oracle_gather_dequant(_ptr(ids), T, stride, C, _ptr(w), _ptr(s), R, row_start, D, block_size,
                                     _ptr(out), _ptr(raw), _ptr(rsc))
    _check(rc, "oracle_gather_dequant")
    return (out, raw, rsc) if want_raw else out


SCALE_FORMATS = {"fp32": 0, "e8m0": 1, "e4m3": 2}


def gather_dequant_fmt(hash_ids, weight, scale, scale_format="fp32", row_start=0, block_size=32, n_cols=None,
                       want_raw=False):
    """gather_dequant with the block scales as float32 (`scale` float32 [R, D/blk]) or one-byte E8M0 / E4M3
    (`scale` uint8 [R, D/blk]), and int64 or int32 ids [T, stride] -> bf16 bits uint16 [T, C, D] (and, with
    want_raw, the gathered bytes and the gathered scale elements as stored)."""
    ids = np.ascontiguousarray(hash_ids)
    if ids.dtype not in (np.int64, np.int32):
        raise ValueError("ids must be int64 or int32")
    T, stride = ids.shape
    C = stride if n_cols is None else n_cols
    fmt = SCALE_FORMATS[scale_format]
    w = _c(weight, np.uint8)
    s = _c(scale, np.float32 if fmt == 0 else np.uint8)
    R, D = w.shape
    out = np.empty((T, C, D), dtype=np.uint16)
    raw = np.empty((T, C, D), dtype=np.uint8) if want_raw else None
    rsc = np.empty((T, C, D // block_size), dtype=s.dtype) if want_raw else None
    rc = lib().oracle_gather_dequant_fmt(_ptr(ids), ids.dtype.itemsize, T, stride, C, _ptr(w), _ptr(s), fmt, R,
                                         row_start, D, block_size, _ptr(out), _ptr(raw), _ptr(rsc))
    _check(rc, "oracle_gather_dequant_fmt")
    return (out, raw, rsc) if want_raw else out


def wkv(a_bits, w_bits):
    """a [T, K], w [Nout, K] as bf16 bits -> float64 [T, Nout]."""
    a = _c(a_bits, np.uint16)
    w = _c(w_bits, np.uint16)
    T, K = a.shape
    Nout = w.shape[0]
    out = np.empty((T, Nout), dtype=np.float64)
    _check(lib().oracle_wkv(_ptr(a), _ptr(w), _ptr(out), T, K, Nout), "oracle_wkv")
    return out


def wkv_matmul(a_bits, w_bits, chunk: int = 4096):
    """The same projection as `wkv` (stack-hashes page: Engram's `wkv` Linear, y = a w^T, no bias), with
    numpy's float64 matrix product as the contraction step: bf16 operands decoded exactly to float64, the
    sum over K taken by the library routine.  For parity checks over whole workloads, where the plain C
    loop would take minutes; both are pinned against closed forms and against each other."""
    a = bf16_bits_to_float(_c(a_bits, np.uint16)).astype(np.float64)
    w = bf16_bits_to_float(_c(w_bits, np.uint16)).astype(np.float64)
    if a.ndim != 2 or w.ndim != 2 or a.shape[1] != w.shape[1]:
        raise ValueError("wkv_matmul: a must be [T, K] and w [Nout, K]")
    wt = np.ascontiguousarray(w.T)
    out = np.empty((a.shape[0], w.shape[0]), dtype=np.float64)
    for t0 in range(0, a.shape[0], chunk):
        np.matmul(a[t0:t0 + chunk], wt, out=out[t0:t0 + chunk])
    return out


MX_BLOCK = 32  # columns per E8M0 scale of the fp8 block-scaled projection


def mx_quant(x_bits, block_size: int = MX_BLOCK):
    """bf16 bits [rows, K] -> (q uint8 [rows, K] E4M3FN bytes, scale uint8 [rows, K/block] E8M0 bytes) by the
    OCP MX rule (shared exponent floor(log2 amax) - 8, elements rounded to nearest even and saturated)."""
    x = _c(x_bits, np.uint16)
    rows, K = x.shape
    q = np.empty((rows, K), dtype=np.uint8)
    sc = np.empty((rows, K // block_size), dtype=np.uint8)
    _check(lib().oracle_mx_quant(_ptr(x), rows, K, block_size, _ptr(q), _ptr(sc)), "oracle_mx_quant")
    return q, sc


def wkv_mx(a_q, a_s, w_q, w_s, block_size: int = MX_BLOCK):
    """The fp8 block-scaled projection: (a_q [T, K], a_s [T, K/blk]) x (w_q [Nout, K], w_s [Nout, K/blk])^T
    -> float64 [T, Nout] (per block: scale_a * scale_w * sum of the E4M3 products, summed over blocks)."""
    aq, as_, wq, ws = (_c(v, np.uint8) for v in (a_q, a_s, w_q, w_s))
    T, K = aq.shape
    Nout = wq.shape[0]
    if wq.shape[1] != K or as_.shape != (T, K // block_size) or ws.shape != (Nout, K // block_size):
        raise ValueError("wkv_mx: operand shapes disagree")
    out = np.empty((T, Nout), dtype=np.float64)
    _check(lib().oracle_wkv_mx(_ptr(aq), _ptr(as_), _ptr(wq), _ptr(ws), _ptr(out), T, K, Nout, block_size),
           "oracle_wkv_mx")
    return out


def e8m0_decode(byte: int) -> float:
    return float(lib().oracle_e8m0_decode(byte))


def e4m3fn_encode_sat(value: float) -> int:
    return int(lib().oracle_e4m3fn_encode_sat(float(value)))


def mx_dequant(q, scale, block_size: int = MX_BLOCK):
    """float64 values of MX operands: e4m3(q) * e8m0(scale of the block), through the oracle's decoders."""
    dec8 = np.array([e4m3fn_decode(b) for b in range(256)], dtype=np.float64)
    dec_s = np.array([e8m0_decode(b) for b in range(256)], dtype=np.float64)
    q = np.asarray(q, dtype=np.uint8)
    return dec8[q] * np.repeat(dec_s[np.asarray(scale, dtype=np.uint8)], block_size, axis=-1)


def wkv_mx_matmul(a_q, a_s, w_q, w_s, block_size: int = MX_BLOCK, chunk: int = 4096):
    """`wkv_mx` with numpy's float64 matmul as the contraction over the exactly dequantised operands (every
    E4M3 value times a power of two is exact in float64): for whole-workload parity checks."""
    a = mx_dequant(a_q, a_s, block_size)
    wt = np.ascontiguousarray(mx_dequant(w_q, w_s, block_size).T)
    out = np.empty((a.shape[0], wt.shape[1]), dtype=np.float64)
    for t0 in range(0, a.shape[0], chunk):
        np.matmul(a[t0:t0 + chunk], wt, out=out[t0:t0 + chunk])
    return out


def gate_dot(x_bits, kv_bits, q_bits, k_bits, eps):
    """x [T, hc, dim]; kv [T, >= hc*dim] (key = first hc*dim columns); q, k [hc, dim];
    all bf16 bits -> float64 dot [T, hc]."""
    x = _c(x_bits, np.uint16)
    kv = _c(kv_bits, np.uint16)
    q = _c(q_bits, np.uint16)
    k = _c(k_bits, np.uint16)
    T, hc, dim = x.shape
    out = np.empty((T, hc), dtype=np.float64)
    rc = lib().oracle_gate_dot(_ptr(x), _ptr(kv), kv.shape[1], _ptr(q), _ptr(k), float(eps), _ptr(out), T, hc,
                               dim)
    _check(rc, "oracle_gate_dot")
    return out


def gate_output(x_bits, kv_bits, dot, token_mask=None):
    """x [T, hc, dim] and kv [T, >= (hc+1)*dim] (value = columns hc*dim .. (hc+1)*dim) as bf16 bits;
    dot [T, hc]; token_mask [T] (nonzero = takes part) or None -> (gate float64 [T, hc],
    out float64 [T, hc, dim])."""
    x = _c(x_bits, np.uint16)
    kv = _c(kv_bits, np.uint16)
    d = _c(dot, np.float64)
    mask = _c(token_mask, np.uint8)
    T, hc, dim = x.shape
    if d.shape != (T, hc) or (mask is not None and mask.size != T):
        raise ValueError("gate_output: dot must be [T, hc] and token_mask [T]")
    gate = np.empty((T, hc), dtype=np.float64)
    out = np.empty((T, hc, dim), dtype=np.float64)
    rc = lib().oracle_gate_output(_ptr(x), _ptr(kv), kv.shape[1], _ptr(d), _ptr(mask), _ptr(gate), _ptr(out),
                                  T, hc, dim)
    _check(rc, "oracle_gate_output")
    return gate, out


def e4m3fn_decode(byte: int) -> float:
    return float(lib().oracle_e4m3fn_decode(byte))


def bf16_rne(values) -> np.ndarray:
    """float32 -> bf16 bits, one value at a time through the oracle's rounding."""
    v = np.asarray(values, dtype=np.float32).reshape(-1)
    f = lib().oracle_bf16_rne
    return np.array([f(float(x)) for x in v], dtype=np.uint16)


def bf16_bits_to_float(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on in this process."""
    lib().oracle_set_num_threads(int(n))
