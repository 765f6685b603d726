"""Device side of the seeded input generator: builds and loads libsynth.so
(synth/fill.hip) and fills fp8 tables on the GPU from the same counter-based
definition as `synth.table_rows`."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np

from . import normal_fp8_lut

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
SRC = os.path.join(_HERE, "fill.hip")
_lib = None
_lut_dev = {}


def build(verbose: bool = False) -> str:
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    cmd = [hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", SRC, "-o", LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {SRC}:\n{r.stderr}")
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not built (python -c 'import synth.device as d; d.build()')")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_fill_table.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        L.synth_fill_table.restype = ctypes.c_int
        _lib = L
    return _lib


def fill_table(weight, scale, seed: int, block_size: int, stream=None) -> None:
    """Fill device tensors weight (uint8 [R, D]) and scale (float32 [R, D/blk]) in place."""
    import torch

    dev = weight.device
    if dev not in _lut_dev:
        _lut_dev[dev] = torch.from_numpy(normal_fp8_lut().copy()).to(dev)
    R, D = weight.shape
    s = torch.cuda.current_stream(dev) if stream is None else stream
    rc = lib().synth_fill_table(ctypes.c_void_p(weight.data_ptr()), ctypes.c_void_p(scale.data_ptr()), R, D,
                                block_size, ctypes.c_uint64(seed & 0xFFFFFFFFFFFFFFFF),
                                ctypes.c_void_p(_lut_dev[dev].data_ptr()), ctypes.c_void_p(s.cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_table failed ({rc})")


def device_table(seed: int, rows: int, head_dim: int, block_size: int, device="cuda"):
    """(weight uint8 [rows, D], scale float32 [rows, D/blk]) generated on the GPU."""
    import torch

    w = torch.empty((rows, head_dim), dtype=torch.uint8, device=device)
    s = torch.empty((rows, head_dim // block_size), dtype=torch.float32, device=device)
    fill_table(w, s, seed, block_size)
    return w, s


def device_scale_bytes(scale_f32, fmt: str):
    """synth.scale_bytes on a device float32 scale tensor (the same bit-level definition, as torch integer ops)."""
    import torch

    bits = scale_f32.contiguous().view(torch.int32)
    e = (bits >> 23) & 0xFF
    if fmt == "e8m0":
        return e.to(torch.uint8)
    if fmt == "e4m3":
        return (((e - 117) << 3) | ((bits >> 20) & 7)).to(torch.uint8)
    raise ValueError(fmt)


__all__ = ["build", "lib", "fill_table", "device_table", "device_scale_bytes", "LIB_PATH", "np"]
