"""Build libengram.so (HIP, gfx950) in-tree with hipcc.

    python -m gram_hash_embedding_amd.build [-v]

Every source under csrc/ is compiled for gfx950 only and linked into
gram_hash_embedding_amd/libengram.so, which the ctypes binding loads.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libengram.so")
# the measured-ceiling microbenchmarks (include/engram_probe.h), a library of their own
PROBE_SRC = os.path.join(HERE, "probe")
PROBE_LIB_PATH = os.path.join(HERE, "libengram_probe.so")
BUILD_DIR = os.path.join(HERE, "_build")
ROOT = os.path.dirname(HERE)

ARCH = "gfx950"
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 VALU ops (v_pk_*_f32) stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]
# per-source additions: the projection keeps its MFMA accumulators in VGPRs (LLVM's VGPR form of the MFMA),
# so its epilogues use them in place instead of copying each one out of an AGPR first
FILE_FLAGS = {
    "wkv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "wkv16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources() -> list:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line and line.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out:
        print(out, flush=True)
    return obj


def _link(objs, lib_path: str, verbose: bool) -> None:
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip into libengram.so and probe/*.hip into libengram_probe.so.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    probes = sorted(os.path.join(PROBE_SRC, f) for f in os.listdir(PROBE_SRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probes))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs + probes))
    _link(objs[:len(srcs)], LIB_PATH, verbose)
    _link(objs[len(srcs):], PROBE_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
