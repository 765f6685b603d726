"""Benchmark of the Engram forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3]

One step is one pass of the whole path over one batch of synthetic input
already resident in HBM: the hash of all tokens, then per engram layer the
fp8 gather + dequant, the wkv projection and the gate pre-activation dot.
(The decode workload, --config 4: one step is its 64 forward calls of one
token per sequence, after an untimed hash of the 4,096-token history.)
The default workload is the long prefill: one sequence of 65,536 tokens, one
engram layer with the released 384,006,168-row fp8 table (24.6 GB, D = 64,
8 hash heads, n-grams up to 4), dim 5120, hc_mult 4.

The table is resident twice: in the pages' layout (fp8 rows and fp32 scales in
two tensors) and packed (engram_pack_table: one 2*D-byte record per row, the
row's scales in its own line).  The gathered values are identical; `--table`
picks which layout the `value` path reads (default: packed).

One step is timed several ways, each its own loop of `--steps` steps:
  fused           the path with the projection and the gate pre-activation in
                  one entry point (keys reduced in the projection, never
                  stored)
  fused_hash_gather  the fused path with the hash and every layer's gather in one
                  launch (engram_hash_gather_packed; packed table only)
  *_layers        (several layers) the same with every layer's projection in
                  one launch (engram_wkv_gate_layers)
                  -- `value` and `ms_per_step` are the fastest of these
                  (`config.value_path`)
  fused_*_table   the same on the other table layout
  unfused         the same path as four entry points (kv written, then read)
  module_fused    the whole module: fused path + gate, mask and residual
  module_unfused  the whole module: unfused projection + fused dot/gate/residual
The decode workload (64 one-token calls per step) also replays the fused,
fused_hash_gather and unfused steps as HIP graphs (`*_graph`): launched one by
one from Python the GPU waits on the host between kernels, so there `value`
comes from the graph replays (`config.launch`).

Prints one JSON line: whole-job tokens/s, every path's time, per-kernel
timings from HIP events on the launch stream, the roofline of the dominant
kernel (the fused projection, bf16 MFMA) against the spec peak and against
the ceiling measured in the same run (`measured_peaks`: register-only MFMA
loops, streaming HBM read and copy, libengram_probe.so), the gathers also
timed on a cold Infinity Cache, the gather-stress and decode workloads as
`extra_configs` (with --config 3 and unless --no-extra), and the CPU oracle's
throughput on this host (`cpu_baseline`).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Engram fwd tokens/s on 1 MI355X; gather HBM GB/s & wkv MFMA % of peak"
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, TFLOP/s
FLUSH_BYTES = 512 << 20      # read between cold-cache repetitions: twice the 256 MB Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(cfg, has_mask: bool):
    """Bytes / flops each kernel must move or do per token (per layer for the per-layer kernels)."""
    E, C, D, blk = cfg.n_layers, cfg.n_hash_cols, cfg.head_dim, cfg.block_size
    return {
        # input id, mask byte, token_map entry, cache write, E*C int64 ids out
        "hash_bytes": 8 + (1 if has_mask else 0) + 8 + 8 + 8 * E * C,
        # per column: int64 id in, D fp8 bytes + D/blk fp32 scales gathered, D bf16 out
        "gather_bytes": C * (8 + D + 4 * (D // blk) + 2 * D),
        # the same gathered, written as MX fp8: D E4M3 bytes and D/32 E8M0 bytes out per column
        "gather_mx_bytes": C * (8 + D + 4 * (D // blk) + D + D // 32),
        "wkv_flops": 2 * cfg.K * cfg.n_out,
        # A row in, kv row out (the W read is once per launch, added separately)
        "wkv_bytes": 2 * cfg.K + 2 * cfg.n_out,
        # x copy rows + key rows in (bf16), hc fp32 dots out
        "gate_bytes": 2 * cfg.hc_mult * cfg.dim * 2 + 4 * cfg.hc_mult,
        # x copy rows, key rows, the value row in; output rows (bf16) and hc fp32 dots out; mask byte
        "gate_output_bytes": 2 * cfg.hc_mult * cfg.dim * 3 + 2 * cfg.dim + 4 * cfg.hc_mult + (1 if has_mask else 0),
        # fused projection + gate: A row and x copy rows in, value row and hc dots out (W once per launch)
        "wkv_gate_bytes": 2 * cfg.K + 2 * cfg.hc_mult * cfg.dim + 2 * cfg.dim + 4 * cfg.hc_mult,
        # x copy rows, the value row, hc dots in; output rows out; mask byte
        "gate_residual_bytes": 2 * cfg.hc_mult * cfg.dim * 2 + 2 * cfg.dim + 4 * cfg.hc_mult + (1 if has_mask else 0),
    }


def source_sha(names) -> str:
    """First 16 hex digits of the SHA-256 of the named csrc files' contents, concatenated in order."""
    h = hashlib.sha256()
    for name in names:
        h.update(open(os.path.join(ROOT, "gram_hash_embedding_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel_files, kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 counter summary, if it was taken
    on the current source of `kernel_files`; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != source_sha(kernel_files):
        return None
    return rec.get("bytes_per_launch")


def _stream_ptr():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _event_ms(fn, reps: int, between=None) -> list:
    """Per-repetition milliseconds of fn() between two HIP events on the current stream; `between` (untimed)
    runs before every repetition."""
    import torch

    out = []
    for _ in range(reps):
        if between is not None:
            between()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        out.append(s.elapsed_time(e))
    return out


def measured_peaks(dev) -> dict:
    """Ceilings measured on this GPU right now (include/engram_probe.h): register-only MFMA loops on random
    operands (256 workgroups x 8 waves, two per SIMD), a streaming read of 4 GiB and a copy of 2 GiB."""
    import torch

    from gram_hash_embedding_amd import build as engram_build

    P = ctypes.CDLL(engram_build.PROBE_LIB_PATH)
    P.engram_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_void_p]
    P.engram_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    P.engram_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    ops = torch.randint(0, 256, (1 << 16,), dtype=torch.uint8, device=dev, generator=g)
    out = torch.zeros(256 * 8, dtype=torch.float32, device=dev)
    res = {}
    # (name, probe kind, flop per MFMA, MFMAs per iteration, iterations)
    for name, kind, flop, per_it, iters in (("bf16_32x32x16_TFLOP/s", 0, 32768, 4, 100000),
                                            ("bf16_16x16x32_TFLOP/s", 2, 16384, 8, 100000),
                                            ("fp8_32x32x64_TFLOP/s", 1, 131072, 4, 50000),
                                            ("fp8_mx_32x32x64_TFLOP/s", 3, 131072, 4, 30000),
                                            ("fp8_mx_16x16x128_TFLOP/s", 4, 65536, 8, 50000)):
        def run():
            if P.engram_probe_mfma(kind, ops.data_ptr(), out.data_ptr(), 256, 8, iters, _stream_ptr()) != 0:
                raise RuntimeError("engram_probe_mfma failed")
        run()
        ms = min(_event_ms(run, 3))
        res[name] = round(256 * 8 * iters * per_it * flop / (ms * 1e9), 1)
    # the ceilings the kernels are held to: the faster bf16 instruction; for the MX (block-scaled) fp8 kernels the
    # faster scaled instruction; for fp8 without block scales the unscaled one
    res["bf16_mfma_TFLOP/s"] = max(res["bf16_32x32x16_TFLOP/s"], res["bf16_16x16x32_TFLOP/s"])
    res["fp8_mx_mfma_TFLOP/s"] = max(res["fp8_mx_32x32x64_TFLOP/s"], res["fp8_mx_16x16x128_TFLOP/s"])
    res["fp8_mfma_TFLOP/s"] = max(res["fp8_32x32x64_TFLOP/s"], res["fp8_mx_mfma_TFLOP/s"])
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(3)
    red = torch.empty(P.engram_probe_read_grid(), dtype=torch.float32, device=dev)

    def read():
        if P.engram_probe_read(src.data_ptr(), n, red.data_ptr(), _stream_ptr()) != 0:
            raise RuntimeError("engram_probe_read failed")
    read()
    res["hbm_read_GB/s"] = round(n / (min(_event_ms(read, 3)) * 1e6), 1)
    m = 2 << 30
    dst = torch.empty(m, dtype=torch.uint8, device=dev)

    def copy():
        if P.engram_probe_copy(src.data_ptr(), dst.data_ptr(), m, _stream_ptr()) != 0:
            raise RuntimeError("engram_probe_copy failed")
    copy()
    res["hbm_copy_GB/s"] = round(2 * m / (min(_event_ms(copy, 3)) * 1e6), 1)
    res["how"] = ("register-only loops of each MFMA instruction on random operands (E8M0 scales from registers for "
                  "the fp8_mx rows), 256 workgroups x 8 waves; bf16_mfma = the faster bf16 instruction, fp8_mx_mfma = "
                  "the faster block-scaled fp8 one (the MX kernels' ceiling), fp8_mfma = the faster fp8 one of all; "
                  "16-byte streaming read of 4 GiB; copy of 2 GiB (bytes read + written)")
    del src, dst, ops, out, red
    torch.cuda.empty_cache()
    return res


def cpu_baseline(wl, sample_tokens: int, sample_1thread: int):
    """The CPU oracle, as it stands, on this host: the hash and the gather + dequant over every token of the
    workload (the gather reads rows at their real offsets of a full-size host table whose untouched pages are
    never materialised), the projection and the gate dot on the first `sample_tokens` tokens (all threads) and
    `sample_1thread` tokens (one thread), extrapolated linearly to the workload."""
    import numpy as np
    import torch

    import oracle
    import synth

    cfg, hi = wl.cfg, wl.host
    B, L = hi.input_ids.shape
    T = B * L
    C, D, blk, E = cfg.n_hash_cols, cfg.head_dim, cfg.block_size, cfg.n_layers
    threads = oracle.num_threads()
    ids = oracle.hash(hi.input_ids, 0, hi.token_mask, hi.token_map, np.zeros((B, L), np.int64), hi.multipliers,
                      hi.primes, hi.offsets, cfg.pad_id, synth.DEAD)
    tables = []
    for e in range(E):
        tab = synth.SparseHostTable(synth.table_seed(cfg, e), cfg.rows_alloc[e], D, blk)
        tab.fill(ids.reshape(T, E, C)[:, e])
        tables.append(tab)
    x_all = wl.x[0].view(T, cfg.hc_mult, cfg.dim)
    weights = [(lw.wkv.contiguous().view(torch.int16).cpu().numpy().view(np.uint16),
                lw.q_weight.view(torch.int16).cpu().numpy().view(np.uint16),
                lw.k_weight.view(torch.int16).cpu().numpy().view(np.uint16)) for lw in wl.fwd.layers]

    def timed(n_threads: int, S: int) -> dict:
        oracle.set_num_threads(n_threads)
        t = {}
        t0 = time.perf_counter()
        oracle.hash(hi.input_ids, 0, hi.token_mask, hi.token_map, np.zeros((B, L), np.int64), hi.multipliers,
                    hi.primes, hi.offsets, cfg.pad_id, synth.DEAD)
        t["hash"] = time.perf_counter() - t0
        x_bits = x_all[:S].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        for e in range(E):
            w_bits, q_bits, k_bits = weights[e]
            t0 = time.perf_counter()
            a = oracle.gather_dequant(ids.reshape(T, E * C)[:, e * C:(e + 1) * C], tables[e].weight,
                                      tables[e].scale, block_size=blk)
            t1 = time.perf_counter()
            kv = oracle.wkv(a[:S].reshape(S, C * D), w_bits)
            t2 = time.perf_counter()
            kv_bf16 = torch.from_numpy(kv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            t3 = time.perf_counter()
            oracle.gate_dot(x_bits, kv_bf16, q_bits, k_bits, cfg.eps)
            t4 = time.perf_counter()
            t["gather_dequant"] = t.get("gather_dequant", 0.0) + (t1 - t0)
            t["wkv_sample"] = t.get("wkv_sample", 0.0) + (t2 - t1)
            t["gate_dot_sample"] = t.get("gate_dot_sample", 0.0) + (t4 - t3)
        total = t["hash"] + t["gather_dequant"] + (t["wkv_sample"] + t["gate_dot_sample"]) * T / S
        return {"tokens_per_s": round(T / total, 3), "threads": n_threads, "sample_tokens": S,
                "seconds": {k: round(v, 3) for k, v in t.items()}, "extrapolated_s": round(total, 2)}

    all_t = timed(threads, min(sample_tokens, T))
    one_t = timed(1, min(sample_1thread, T))
    oracle.set_num_threads(threads)
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": all_t["tokens_per_s"],
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"hash and gather+dequant over all {T} tokens (full-size sparse host table); wkv and gate dot on "
                   f"the first {all_t['sample_tokens']} tokens ({one_t['sample_tokens']} at one thread), "
                   f"extrapolated linearly to {T}"),
        "cpu_model": model,
        "host_cpus": os.cpu_count(),
        "all_threads": all_t,
        "one_thread": one_t,
        "value_1thread": one_t["tokens_per_s"],
    }


def measure_workload(cfg, args, dev, peaks, full: bool) -> dict:
    """Build one workload, time its step in every launch arrangement (with `full`, also the other table layout,
    the four-entry-point path and the whole module), and the kernels; returns the workload's record (the
    workload object under "_wl")."""
    import torch

    import synth.workload as sw

    log(f"building workload {cfg.name} ...")
    t_build = time.perf_counter()
    fp8 = full and cfg.K % 128 == 0
    wl = sw.build(cfg, device=dev, packed=True, x_steps=max(1, cfg.decode_steps), fp8=fp8)
    fwd = wl.fwd
    if cfg.decode_steps:
        # decode: the compressed-id cache holds the first start_pos tokens of every sequence (untimed); one
        # bench step is then `decode_steps` forward calls of one token per sequence, each with its own stream
        fwd.hash(wl.input_ids[:, :cfg.start_pos].contiguous(), 0)
        P = cfg.start_pos
        step_ids = [wl.input_ids[:, P + s:P + s + 1].contiguous() for s in range(cfg.decode_steps)]
        T = cfg.batch * cfg.decode_steps
    else:
        T = cfg.tokens
    torch.cuda.synchronize()
    log(f"workload ready in {time.perf_counter() - t_build:.1f} s")

    def make_step(fused, output, packed, hg=False, al=False, f8=False, gmx=False):
        def step(events=None):
            if cfg.decode_steps:
                for s in range(cfg.decode_steps):
                    fwd.step(step_ids[s], cfg.start_pos + s, wl.x[s], None, events=events, output=output,
                             fused=fused, packed=packed, hash_gather=hg, all_layers=al, fp8=f8, gather_mx=gmx)
            else:
                fwd.step(wl.input_ids, cfg.start_pos, wl.x[0], wl.token_mask, events=events, output=output,
                         fused=fused, packed=packed, hash_gather=hg, all_layers=al, fp8=f8, gather_mx=gmx)
        return step

    def loop(fused, output, packed, hg=False, al=False, f8=False, gmx=False):
        """warmup, then `steps` timed steps; (seconds per step, {kernel: [(start, end) events]})"""
        step = make_step(fused, output, packed, hg, al, f8, gmx)
        for _ in range(args.warmup):
            step()
        events = {}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(events)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps, events

    # The path itself (hash -> per layer gather+dequant -> projection -> gate pre-activation), fused
    # (engram_wkv_gate: keys reduced in the projection) on the table layout `--table` picks -- the
    # `value` -- and on the other layout; as four separate entry points; then the whole module (gate,
    # mask, residual -> output stream) both ways.
    main_packed = args.table == "packed"
    paths = {}
    kern_events = {}
    # the fused path's launch arrangements: hash and gathers separate or one launch (packed table), the layers'
    # projections one launch each or one for all (more than one layer)
    variants = [("fused", False, False)]
    if main_packed:
        variants.append(("fused_hash_gather", True, False))
    if cfg.n_layers > 1:
        variants += [(n + "_layers", hg, True) for n, hg, _ in variants]
    runs = [(n, True, False, main_packed, hg, al, False, False) for n, hg, al in variants]
    if full:
        runs += [("fused_" + ("pages_table" if main_packed else "packed_table"), True, False, not main_packed, False,
                  False, False, False),
                 ("unfused", False, False, main_packed, False, False, False, False),
                 ("module_fused", True, True, main_packed, False, False, False, False),
                 ("module_unfused", False, True, main_packed, False, False, False, False)]
    if fp8:
        # the fp8 block-scaled projection (gathered rows quantised to MX fp8, engram_wkv_mx, engram_gate_dot)
        runs.append(("fp8_unfused", False, False, main_packed, False, False, True, False))
        # and fused (engram_wkv_mx_gate: keys reduced in the projection), where K allows it; then with the
        # gathers writing MX fp8 rows themselves (engram_gather_mx: no bf16 rows, no quantiser pass)
        if cfg.K >= 384:
            runs.append(("fp8_fused", True, False, main_packed, False, False, True, False))
            runs.append(("fp8_fused_gather_mx", True, False, main_packed, False, False, True, True))
    for name, fused, output, packed, hg, al, f8, gmx in runs:
        sec, ev = loop(fused, output, packed, hg, al, f8, gmx)
        paths[name] = {"ms_per_step": round(1e3 * sec, 4), "tokens_per_s": round(T / sec, 1),
                       "table": "packed" if packed else "pages"}
        if f8:
            paths[name]["dtype"] = "fp8 (OCP MX: E4M3 + E8M0 per 32 columns) projection, bf16 elsewhere"
        for k, v in ev.items():
            kern_events.setdefault(k, v)  # the first loop that runs a kernel times it
    value_mode = "eager"
    if cfg.decode_steps:
        # A decode step is 64 small calls: launched one by one from Python, the GPU waits on the host between
        # kernels.  The same step captured once as a HIP graph (the library's launches on torch's capture
        # stream; every buffer already allocated) and replayed measures the path itself; that is `value`.
        graphs = [(n, True, False, hg, al) for n, hg, al in variants]
        if full:
            graphs.append(("unfused", False, False, False, False))
        for name, fused, output, hg, al in graphs:
            step = make_step(fused, output, main_packed, hg, al)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            for _ in range(args.warmup):
                graph.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                graph.replay()
            torch.cuda.synchronize()
            sec = (time.perf_counter() - t0) / args.steps
            paths[name + "_graph"] = {"ms_per_step": round(1e3 * sec, 4), "tokens_per_s": round(T / sec, 1),
                                      "table": "packed" if main_packed else "pages"}
            del graph
        value_mode = "hip_graph"
    # `value`: the fused path in its fastest launch arrangement here (hash and gathers: one launch at decode,
    # separate at a long prefill, where the standalone gather hides more latency; with several layers, their
    # projections as one launch or one each)
    suffix = "_graph" if value_mode == "hip_graph" else ""
    value_path = min((n + suffix for n, _, _ in variants), key=lambda n: paths[n]["ms_per_step"])
    sec_main = paths[value_path]["ms_per_step"] / 1e3

    algo = algorithmic(cfg, wl.token_mask is not None)
    kern = {}
    for name, pairs in kern_events.items():
        ms = [s.elapsed_time(e) for s, e in pairs]
        kern[name] = {"launches": len(ms), "avg_us": round(1e3 * sum(ms) / len(ms), 2)}
    T_launch = cfg.batch if cfg.decode_steps else T  # tokens one launch processes
    E = cfg.n_layers
    W_bytes = 2 * cfg.K * cfg.n_out
    if "hash" in kern:
        kern["hash"]["GB/s"] = round(T_launch * algo["hash_bytes"] / (kern["hash"]["avg_us"] * 1e3), 1)
    for name in ("gather_dequant", "gather_dequant_packed"):
        if name in kern:
            g = kern[name]
            g["GB/s"] = round(T_launch * algo["gather_bytes"] / (g["avg_us"] * 1e3), 1)
            g["frac_hbm"] = round(g["GB/s"] / PEAK_HBM_GBS, 4)
    for name in ("gather_mx", "gather_mx_packed"):
        if name in kern:
            g = kern[name]
            g["GB/s"] = round(T_launch * algo["gather_mx_bytes"] / (g["avg_us"] * 1e3), 1)
            g["frac_hbm"] = round(g["GB/s"] / PEAK_HBM_GBS, 4)
    if "hash_gather" in kern:  # the hash and every layer's gather in one launch (ids not read back)
        hg = kern["hash_gather"]
        hg_bytes = algo["hash_bytes"] + E * (algo["gather_bytes"] - 8 * cfg.n_hash_cols)
        hg["GB/s"] = round(T_launch * hg_bytes / (hg["avg_us"] * 1e3), 1)
        hg["frac_hbm"] = round(hg["GB/s"] / PEAK_HBM_GBS, 4)
    # The gathers again on a cold Infinity Cache: before every repetition (untimed) a 512 MB buffer, twice the
    # MALL, is streamed through it by a read-only kernel, so no table line of the previous repetition is still
    # on chip and no dirty line is left to be written back during the timed gather.  (In the step a gather
    # follows the previous step's projection, which streams gigabytes through the same caches.)
    flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    flush_red = torch.empty(2048, dtype=torch.float32, device=dev)
    from gram_hash_embedding_amd import build as engram_build

    probe = ctypes.CDLL(engram_build.PROBE_LIB_PATH)
    probe.engram_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]

    def cold():
        if probe.engram_probe_read(flush.data_ptr(), FLUSH_BYTES, flush_red.data_ptr(), _stream_ptr()) != 0:
            raise RuntimeError("engram_probe_read failed")
    ids = fwd._buf("ids", (cfg.batch, 1 if cfg.decode_steps else cfg.seqlen, E, cfg.n_hash_cols), torch.int64,
                   wl.input_ids.device)
    for name, packed in (("gather_dequant_packed", True), ("gather_dequant", False)):
        if name not in kern:
            continue
        ms = _event_ms(lambda: fwd.gather(0, ids, packed=packed), 10, between=cold)
        g = kern[name]
        us = 1e3 * sum(ms) / len(ms)
        g["cold_us"] = round(us, 2)
        g["cold_GB/s"] = round(T_launch * algo["gather_bytes"] / (us * 1e3), 1)
        g["cold_frac_hbm"] = round(g["cold_GB/s"] / PEAK_HBM_GBS, 4)
        if peaks:
            g["frac_hbm_measured_copy"] = round(g["GB/s"] / peaks["hbm_copy_GB/s"], 4)
    del flush
    for name, layers in (("wkv", 1), ("wkv_gate", 1), ("wkv_gate_layers", E)):
        if name not in kern:
            continue
        w = kern[name]
        w["TFLOP/s"] = round(layers * T_launch * algo["wkv_flops"] / (w["avg_us"] * 1e6), 1)
        w["frac_mfma"] = round(w["TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
        if peaks:
            w["frac_mfma_measured"] = round(w["TFLOP/s"] / peaks["bf16_mfma_TFLOP/s"], 4)
        if cfg.decode_steps and name.startswith("wkv_gate"):
            # below the ridge at 256 tokens: the weights (and the stream rows) against HBM too
            byts = layers * (W_bytes + T_launch * algo["wkv_gate_bytes"])
            w["GB/s"] = round(byts / (w["avg_us"] * 1e3), 1)
            w["frac_hbm"] = round(w["GB/s"] / PEAK_HBM_GBS, 4)
    for name in ("wkv_mx", "wkv_mx_gate"):  # the fp8 projection, alone and fused with the gate (finalize included)
        if name not in kern:
            continue
        w = kern[name]
        w["TFLOP/s"] = round(T_launch * algo["wkv_flops"] / (w["avg_us"] * 1e6), 1)
        w["frac_fp8_mfma"] = round(w["TFLOP/s"] / PEAK_FP8_TFLOPS, 4)
        if peaks:
            w["frac_fp8_mfma_measured"] = round(w["TFLOP/s"] / peaks["fp8_mx_mfma_TFLOP/s"], 4)
    if "mx_quant" in kern:
        q = kern["mx_quant"]  # bf16 rows in, E4M3 bytes and E8M0 scales out
        q["GB/s"] = round(T_launch * (2 * cfg.K + cfg.K + cfg.K // 32) / (q["avg_us"] * 1e3), 1)
        q["frac_hbm"] = round(q["GB/s"] / PEAK_HBM_GBS, 4)
    for name, key in (("gate_dot", "gate_bytes"), ("gate_output", "gate_output_bytes"),
                      ("gate_residual", "gate_residual_bytes")):
        if name in kern:
            k = kern[name]
            k["GB/s"] = round(T_launch * algo[key] / (k["avg_us"] * 1e3), 1)
            k["frac_hbm"] = round(k["GB/s"] / PEAK_HBM_GBS, 4)
    rec = {
        "workload": cfg.name,
        "config": {
            "workload": f"{cfg.name}: B={cfg.batch} L={cfg.seqlen} start_pos={cfg.start_pos}, {E} engram layer(s) "
                        f"of {cfg.rows_alloc[0]:,} fp8 rows x D={cfg.head_dim}, {cfg.n_heads} hash heads, "
                        f"max n-gram {cfg.max_ngram_size}, dim={cfg.dim}, hc_mult={cfg.hc_mult}",
            "global_batch": cfg.batch,
            "seq_len": cfg.seqlen,
            "tokens_per_step": T,
            "decode_steps": cfg.decode_steps,
            "launch": value_mode,
            "value_path": value_path,
            "engram_layers": E,
            "table_rows": list(cfg.rows_alloc[:E]),
            "head_dim": cfg.head_dim,
            "n_hash_cols": cfg.n_hash_cols,
            "dim": cfg.dim,
            "hc_mult": cfg.hc_mult,
            "table_layout": args.table,
            "parallelism": "single GPU",
        },
        "value": round(T / sec_main, 1),
        "ms_per_step": round(1e3 * sec_main, 4),
        "paths": paths,
        "kernels": kern,
        "kernel_timing": ("HIP events on the launch stream around each entry point of the eager loops"
                          + ("; a decode call's kernels wait on the host between launches, so these include those "
                             "gaps (the kernel trace holds the device durations)" if cfg.decode_steps else "")
                          + "; cold_*: each repetition after an untimed streaming read of 512 MB"),
        "_wl": wl,
    }
    if cfg.decode_steps and "wkv_gate_layers" in kern:
        # the decode projection of both layers, launched back to back (device time without host gaps)
        x3 = [wl.x[0].view(cfg.batch, cfg.hc_mult, cfg.dim)] * E
        L = fwd.layers
        rows = [fwd._bufs[("a", e)][:cfg.batch * cfg.K].view(cfg.batch, cfg.K) for e in range(E)]
        vals = [fwd._bufs[("value", e)][:cfg.batch * cfg.dim].view(cfg.batch, cfg.dim) for e in range(E)]
        dots = [fwd._bufs[("dot", e)][:cfg.batch * cfg.hc_mult].view(cfg.batch, cfg.hc_mult) for e in range(E)]
        from gram_hash_embedding_amd import engram_wkv_gate_layers
        ws = fwd._bufs["workspace"]

        def proj():
            for _ in range(20):
                engram_wkv_gate_layers(rows, [lw.wkv for lw in L], x3, [lw.q_weight for lw in L],
                                       [lw.k_weight for lw in L], cfg.eps, value=vals, dot=dots, workspace=ws)
        us = 1e3 * min(_event_ms(proj, 3)) / 20
        w = kern["wkv_gate_layers"]
        w["back_to_back_us"] = round(us, 2)
        w["back_to_back_TFLOP/s"] = round(E * T_launch * algo["wkv_flops"] / (us * 1e6), 1)
        w["back_to_back_frac_mfma"] = round(w["back_to_back_TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
        byts = E * (W_bytes + T_launch * algo["wkv_gate_bytes"])
        w["back_to_back_GB/s"] = round(byts / (us * 1e3), 1)
        w["back_to_back_frac_hbm"] = round(w["back_to_back_GB/s"] / PEAK_HBM_GBS, 4)
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload (1..6); 3 = long prefill")
    ap.add_argument("--cpu-sample", type=int, default=2048, help="tokens of the CPU oracle's projection sample")
    ap.add_argument("--cpu-sample-1thread", type=int, default=128,
                    help="tokens of the CPU oracle's one-thread projection sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-ceiling probes")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the gather-stress and decode workloads (extra_configs) after the long prefill")
    ap.add_argument("--table", choices=("packed", "pages"), default="packed",
                    help="table layout of the `value` path: one record per row (engram_pack_table) or the pages' "
                         "two tensors; the other is timed beside it")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a counter reference for rocprofv3)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by sequence with no exchange; only the one-GPU share is built)", file=sys.stderr)
        return 2

    import torch

    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe_mb:
        # a plain copy of known size: the reference that rocprofv3's FETCH_SIZE / WRITE_SIZE are scaled by
        n = args.copy_probe_mb << 20
        src = torch.full((n,), 7, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: {args.copy_probe_mb} MiB device-to-device")

    peaks = None
    if not args.no_peaks:
        log("measured ceilings ...")
        peaks = measured_peaks(dev)
        log(f"  {peaks}")

    cfg = synth.CONFIGS[args.config]
    rec = measure_workload(cfg, args, dev, peaks, full=True)
    wl = rec.pop("_wl")
    kern = rec["kernels"]
    algo = algorithmic(cfg, wl.token_mask is not None)
    T_launch = cfg.batch if cfg.decode_steps else rec["config"]["tokens_per_step"]
    W_bytes = 2 * cfg.K * cfg.n_out
    dom = "wkv_gate_layers" if cfg.decode_steps and "wkv_gate_layers" in kern else "wkv_gate"
    wg = kern[dom]
    roofline = {
        "kernel": f"{dom} (fused projection + gate pre-activation; finalize launch included)",
        "bound": "mfma",
        "achieved": wg["TFLOP/s"],
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": wg["frac_mfma"],
        "traffic": load_traffic(("wkv.hip", "wkv16.hip"), "wkv_gate", cfg.name),
        "algorithmic_bytes_per_launch": T_launch * algo["wkv_gate_bytes"] + W_bytes,
    }
    if peaks:
        roofline["peak_measured"] = peaks["bf16_mfma_TFLOP/s"]
        roofline["frac_measured"] = round(wg["TFLOP/s"] / peaks["bf16_mfma_TFLOP/s"], 4)
    result = {
        "metric": METRIC,
        "value": rec["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: Zipf(1.1) token ids, counter-generated fp8 table, N(0,1)/N(0,0.02) bf16)",
        "config": rec["config"],
        "roofline": roofline,
        "measured_peaks": peaks,
        "paths": rec["paths"],
        "kernels": kern,
        "kernel_timing": rec["kernel_timing"],
        "cpu_baseline": None,
        "extra_configs": None,
    }
    if not args.no_cpu_baseline:
        log(f"CPU oracle baseline ({args.cpu_sample} / {args.cpu_sample_1thread} projection tokens) ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample, args.cpu_sample_1thread)
    if args.config == 3 and not args.no_extra:
        del wl
        torch.cuda.empty_cache()
        extra = {}
        for idx in (5, 4):
            r = measure_workload(synth.CONFIGS[idx], args, dev, peaks, full=False)
            r.pop("_wl")
            extra[r.pop("workload")] = r
            torch.cuda.empty_cache()
        result["extra_configs"] = extra
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
