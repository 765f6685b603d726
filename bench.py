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

One step is timed five ways, each its own loop of `--steps` steps:
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
kernel (the fused projection, bf16 MFMA), and the CPU oracle's throughput on
a bounded sample on this host.
"""
from __future__ import annotations

import argparse
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


def source_sha(name: str) -> str:
    path = os.path.join(ROOT, "gram_hash_embedding_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(kernel_file: str, kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 counter summary, if it was taken
    on the current source of `kernel_file`; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != source_sha(kernel_file):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, sample_tokens: int):
    """The CPU oracle, as it stands, over the first `sample_tokens` tokens of the workload."""
    import numpy as np
    import torch

    import oracle
    import synth

    cfg, hi = wl.cfg, wl.host
    B, L = hi.input_ids.shape
    S = min(sample_tokens, L)
    ids_in = np.ascontiguousarray(hi.input_ids[:1, :S])
    mask = None if hi.token_mask is None else np.ascontiguousarray(hi.token_mask[:1, :S])
    timings = {}
    t0 = time.perf_counter()
    ids = oracle.hash(ids_in, 0, mask, hi.token_map, np.zeros((1, S), np.int64), hi.multipliers, hi.primes,
                      hi.offsets, cfg.pad_id, synth.DEAD)
    timings["hash"] = time.perf_counter() - t0
    C, D, blk = cfg.n_hash_cols, cfg.head_dim, cfg.block_size
    x_bits = wl.x[0][:S].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    for e in range(cfg.n_layers):
        lw = wl.fwd.layers[e]
        cw, cs, remap = synth.compact_table(ids.reshape(S, cfg.n_layers, C)[:, e], cfg.rows_alloc[e],
                                            synth.table_seed(cfg, e), D, blk)
        w_bits = lw.wkv.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        q_bits = lw.q_weight.view(torch.int16).cpu().numpy().view(np.uint16)
        k_bits = lw.k_weight.view(torch.int16).cpu().numpy().view(np.uint16)
        t0 = time.perf_counter()
        a = oracle.gather_dequant(remap, cw, cs, block_size=blk)
        t1 = time.perf_counter()
        kv = oracle.wkv(a.reshape(S, C * D), w_bits)
        t2 = time.perf_counter()
        kv_bf16 = torch.from_numpy(kv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        t3 = time.perf_counter()
        oracle.gate_dot(x_bits, kv_bf16, q_bits, k_bits, cfg.eps)
        t4 = time.perf_counter()
        timings["gather_dequant"] = timings.get("gather_dequant", 0.0) + (t1 - t0)
        timings["wkv"] = timings.get("wkv", 0.0) + (t2 - t1)
        timings["gate_dot"] = timings.get("gate_dot", 0.0) + (t4 - t3)
    total = sum(timings.values())
    return {
        "value": round(S / total, 3),
        "unit": "tokens/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"first {S} tokens of the workload through the whole path (hash, gather+dequant, wkv, gate dot); "
                  f"{total:.2f} s of CPU time",
        "seconds": {k: round(v, 3) for k, v in timings.items()},
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload (1..5); 3 = long prefill")
    ap.add_argument("--cpu-sample", type=int, default=2048, help="tokens of the CPU oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    import synth.workload as sw

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

    cfg = synth.CONFIGS[args.config]
    log(f"building workload {cfg.name} ...")
    t_build = time.perf_counter()
    wl = sw.build(cfg, device=dev, packed=True, x_steps=max(1, cfg.decode_steps))
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

    def make_step(fused, output, packed, hg=False, al=False):
        def step(events=None):
            if cfg.decode_steps:
                for s in range(cfg.decode_steps):
                    fwd.step(step_ids[s], cfg.start_pos + s, wl.x[s], None, events=events, output=output,
                             fused=fused, packed=packed, hash_gather=hg, all_layers=al)
            else:
                fwd.step(wl.input_ids, cfg.start_pos, wl.x[0], wl.token_mask, events=events, output=output,
                         fused=fused, packed=packed, hash_gather=hg, all_layers=al)
        return step

    def loop(fused, output, packed, hg=False, al=False):
        """warmup, then `steps` timed steps; (seconds per step, {kernel: [(start, end) events]})"""
        step = make_step(fused, output, packed, hg, al)

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
    runs = [(n, True, False, main_packed, hg, al) for n, hg, al in variants]
    runs += [("fused_" + ("pages_table" if main_packed else "packed_table"), True, False, not main_packed, False, False),
             ("unfused", False, False, main_packed, False, False),
             ("module_fused", True, True, main_packed, False, False),
             ("module_unfused", False, True, main_packed, False, False)]
    for name, fused, output, packed, hg, al in runs:
        sec, ev = loop(fused, output, packed, hg, al)
        paths[name] = {"ms_per_step": round(1e3 * sec, 4), "tokens_per_s": round(T / sec, 1),
                       "table": "packed" if packed else "pages"}
        for k, v in ev.items():
            kern_events.setdefault(k, v)  # the first loop that runs a kernel times it
    sec_main = paths["fused"]["ms_per_step"] / 1e3
    value_mode = "eager"
    if cfg.decode_steps:
        # A decode step is 64 small calls: launched one by one from Python, the GPU waits on the host between
        # kernels.  The same step captured once as a HIP graph (the library's launches on torch's capture
        # stream; every buffer already allocated) and replayed measures the path itself; that is `value`.
        graphs = [(n, True, False, hg, al) for n, hg, al in variants] + [("unfused", False, False, False, False)]
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
    value = T / sec_main

    algo = algorithmic(cfg, wl.token_mask is not None)
    kern = {}
    for name, pairs in kern_events.items():
        ms = [s.elapsed_time(e) for s, e in pairs]
        kern[name] = {"launches": len(ms), "avg_us": round(1e3 * sum(ms) / len(ms), 2)}
    T_launch = cfg.batch if cfg.decode_steps else T  # tokens one launch processes
    E = cfg.n_layers
    W_bytes = 2 * cfg.K * cfg.n_out
    kern["hash"]["GB/s"] = round(T_launch * algo["hash_bytes"] / (kern["hash"]["avg_us"] * 1e3), 1)
    for name in ("gather_dequant", "gather_dequant_packed"):
        g = kern[name]
        g["GB/s"] = round(T_launch * algo["gather_bytes"] / (g["avg_us"] * 1e3), 1)
        g["frac_hbm"] = round(g["GB/s"] / PEAK_HBM_GBS, 4)
    if "hash_gather" in kern:  # the hash and every layer's gather in one launch (ids not read back)
        hg = kern["hash_gather"]
        hg_bytes = algo["hash_bytes"] + E * (algo["gather_bytes"] - 8 * cfg.n_hash_cols)
        hg["GB/s"] = round(T_launch * hg_bytes / (hg["avg_us"] * 1e3), 1)
        hg["frac_hbm"] = round(hg["GB/s"] / PEAK_HBM_GBS, 4)
    if not cfg.decode_steps:
        # The gathers also back to back (the same launch 20 times between two events): inside the step a
        # gather follows the previous step's projection, whose stores are still draining to HBM.
        ids = fwd._buf("ids", (cfg.batch, cfg.seqlen, E, cfg.n_hash_cols), torch.int64, wl.input_ids.device)
        for name, packed in (("gather_dequant_packed", True), ("gather_dequant", False)):
            for _ in range(3):
                fwd.gather(0, ids, packed=packed)
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0.record()
            for _ in range(20):
                fwd.gather(0, ids, packed=packed)
            t1.record()
            torch.cuda.synchronize()
            us = 1e3 * t0.elapsed_time(t1) / 20
            g = kern[name]
            g["back_to_back_us"] = round(us, 2)
            g["back_to_back_GB/s"] = round(T_launch * algo["gather_bytes"] / (us * 1e3), 1)
            g["back_to_back_frac_hbm"] = round(g["back_to_back_GB/s"] / PEAK_HBM_GBS, 4)
    for name, layers in (("wkv", 1), ("wkv_gate", 1), ("wkv_gate_layers", E)):
        if name not in kern:
            continue
        w = kern[name]
        w["TFLOP/s"] = round(layers * T_launch * algo["wkv_flops"] / (w["avg_us"] * 1e6), 1)
        w["frac_mfma"] = round(w["TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
    for name, key in (("gate_dot", "gate_bytes"), ("gate_output", "gate_output_bytes"),
                      ("gate_residual", "gate_residual_bytes")):
        k = kern[name]
        k["GB/s"] = round(T_launch * algo[key] / (k["avg_us"] * 1e3), 1)
        k["frac_hbm"] = round(k["GB/s"] / PEAK_HBM_GBS, 4)

    workload = cfg.name
    wg = kern["wkv_gate"]
    roofline = {
        "kernel": "wkv_gate (fused projection + gate pre-activation; finalize launch included)",
        "bound": "mfma",
        "achieved": wg["TFLOP/s"],
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": wg["frac_mfma"],
        "traffic": load_traffic("wkv.hip", "wkv_gate", workload),
        "algorithmic_bytes_per_launch": T_launch * algo["wkv_gate_bytes"] + W_bytes,
    }
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(1e3 * sec_main, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: Zipf(1.1) token ids, counter-generated fp8 table, N(0,1)/N(0,0.02) bf16)",
        "config": {
            "workload": f"{workload}: B={cfg.batch} L={cfg.seqlen} start_pos={cfg.start_pos}, {E} engram layer(s) "
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
        "roofline": roofline,
        "paths": paths,
        "kernels": kern,
        "kernel_timing": ("HIP events on the launch stream around each entry point of the eager loops"
                          + ("; a decode call's kernels wait on the host between launches, so these include those "
                             "gaps (the kernel trace holds the device durations)" if cfg.decode_steps else "")),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        log(f"CPU oracle baseline on {args.cpu_sample} tokens ...")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
