#!/usr/bin/env python3
"""Benchmark: sparse latent attention decode, B=64, T=32768, k=2048, bf16, one MI355X.

One step = one mla_sparse_decode call (absorb W_UK, sparse attention, merge and
absorb W_UV) over one batch of synthetic inputs already resident in HBM.
The timed steps cycle through several independently seeded query sets
(queries, index lists and weights) over one resident 2.4 GB cache, so the
rows a step gathers are not left in the 256 MB last-level cache by the step
before.

Prints one JSON line.  `value` is selected KV positions per second (B * k per
step), from a timed pass of K steps with nothing but the steps on the stream.
`roofline` covers the attention kernel: a second timed pass runs the same K
steps with a start and a stop HIP event on the attention kernel of every step,
timestamped by that kernel's own dispatch on its stream (the library launches
it with hipExtLaunchKernel), so each interval is the kernel's duration.  The
events still add about a microsecond per step, which is why they stay out of
the first pass; they use a device-scope release (hipEventReleaseToDevice).
`cpu_baseline` times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
ROW_BYTES = 576 * 2            # one selected latent + rotary row, bf16
ROW_FLOPS = 2 * 128 * 576 + 2 * 128 * 512   # scores + mix for 128 heads


def step_bytes(B: int, k: int) -> int:
    """Algorithmic HBM bytes of one decode call: the selected latent and rotary rows, W_UK and
    W_UV, the queries (q_nope, q_pe), the output and the index lists."""
    return B * k * ROW_BYTES + 2 * 128 * 128 * 512 * 2 + B * 128 * (128 + 64 + 128) * 2 + B * k * 4


def step_flops(B: int, k: int) -> int:
    """Algorithmic FLOP of one decode call: scores and mix per selected row, both absorptions."""
    return B * k * ROW_FLOPS + 2 * 2 * B * 128 * 128 * 512
# The code that decides what the decode kernels read and write: the bf16 kernels, the shared
# constants and the host-side work split.
KERNEL_SOURCES = tuple(os.path.join(ROOT, "sparse_latent_attention_amd", "csrc", f)
                       for f in ("mla_bf16.hip", "mla_internal.h", "mla_sparse.cpp"))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_traffic_b64_t32k_k2048.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=1000,
                   help="untimed steps first: clocks and address translation need tens of ms of load to settle")
    p.add_argument("--sets", type=int, default=8, help="independently seeded query sets to rotate")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-rerun-case", action="store_true",
                   help="skip timing the forced case in which splits run again from exact maxima")
    p.add_argument("--no-mall-flush", action="store_true",
                   help="skip the extra pass that writes a 512 MiB buffer before every call")
    p.add_argument("--cpu-rows", type=int, default=0,
                   help="batch rows timed on the CPU oracle (0 = size to ~15 s)")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="after the timed passes, run three plain device copies of this many MiB "
                        "(the known-size kernel that scales the traffic counters)")
    p.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                        "this script with --copy-calibration-mib into " + os.path.relpath(TRAFFIC_FILE, ROOT))
    p.add_argument("--traffic-command", default="", help="command line recorded with --write-traffic")
    p.add_argument("--project", action="store_true",
                   help="time the output projection at B=64 instead of decode; prints its own JSON line")
    p.add_argument("--prefill", action="store_true",
                   help="time the prefill chunk (S=T=4096, k=min(t+1, 2048), bf16) instead of decode; "
                        "prints its own JSON line (not the headline metric)")
    p.add_argument("--dequant", action="store_true",
                   help="time the FP8 wkv_b dequantisation; prints its own JSON line")
    p.add_argument("--append", action="store_true",
                   help="time the cache append of a 4096-position chunk; prints its own JSON line")
    p.add_argument("--no-prefill-extras", action="store_true",
                   help="skip timing the prefill chunk (both forms) beside the decode line")
    p.add_argument("--prefill-explicit", action="store_true",
                   help="time the same prefill chunk in the explicit form (keys and values "
                        "up-projected per head); prints its own JSON line")
    return p.parse_args()


HIP_EVENT_RELEASE_TO_DEVICE = 0x40000000


def hip_runtime():
    """The HIP runtime library this process already uses (the one torch loaded)."""
    import ctypes
    path = "libamdhip64.so"
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
    hip = ctypes.CDLL(path)
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def device_events(hip, n):
    import ctypes
    evs = []
    for _ in range(n):
        ev = ctypes.c_void_p()
        if hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_RELEASE_TO_DEVICE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        evs.append(ev)
    return evs


def source_hash(text=None) -> str:
    """Hash of the kernel sources' code: comments and blank space are dropped, so an edit
    to a comment keeps the counter record, and any change to the code voids it."""
    if text is None:
        text = "\n".join(open(p).read() for p in KERNEL_SOURCES)
    code = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    code = re.sub(r"//[^\n]*", " ", code)
    code = " ".join(code.split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per attention launch and per decode call (the three kernels) from committed
    rocprofv3 counters, if still current: (attention, step), None where unknown."""
    if not os.path.exists(TRAFFIC_FILE):
        return None, None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("kernel_source_sha256_16") != source_hash():
        return None, None
    return rec.get("bytes_per_launch"), rec.get("step_bytes_per_call")


def _counter_per_dispatch(out_dir: str, counter: str):
    """[(dispatch id, kernel name, value summed over instances)] from a rocprofv3 --pmc CSV run."""
    import csv
    import glob
    files = glob.glob(os.path.join(out_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {out_dir}")
    acc = {}
    for row in csv.DictReader(open(files[0])):
        if row["Counter_Name"] != counter:
            continue
        key = (int(row["Dispatch_Id"]), row["Kernel_Name"])
        acc[key] = acc.get(key, 0.0) + float(row["Counter_Value"])
    return [(d, n, v) for (d, n), v in sorted(acc.items())]


def write_traffic(fetch_dir: str, write_dir: str, copy_mib: int, command: str):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the attention kernel by what the
    same counters read for the calibration copy (copy_mib MiB read and written, the last
    three copy dispatches of the run), and record the result next to the kernel's hash."""
    units = 64 * 2048
    known = copy_mib * 2 ** 20
    rec = {"kernel_source_sha256_16": source_hash(),
           "workload": "decode B=64 T=32768 k=2048, bf16 (bench.py defaults)",
           "command": command, "calibration_copy_bytes": known}
    for tag, d, counter in (("read", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_per_dispatch(d, counter)
        attn = [v for _, n, v in rows if "attn_bf16" in n]
        uv = [v for _, n, v in rows if "uv_bf16" in n]
        absorb = [v for _, n, v in rows if "absorb_q_bf16" in n]
        copies = [v for _, n, v in rows if "copyBuffer" in n][-3:]
        if not attn or len(copies) < 3:
            raise SystemExit(f"{d}: attention dispatches or calibration copies missing")
        factor = known / (1024.0 * float(np.mean(copies)))
        rec[f"{counter}_kib_attention"] = float(np.mean(attn))
        rec[f"{counter}_kib_uv"] = float(np.mean(uv)) if uv else None
        rec[f"{counter}_kib_absorb"] = float(np.mean(absorb)) if absorb else None
        rec[f"{counter}_kib_calibration_copy"] = float(np.mean(copies))
        rec[f"{tag}_scale"] = factor
        rec[f"{tag}_bytes_per_launch"] = float(np.mean(attn)) * 1024.0 * factor
        if not uv or not absorb:
            raise SystemExit(f"{d}: W_UK absorb or merge + W_UV dispatches missing")
        rec[f"{tag}_step_bytes_per_call"] = float(np.mean(attn) + np.mean(uv) + np.mean(absorb)) * 1024.0 * factor
    rec["bytes_per_launch"] = rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
    rec["step_bytes_per_call"] = rec["read_step_bytes_per_call"] + rec["write_step_bytes_per_call"]
    rec["algorithmic_bytes_per_launch"] = units * ROW_BYTES
    rec["algorithmic_step_bytes_per_call"] = step_bytes(64, 2048)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, rows_wanted: int):
    """Time the fp64 oracle on whole batch rows of the same workload (set 0).

    Returns the baseline object (the explicit form the oracle defines, all host threads)
    and two more timings, labelled apart: the absorbed fp64 form on the selected rows
    (the GPU's algorithm on the CPU) and the explicit form on one thread."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threadpool_limits = None
        cores = os.cpu_count() or 1
    w_uk, w_uv = synth.weights(cfg)
    rows = {}

    def inputs(b):
        if b not in rows:
            kv, pe = synth.decode_batch_row(cfg, b)
            qn, qp, idx = synth.decode_query_set(cfg, b, 0)
            rows[b] = (qn, qp, kv, pe, idx)
        return rows[b]

    def explicit(b):
        qn, qp, kv, pe, idx = inputs(b)
        t0 = time.perf_counter()
        oracle.attend_explicit_gather(qn, qp, kv, pe, w_uk, w_uv, idx)
        return time.perf_counter() - t0

    def absorbed(b):
        qn, qp, kv, pe, idx = inputs(b)
        t0 = time.perf_counter()
        oracle.decode_absorbed(qn, qp, kv[idx], pe[idx], w_uk, w_uv, np.arange(len(idx)))
        return time.perf_counter() - t0

    first = explicit(0)
    n = rows_wanted if rows_wanted > 0 else max(1, min(cfg.B, int(15.0 / max(first, 1e-3))))
    spent = first + sum(explicit(b) for b in range(1, n))
    model = _cpu_model()
    base = {"value": n * cfg.k / spent, "unit": "selected KV positions/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{n} of {cfg.B} batch rows x {cfg.k} selected positions, explicit fp64 "
                      f"form, {spent:.1f} s on {model}"}
    t_abs = sum(absorbed(b) for b in range(n))
    extra = {"cpu_baseline_absorbed": {
        "value": n * cfg.k / t_abs, "unit": "selected KV positions/s", "cores": int(cores),
        "kind": "oracle absorbed form",
        "sample": f"{n} of {cfg.B} batch rows x {cfg.k} selected positions, absorbed fp64 form "
                  f"on the selected rows, {t_abs:.1f} s"}}
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            one = explicit(0)
            m = max(1, min(n, int(10.0 / max(one, 1e-3))))
            t1 = one + sum(explicit(b) for b in range(1, m))
        extra["cpu_baseline_1thread"] = {
            "value": m * cfg.k / t1, "unit": "selected KV positions/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{m} of {cfg.B} batch rows x {cfg.k} selected positions, explicit fp64 "
                      f"form, one thread, {t1:.1f} s"}
    return base, extra


EXPLICIT_PAIR_FLOPS = 2 * 128 * (192 + 128)   # explicit form: scores + mix for 128 heads


def prefill_measure(torch, synth, mla, explicit, steps, warm, inp=None):
    """Time one prefill chunk of one sequence: S = T = 4096 queries from position 0, query t
    selecting min(t + 1, 2048) positions up to its own.  Returns the chunk's algorithmic FLOP,
    its selected (query, position) pairs and the mean time per call.  Latent form: the
    absorptions plus 278,528 FLOP per selected pair.  Explicit form: the up-projection of
    every visible position's keys and values (2 x 256 x 512 x 128 FLOP each) plus 81,920 FLOP
    per selected pair."""
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS["prefill_s4096"]
    if inp is None:
        inp = synth.prefill_inputs(cfg)

    def up(x):
        x = np.ascontiguousarray(x)
        if x.dtype in (np.int32, np.int64):
            return torch.from_numpy(x).to(dev)
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    d = {name: up(v) for name, v in inp.items()}
    S, k = cfg.S, cfg.k
    pairs = int((d["topk_idx"] >= 0).sum().item())
    if explicit:
        visible = min(cfg.start_pos + S, cfg.T)
        flop = pairs * EXPLICIT_PAIR_FLOPS + 2 * visible * 128 * 256 * 512
        ws = torch.empty(mla.prefill_explicit_workspace_size(S, cfg.T, k, cfg.start_pos, torch.bfloat16),
                         dtype=torch.uint8, device=dev)
        entry = mla.prefill_explicit
    else:
        flop = pairs * ROW_FLOPS + 2 * 2 * S * 128 * 128 * 512
        ws = torch.empty(mla.prefill_chunk_workspace_size(S, cfg.T, k, torch.bfloat16), dtype=torch.uint8,
                         device=dev)
        entry = mla.prefill_chunk
    out = torch.empty((S, 128, 128), dtype=torch.bfloat16, device=dev)

    def call():
        entry(d["q_nope"], d["q_pe"], d["kv_cache"], d["pe_cache"], d["topk_idx"],
              d["w_uk"], d["w_uv"], start_pos=cfg.start_pos, out=out, workspace=ws)

    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / steps
    del d, ws, out
    return {"flop": flop, "pairs": pairs, "sec": sec}


def bench_prefill(args, torch, synth, mla, explicit=False):
    """The prefill chunk as its own benchmark line (prefill_measure)."""
    steps = min(args.steps, 50)
    warm = min(args.warmup, 10)
    m = prefill_measure(torch, synth, mla, explicit, steps, warm)
    form = "explicit" if explicit else "latent"
    flop, pairs, sec = m["flop"], m["pairs"], m["sec"]
    tflops = flop / sec / 1e12
    print(json.dumps({
        "metric": f"prefill chunk FLOP/s, {form} form (S=T=4096, k=min(t+1,2048))", "value": flop / sec,
        "unit": "FLOP/s", "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": sec * 1e3,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic prefill_s4096 inputs",
        "config": {"workload": f"prefill chunk ({form} form) S=4096, T=4096, k=min(t+1, 2048), 128 heads, bf16",
                   "pairs": pairs, "flop": flop},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_PEAK_TFLOPS, "traffic": None}}), flush=True)


def bench_project(args, torch, synth, mla):
    """The output projection Delta = o W_O at the decode batch (B=64): a weight-streaming product
    whose algorithmic bytes are the 235 MB bf16 weight plus the head outputs and the result (the
    14.7 MB of float32 partial sums the kernels exchange are not algorithmic)."""
    dev = torch.device("cuda:0")
    B = 64
    inp = synth.projection_inputs(B, "bf16")

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    o, w = up(inp["o"]), up(inp["w_o"])
    out = torch.empty((B, 7168), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mla.output_projection_workspace_size(B, torch.bfloat16), dtype=torch.uint8, device=dev)
    steps, warm = min(args.steps, 200), min(args.warmup, 50)
    for _ in range(warm):
        mla.output_projection(o, w, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        mla.output_projection(o, w, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / steps
    nbytes = 7168 * 16384 * 2 + B * 16384 * 2 + B * 7168 * 2
    gbs = nbytes / sec / 1e9
    print(json.dumps({
        "metric": "output projection weight-stream rate (B=64, 7168 x 16384 bf16)", "value": gbs,
        "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": sec * 1e3,
        "higher_is_better": True, "dtype": "bf16", "data": "synthetic projection_inputs",
        "config": {"workload": "output projection o [64, 16384] . W_O [7168, 16384]^T, bf16", "bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None}}), flush=True)


def bench_append(args, torch, synth, mla):
    """The cache append of 4096-position prefill chunks of 8 sequences (B = 8, S = 4096 into 4096-row caches):
    per position 576 down-projection outputs read and 576 cache values written, bf16.  The
    one-position decode append of 64 sequences is timed beside it (a latency figure)."""
    dev = torch.device("cuda:0")

    def up(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.float32:
            return torch.from_numpy(x).to(dev)
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    def timed(cfg, steps, warm):
        d = {name: up(v) for name, v in synth.append_inputs(cfg).items()}

        def call():
            mla.cache_append(d["kv_a_out"], d["norm_weight"], d["cos_sin"], d["kv_cache"], d["pe_cache"],
                             start_pos=cfg.start_pos)
        for _ in range(warm):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / steps

    from synth.generators import AppendConfig
    steps, warm = min(args.steps, 200), min(args.warmup, 50)
    sec = timed(AppendConfig(80, "append_chunk", B=8, S=4096, T=4096, start_pos=0, dtype="bf16"), steps, warm)
    sec_dec = timed(AppendConfig(81, "append_decode", B=64, S=1, T=64, start_pos=63, dtype="bf16"),
                    steps, warm)
    nbytes = 8 * 4096 * (576 + 576) * 2 + 512 * 2 + 4096 * 32 * 2 * 4
    gbs = nbytes / sec / 1e9
    print(json.dumps({
        "metric": "cache append rate (B=8 x S=4096 positions, bf16)", "value": gbs, "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": sec * 1e3, "higher_is_better": True,
        "dtype": "bf16", "data": "synthetic append_inputs",
        "config": {"workload": "cache append: RMSNorm of 512 latent values, rotation of 64 rotary values, "
                               "write at start_pos; B=8, S=4096, ld_T=4096, bf16", "bytes": nbytes},
        "decode_append_b64_ms": sec_dec * 1e3,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None}}), flush=True)


def bench_dequant(args, torch, synth, mla):
    """The FP8 wkv_b dequantisation: 16.8 MB of E4M3 codes and 4 KB of block scales read,
    W_UK and W_UV (33.5 MB of bf16) written."""
    dev = torch.device("cuda:0")
    d = synth.fp8_wkv_b_inputs()
    codes = torch.from_numpy(d["codes"]).to(dev)
    scales = torch.from_numpy(d["scales"]).to(dev)
    w_uk = torch.empty((128, 128, 512), dtype=torch.bfloat16, device=dev)
    w_uv = torch.empty_like(w_uk)
    steps, warm = min(args.steps, 200), min(args.warmup, 50)
    for _ in range(warm):
        mla.wkv_b_dequant(codes, scales, w_uk=w_uk, w_uv=w_uv)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        mla.wkv_b_dequant(codes, scales, w_uk=w_uk, w_uv=w_uv)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / steps
    nbytes = codes.numel() + scales.numel() * 4 + 2 * w_uk.numel() * 2
    gbs = nbytes / sec / 1e9
    print(json.dumps({
        "metric": "FP8 wkv_b dequantisation rate (32768 x 512 E4M3, 128 x 128 block scales)", "value": gbs,
        "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm, "ms_per_step": sec * 1e3,
        "higher_is_better": True, "dtype": "fp8->bf16", "data": "synthetic fp8_wkv_b_inputs",
        "config": {"workload": "wkv_b dequantisation: E4M3 codes [32768, 512] x block scales -> "
                               "W_UK, W_UV [128, 128, 512] bf16", "bytes": nbytes},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None}}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(decode batch rows shard across GPUs with no exchange, so N GPUs run N copies "
              "of this one-GPU step)", file=sys.stderr)
        sys.exit(2)
    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], args.copy_calibration_mib,
                      args.traffic_command)
        return

    import torch
    import synth
    import sparse_latent_attention_amd as mla

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    mla._lib.load()
    if args.prefill or args.prefill_explicit:
        bench_prefill(args, torch, synth, mla, explicit=args.prefill_explicit)
        return
    if args.project:
        bench_project(args, torch, synth, mla)
        return
    if args.append:
        bench_append(args, torch, synth, mla)
        return
    if args.dequant:
        bench_dequant(args, torch, synth, mla)
        return
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS["sparse_b64_t32k"]
    B, T, k = cfg.B, cfg.T, cfg.k

    def up(x):
        x = np.ascontiguousarray(x)
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    t0 = time.time()
    kv = torch.empty((B, T, 512), dtype=torch.bfloat16, device=dev)
    pe = torch.empty((B, T, 64), dtype=torch.bfloat16, device=dev)
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for b, (kv_b, pe_b) in enumerate(ex.map(lambda r: synth.decode_batch_row(cfg, r), range(B))):
            kv[b].copy_(up(kv_b))
            pe[b].copy_(up(pe_b))
    sets = []
    for s in range(args.sets):
        qs = [synth.decode_query_set(cfg, b, s) for b in range(B)]
        w_uk, w_uv = synth.weights(cfg, seed=synth.DEFAULT_SEED + s)
        sets.append({
            "q_nope": up(np.stack([q[0] for q in qs])), "q_pe": up(np.stack([q[1] for q in qs])),
            "idx": torch.from_numpy(np.stack([q[2] for q in qs])).to(dev),
            "w_uk": up(w_uk), "w_uv": up(w_uv)})
    out = torch.empty((B, 128, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mla.decode_workspace_size(B, T, k, torch.bfloat16), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    # One checked call through the Python binding, then the timed loop calls the C
    # entry point directly with pre-marshalled pointers (no per-call Python checks).
    s0 = sets[0]
    mla.decode(s0["q_nope"], s0["q_pe"], kv, pe, s0["idx"], s0["w_uk"], s0["w_uv"], out=out,
               workspace=ws)
    lib = mla._lib.load()
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    scale = ctypes.c_float(mla.SOFTMAX_SCALE)
    argv = [(P(s["q_nope"]), P(s["q_pe"]), P(kv), P(pe), P(s["idx"]), P(s["w_uk"]), P(s["w_uv"]),
             P(out), B, T, T, k, scale, mla.MLA_BF16, P(ws), ws.numel(), stream) for s in sets]

    def step(i, ev=None):
        if ev is not None:
            lib.mla_set_attention_events(ev[0], ev[1])
        st = lib.mla_sparse_decode(*argv[i % len(argv)])
        if st != 0:
            raise RuntimeError(f"mla_sparse_decode returned {st}")

    for i in range(args.warmup):
        step(i)
    hip = hip_runtime()
    flat = device_events(hip, 2 * args.steps)
    evs = list(zip(flat[0::2], flat[1::2]))
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)

    # pass 1: throughput
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps

    # pass 2: the same steps, each attention kernel timed by its own dispatch's events
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    stop.record()
    torch.cuda.synchronize()
    ms_events = start.elapsed_time(stop) / args.steps
    attn_ms = []
    for a, b in evs:
        t = ctypes.c_float()
        if hip.hipEventElapsedTime(ctypes.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        attn_ms.append(t.value)
    for e in flat:
        hip.hipEventDestroy(e)
    attn_avg_ms = float(np.mean(attn_ms))
    attn_pct = [float(np.percentile(attn_ms, q)) for q in (10, 50, 90)]

    # pass 3: a 512 MiB write before every call evicts the 256 MB last-level
    # cache; each call is bracketed by events after its write (median)
    flushed_ms = None
    if not args.no_mall_flush:
        n_flush = min(args.steps, 100)
        scratch = torch.empty(512 * 2 ** 20, dtype=torch.uint8, device=dev)
        fev = device_events(hip, 2 * n_flush)
        torch.cuda.synchronize()
        for i in range(n_flush):
            scratch.fill_(i & 255)
            if hip.hipEventRecord(fev[2 * i], stream) != 0:
                raise RuntimeError("hipEventRecord failed")
            step(args.warmup + i)
            if hip.hipEventRecord(fev[2 * i + 1], stream) != 0:
                raise RuntimeError("hipEventRecord failed")
        torch.cuda.synchronize()
        per = []
        for i in range(n_flush):
            t = ctypes.c_float()
            if hip.hipEventElapsedTime(ctypes.byref(t), fev[2 * i], fev[2 * i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            per.append(t.value)
        for e in fev:
            hip.hipEventDestroy(e)
        flushed_ms = float(np.median(per))
        del scratch

    # pass 4: a forced worst case for the softmax reference.  With W_UK = 0 and softmax
    # scale 10 the scores spread over hundreds of log2 units, so later tiles beat their
    # split's first-tile reference and the splits run again from their exact maxima.
    rerun = None
    if not args.no_rerun_case:
        s_r = sets[0]
        wz = torch.zeros_like(s_r["w_uk"])
        ws_r = torch.empty_like(ws)
        rargs = (P(s_r["q_nope"]), P(s_r["q_pe"]), P(kv), P(pe), P(s_r["idx"]), P(wz), P(s_r["w_uv"]),
                 P(out), B, T, T, k, ctypes.c_float(10.0), mla.MLA_BF16, P(ws_r), ws_r.numel(), stream)
        n_r = min(args.steps, 100)
        for _ in range(10):
            if lib.mla_sparse_decode(*rargs) != 0:
                raise RuntimeError("mla_sparse_decode failed (forced case)")
        torch.cuda.synchronize()
        diag = mla.diagnostics(ws_r, B, k, torch.bfloat16)
        start.record()
        for _ in range(n_r):
            lib.mla_sparse_decode(*rargs)
        stop.record()
        torch.cuda.synchronize()
        # the workspace holds the absorbed queries, then per split the bf16 mixes and the fp32
        # maxima and sums of every (row, head), then 256 bytes of diagnostics
        n_split = round((ws.numel() - 256 - B * 128 * 576 * 2) / (B * 128 * (512 * 2 + 8)))
        rerun = {"ms_per_step": start.elapsed_time(stop) / n_r, "steps": n_r,
                 "splits_rerun_per_call": diag["reruns"], "splits_per_call": n_split,
                 "case": "W_UK = 0, softmax scale 10 (scores spread over hundreds of log2 units)"}
        del ws_r, wz

    # the prefill chunk in both forms, reported beside the headline (not part of it); after
    # the decode passes, so that the decode's own kernels come first in a trace
    prefill_extra = None
    if not args.no_prefill_extras:
        inp = synth.prefill_inputs(synth.CONFIGS["prefill_s4096"])
        prefill_extra = {"workload": "prefill chunk S=4096, T=4096, k=min(t+1, 2048), 128 heads, bf16, "
                                     "20 calls after 3 warmup calls",
                         "unit": "ms per chunk; algorithmic TFLOP/s; fraction of the bf16 MFMA peak"}
        for form in ("latent", "explicit"):
            m = prefill_measure(torch, synth, mla, form == "explicit", 20, 3, inp)
            tf = m["flop"] / m["sec"] / 1e12
            prefill_extra[form] = {"ms_per_step": m["sec"] * 1e3, "tflops": tf, "frac": tf / BF16_PEAK_TFLOPS,
                                   "flop": m["flop"]}

    units = B * k
    achieved = units * ROW_BYTES / (attn_avg_ms * 1e-3) / 1e9
    traffic, step_traffic = traffic_from_profile()
    roof_bytes = step_bytes(B, k)
    t_hbm_ms = roof_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
    t_mfma_ms = step_flops(B, k) / (BF16_PEAK_TFLOPS * 1e12) * 1e3
    t_roof_ms = max(t_hbm_ms, t_mfma_ms)
    step_achieved = roof_bytes / (ms * 1e-3) / 1e9

    result = {
        "metric": "selected KV positions/s (sparse MLA decode B=64 T=32K k=2048)",
        "value": units / (ms * 1e-3),
        "unit": "selected KV positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic: seeded N(0,1) queries, RMS-normalised latent rows, uniform top-k "
                f"indices; {args.sets} rotating query/index/weight sets over one resident cache",
        "config": {"workload": "sparse_b64_t32k: decode B=64, T=32768, k=2048, 128 heads, bf16",
                   "B": B, "T": T, "k": k, "heads": 128, "parallelism": "none (1 GPU)"},
        "step_roofline": {"bound": "hbm" if t_hbm_ms >= t_mfma_ms else "mfma", "achieved": step_achieved,
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": t_roof_ms / ms,
                          "traffic": step_traffic, "algorithmic_bytes": roof_bytes,
                          "scope": "whole decode call (W_UK absorb, attention, merge + W_UV) per step"},
        "step_roofline_frac": t_roof_ms / ms,
        "ms_per_step_forced_rerun": rerun,
        "attention_kernel_ms": attn_avg_ms,
        "attention_kernel_ms_p10_p50_p90": attn_pct,
        "ms_per_step_mall_flushed": flushed_ms,
        "ms_per_step_with_attention_events": ms_events,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "prefill_s4096": prefill_extra,
    }
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 2 ** 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        base, extra = cpu_baseline(cfg, args.cpu_rows)
        result["cpu_baseline"] = base
        result.update(extra)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
