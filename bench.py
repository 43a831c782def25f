#!/usr/bin/env python3
"""Throughput of the PLE n-gram embedding path on one MI355X.

A step is one ple_forward over one batch of the workload (n-gram IDs ->
gather/dequant from the 51.2 GB FP8 table in HBM -> projection -> gate /
short conv / residual add). The default workload is the 32,768-token Zipf
prefill, the one the gather roofline target is stated for; --workload picks
another (tiny, decode, ragged, long). Inputs are resident in HBM before the
timed region; the timed region is K back-to-back steps between two device
synchronizations.

Printed: one JSON line with the step throughput (tokens/s), the roofline of
the dominant kernel measured with HIP events inside the same run, per-stage
durations, and the CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "PLE fused tokens/s (hash+gather+dequant+proj+fuse); gather HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
D = 2560

# Algorithmic bytes / flop per unit (one token, or one valid lookup).
#  gather: per valid lookup 2560 B of codes + 4 B scale; per token 8 B of row
#          ids read and 5120 B of bf16 x written
#  proj:   2 * 2560 * 2560 flop per token
#  fuse:   per token h 5120 B + e 5120 B read, out 5120 B written
#  hash:   per token 4 B token read (+ history), 8 B ids written
GATHER_BYTES_PER_LOOKUP = 2560 + 4
GATHER_BYTES_PER_TOKEN = 8 + 2 * D
# 16-lookup layout: per valid head lookup 160 B of codes + 4 B scale; per
# token 64 B of row ids and 5120 B of bf16 x
HEADS_BYTES_PER_LOOKUP = 160 + 4
HEADS_BYTES_PER_TOKEN = 64 + 2 * D
# NVFP4 table: per valid lookup 1280 B of E2M1 codes + 160 B of E4M3 block
# scales + 4 B row scale; per token as the FP8 table
NVFP4_BYTES_PER_LOOKUP = D // 2 + D // 16 + 4
PROJ_FLOP_PER_TOKEN = 2 * D * D
FUSE_BYTES_PER_TOKEN = 3 * 2 * D


KERNEL_SOURCES = {
    "proj_kernel": ["sparse_memory_gather_amd/csrc/ple_proj.hip", "sparse_memory_gather_amd/csrc/ple_kernels.h"],
    "proj_w320_kernel": ["sparse_memory_gather_amd/csrc/ple_proj.hip",
                         "sparse_memory_gather_amd/csrc/ple_kernels.h"],
    "gather_kernel": ["sparse_memory_gather_amd/csrc/ple_gather.hip", "sparse_memory_gather_amd/csrc/ple_kernels.h"],
    "gather_heads_kernel": ["sparse_memory_gather_amd/csrc/ple_gather.hip",
                            "sparse_memory_gather_amd/csrc/ple_kernels.h"],
    "gather_nvfp4_kernel": ["sparse_memory_gather_amd/csrc/ple_gather.hip",
                            "sparse_memory_gather_amd/csrc/ple_kernels.h"],
    "fuse_stream_kernel": ["sparse_memory_gather_amd/csrc/ple_fuse.hip",
                           "sparse_memory_gather_amd/csrc/ple_kernels.h"],
}


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary
    (profiles/hbm_traffic_<workload>.md), or None when there is none or the
    kernel's source has changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    h = hashlib.sha256()
    for src in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    digest = h.hexdigest()[:16]
    with open(path) as f:
        for line in f:
            m = re.match(r"traffic: kernel=(\S+) source_sha256=(\S+) bytes_per_launch=(\d+)", line.strip())
            if m and m.group(1) == kernel and m.group(2) == digest:
                return int(m.group(3))
    return None


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, stream) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventSynchronize(b) == 0
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)


def describe(name, wl, layout="two"):
    if layout == "heads":
        return describe(name, wl) + ", read as 16 head tables of 160-byte rows (16 lookups per token)"
    if layout == "nvfp4":
        return (describe(name, wl).replace("FP8 E4M3 table (51.2 GB)", "NVFP4 table (28.9 GB)")
                .replace("FP8 table", "NVFP4 table")
                + "; NVFP4 rows: 1280 B of E2M1 codes, 160 E4M3 scales per 16 elements, fp32 row scale")
    T = len(wl.chunks[0][0])
    if name == "prefill":
        return f"prefill: 1 sequence x 32768 Zipf(1.1) tokens, {wl.R:,}-row x 2560 FP8 E4M3 table (51.2 GB) in HBM"
    if name == "ragged":
        return f"ragged prefill: 64 sequences x 256 uniform tokens, {wl.R:,}-row FP8 table in HBM"
    if name == "decode":
        return f"decode: 8 sequences x 1 token per step after 4096-token histories, {wl.R:,}-row FP8 table in HBM"
    if name == "long":
        return f"long context: 262144 tokens as 16 x 16384-token chunks with carried state, {wl.R:,}-row FP8 table"
    return f"tiny: 1 x {T} uniform tokens, {wl.R:,}-row FP8 table"


def cpu_baseline(wl, name, W, cw, h0, budget_s=12.0, layout="two"):
    """The CPU oracle (as it stands) on the first N tokens of the workload's
    first chunk, N sized so that the run takes about `budget_s` seconds."""
    import numpy as np

    import oracle
    from gen import table

    toks, cu = wl.chunks[0]
    S = len(cu) - 1

    def run(n):
        # the first n tokens, cut at the same sequence boundaries
        cut = np.minimum(cu, n).astype(np.int32)
        t0 = time.perf_counter()
        if layout == "nvfp4":
            oracle.forward_nvfp4(toks[:n], cut, h0[:n], W, cw, wl.R, table.nvfp4_rows_cpu,
                                 np.zeros((S, 2), np.int32), np.zeros(S, np.int32), np.zeros((S, 3, D)))
        elif layout == "heads":
            oracle.forward_heads(toks[:n], cut, h0[:n], W, cw, wl.R,
                                 lambda hs, rs: table.slices_cpu(hs, rs, wl.R),
                                 np.zeros((S, 2), np.int32), np.zeros(S, np.int32), np.zeros((S, 3, D)))
        else:
            oracle.forward(toks[:n], cut, h0[:n], W, cw, wl.R, table.rows_cpu,
                           np.zeros((S, 2), np.int32), np.zeros(S, np.int32), np.zeros((S, 3, D)))
        return time.perf_counter() - t0

    T = len(toks)
    probe = min(64, T)
    tp = run(probe)
    n = int(min(T, max(probe, round(probe * budget_s / max(tp, 1e-6) / 64) * 64)))
    dt = run(n)
    result = {"value": round(n / dt, 2), "unit": "tokens/s", "cores": oracle.num_threads(),
              "kind": "oracle",
              "sample": f"first {n} of {T} tokens of the {name} workload's first chunk, one call "
                        f"({dt:.1f} s); table rows rebuilt on demand by the CPU generator"}
    # the same oracle on one thread, a smaller sample (about a quarter of the budget)
    threads = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        n1 = int(min(T, max(probe, round(n / max(threads, 1) / 4 / 64) * 64)))
        dt1 = run(n1)
    finally:
        oracle.set_num_threads(threads)
    result["single_thread"] = {"value": round(n1 / dt1, 2), "unit": "tokens/s",
                               "sample": f"first {n1} tokens, one call ({dt1:.1f} s)"}
    result["host"] = host_description()
    return result


def host_description():
    """CPU model, logical CPUs and memory of the machine the oracle ran on."""
    model, mem_gb = None, None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    mem_gb = round(int(line.split()[1]) / 2 ** 20, 1)
                    break
    except OSError:
        pass
    return {"cpu": model, "logical_cpus": os.cpu_count(), "mem_gib": mem_gb}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill", choices=["tiny", "decode", "prefill", "ragged", "long"])
    ap.add_argument("--overlap", action="store_true",
                    help="long workload: IDs and rows of the next chunk on a second stream (ple_forward_x)")
    ap.add_argument("--layout", default="two", choices=["two", "heads", "nvfp4"],
                    help="two: 2 lookups of 2560-byte FP8 rows per token; heads: 16 lookups of 160-byte "
                         "rows; nvfp4: 2 lookups of NVFP4 rows (E2M1 codes, E4M3 scale per 16 elements)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="also time a plain device copy of the gather's output size (x bytes read, "
                         "x bytes written) after a 1 GiB cache flush: the rate an HBM-bound kernel "
                         "moving the gather's bytes could reach")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.exit("bench.py measures one GPU: the path runs on a single MI355X (how it would shard "
                 "across GPUs is described, not implemented), so --gpus must be 1")

    import numpy as np
    import torch

    import sparse_memory_gather_amd as ple
    from gen import inputs, table

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ple.load_library()
    name = args.workload
    wl = inputs.make_workload(name, decode_steps=max(1, args.steps + args.warmup))
    W, cw = inputs.weights()

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    print(f"[bench] {name}: generating the {wl.R:,}-row table", file=sys.stderr, flush=True)
    heads = args.layout == "heads"
    nvfp4 = args.layout == "nvfp4"
    blocks = None
    if nvfp4:
        tab, blocks, sc = table.nvfp4_gpu(wl.R, device=dev)
    else:
        tab, sc = table.table_gpu(wl.R, device=dev)
    if heads:
        sc = table.head_scales_gpu(wl.R, device=dev)
    Wd, cwd = bf16(W), bf16(cw)
    ws = ple.Workspace(dev)

    # batches, all resident on the device before timing
    batches = []
    if name == "long":
        for i, (t, c) in enumerate(wl.chunks):
            batches.append((torch.from_numpy(t).to(dev), torch.from_numpy(c).to(dev), bf16(wl.hidden(i))))
    elif name == "decode":
        for i, (t, c) in enumerate(wl.chunks):
            batches.append((torch.from_numpy(t).to(dev), torch.from_numpy(c).to(dev), bf16(wl.hidden(i))))
    else:
        t, c = wl.chunks[0]
        batches.append((torch.from_numpy(t).to(dev), torch.from_numpy(c).to(dev), bf16(wl.hidden(0))))
    h0 = wl.hidden(0) if name != "long" else None
    state = ple.State(wl.S, dev)
    if name == "decode":
        hist = wl.history[0]
        hh = bf16(wl.history_hidden(hist.size))
        cu_h = torch.arange(0, hist.size + 1, hist.shape[1], dtype=torch.int32, device=dev)
        ple.ple_forward(torch.from_numpy(hist.reshape(-1)).to(dev), cu_h, tab, sc, Wd, cwd, hh, state,
                        workspace=ws, heads=heads, nvfp4_blocks=blocks)
        del hh
    outs = [torch.empty_like(b[2]) for b in batches] if name in ("long", "decode") else \
        [torch.empty_like(batches[0][2])]
    for b in batches:
        ws.get(b[0].numel(), b[1].numel() - 1)

    if name == "long" and args.overlap:
        # IDs and rows of chunk i+1 on a side stream while chunk i is
        # projected and fused (ple_forward_x); each chunk's n-gram history
        # comes from the token stream, two x buffers alternate
        side = torch.cuda.Stream(device=dev)
        n_ids = 16 if heads else 2
        hists = []
        for i, (t, c) in enumerate(wl.chunks):
            prev = wl.chunks[i - 1][0]      # chunk 0 continues from chunk 15 of the previous step
            hists.append(torch.from_numpy(prev[-2:].reshape(1, 2).astype(np.int32)).to(dev))
        hl2 = torch.full((1,), 2, dtype=torch.int32, device=dev)
        hl0 = torch.zeros((1,), dtype=torch.int32, device=dev)
        T_chunk = batches[0][0].numel()
        xbuf = [torch.empty((T_chunk, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
        rbuf = [torch.empty((T_chunk, n_ids), dtype=torch.int32, device=dev) for _ in range(2)]
        free = [torch.cuda.Event() for _ in range(2)]
        ready = [torch.cuda.Event() for _ in range(2)]
        # both sides on streams of their own: the legacy default stream would
        # serialize them
        main = torch.cuda.Stream(device=dev)
        main.wait_stream(torch.cuda.current_stream(dev))
        for e in free:
            e.record(main)

        def step(k, events=None):
            for i, ((t, c, h), o) in enumerate(zip(batches, outs)):
                j = i % 2
                with torch.cuda.stream(side):
                    side.wait_event(free[j])
                    hl = hl0 if (k == 0 and i == 0) else hl2
                    ple.ple_hash(t, c, hists[i], hl, wl.R, row_ids=rbuf[j], heads=heads)
                    if nvfp4:
                        ple.ple_lookup_nvfp4(rbuf[j], tab, blocks, sc, x=xbuf[j])
                    else:
                        ple.ple_lookup(rbuf[j], tab, sc, x=xbuf[j], heads=heads)
                    ready[j].record(side)
                with torch.cuda.stream(main):
                    main.wait_event(ready[j])
                    ple.ple_forward_x(xbuf[j], t, c, Wd, cwd, h, state, out=o, workspace=ws)
                    free[j].record(main)
        tokens_per_step = sum(b[0].numel() for b in batches)
    else:
        # one prepared call per fixed set of buffers (each long chunk, each
        # decode step's batch, the single prefill/ragged/tiny batch): the
        # argument checks and marshalling happen once, outside the timing
        calls = [ple.Forward(t, c, tab, sc, Wd, cwd, h, state, out=o, workspace=ws, heads=heads,
                             nvfp4_blocks=blocks) for (t, c, h), o in zip(batches, outs)]
        if name == "long":
            def step(k, events=None):
                for call in calls:
                    call(events=events)
            tokens_per_step = sum(b[0].numel() for b in batches)
        else:
            def step(k, events=None):
                calls[k % len(calls)](events=events)
            tokens_per_step = batches[0][0].numel()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    value = tokens_per_step * args.steps / wall

    # per-kernel durations inside the real forward: events around each kernel
    hev = HipEvents()
    stream = torch.cuda.current_stream().cuda_stream
    n_calls = len(batches) if name == "long" else 1
    reps = args.steps
    ev = [hev.create(5) for _ in range(reps * n_calls)]
    torch.cuda.synchronize()
    for k in range(reps):
        if name == "long":
            for j, (t, c, h) in enumerate(batches):
                (calls[j] if not args.overlap else
                 ple.Forward(t, c, tab, sc, Wd, cwd, h, state, out=outs[j], workspace=ws, heads=heads,
                             nvfp4_blocks=blocks))(events=ev[k * n_calls + j])
        else:
            step(k, events=ev[k])
    torch.cuda.synchronize()
    per_launch = np.array([[hev.elapsed_ms(e[i], e[i + 1]) for i in range(4)] for e in ev])
    stage_us = 1e3 * per_launch.mean(axis=0)  # average per launch
    stage_med_us = 1e3 * np.median(per_launch, axis=0)
    tokens_per_call = tokens_per_step / n_calls

    # the same kernels cold: before each step a 1 GiB buffer is read (a max,
    # so no dirty lines are left to write back and nothing is converted),
    # which evicts the L2s and the 256 MB Infinity Cache, so no table row can
    # be served from a cache filled by the previous step
    cold_us = None
    if name in ("prefill", "ragged", "tiny"):
        flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        sink = torch.zeros(reps, dtype=torch.uint8, device=dev)
        ev_cold = [hev.create(5) for _ in range(reps)]
        torch.cuda.synchronize()
        for k in range(reps):
            torch.amax(flush, dim=0, out=sink[k])
            step(k, events=ev_cold[k])
        torch.cuda.synchronize()
        cold_us = 1e3 * np.array([[hev.elapsed_ms(e[i], e[i + 1]) for i in range(4)] for e in ev_cold]).mean(axis=0)
        assert int(sink.sum().item()) == reps
        del flush, sink

    # valid lookups per call (for the gather's algorithmic bytes)
    rid = ple.ple_hash(batches[0][0], batches[0][1], torch.zeros((wl.S, 2), dtype=torch.int32, device=dev),
                       torch.full((wl.S,), 2 if name == "decode" else 0, dtype=torch.int32, device=dev), wl.R,
                       heads=heads)
    n_ids = 16 if heads else 2
    lookups = int((rid >= 0).sum().item()) if name != "decode" else n_ids * batches[0][0].numel()
    if heads:   # distinct (head, row) pairs
        key = rid.to(torch.int64) + torch.arange(16, device=dev, dtype=torch.int64)[None, :] * wl.R
        unique_rows = int(torch.unique(key[rid >= 0]).numel()) if name != "decode" else None
    else:
        unique_rows = int(torch.unique(rid[rid >= 0]).numel()) if name != "decode" else None
    if heads:
        gather_bytes = lookups * HEADS_BYTES_PER_LOOKUP + tokens_per_call * HEADS_BYTES_PER_TOKEN
    elif nvfp4:
        gather_bytes = lookups * NVFP4_BYTES_PER_LOOKUP + tokens_per_call * GATHER_BYTES_PER_TOKEN
    else:
        gather_bytes = lookups * GATHER_BYTES_PER_LOOKUP + tokens_per_call * GATHER_BYTES_PER_TOKEN
    gather_gbs = gather_bytes / (stage_us[1] * 1e-6) / 1e9
    proj_flop = tokens_per_call * PROJ_FLOP_PER_TOKEN
    proj_tflops = proj_flop / (stage_us[2] * 1e-6) / 1e12
    fuse_bytes = tokens_per_call * FUSE_BYTES_PER_TOKEN
    fuse_gbs = fuse_bytes / (stage_us[3] * 1e-6) / 1e9

    gather_name = "gather_heads_kernel" if heads else "gather_nvfp4_kernel" if nvfp4 else "gather_kernel"
    dominant = int(np.argmax(stage_us))
    proj_name = ple.proj_tiling(int(tokens_per_call))
    if dominant == 2:
        roofline = {"kernel": f"ple_proj ({proj_name})", "bound": "mfma",
                    "achieved": round(proj_tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(proj_tflops / BF16_PEAK_TFLOPS, 4),
                    "traffic": recorded_traffic(proj_name, name),
                    "per_launch": {"flop": proj_flop, "avg_us": round(float(stage_us[2]), 2)}}
    elif dominant == 1:
        roofline = {"kernel": f"ple_gather_dequant ({gather_name})", "bound": "hbm",
                    "achieved": round(gather_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gather_gbs / HBM_PEAK_GBS, 4),
                    "traffic": recorded_traffic(gather_name, name),
                    "per_launch": {"bytes": gather_bytes, "avg_us": round(float(stage_us[1]), 2)}}
    else:
        k = ["ple_hash (hash_kernel)", "", "", "ple_gate_conv_fuse (fuse_stream_kernel / fuse_token_kernel)"][dominant]
        nb = fuse_bytes if dominant == 3 else tokens_per_call * 12
        gbs = nb / (stage_us[dominant] * 1e-6) / 1e9
        roofline = {"kernel": k, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "traffic": recorded_traffic("fuse_stream_kernel", name) if dominant == 3 else None,
                    "per_launch": {"bytes": nb, "avg_us": round(float(stage_us[dominant]), 2)}}

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": describe(name, wl, args.layout) + (
                       "; IDs and rows of the next chunk gathered on a second stream during the current one"
                       if args.overlap and name == "long" else ""), "name": name, "layout": args.layout,
                   "tokens_per_step": tokens_per_step,
                   "sequences": wl.S, "table_rows": wl.R,
                   "table_bytes": wl.R * (NVFP4_BYTES_PER_LOOKUP if nvfp4 else D + (64 if heads else 4))},
        "roofline": roofline,
        "stages_us": {"hash": round(float(stage_us[0]), 2), "gather": round(float(stage_us[1]), 2),
                      "proj": round(float(stage_us[2]), 2), "fuse": round(float(stage_us[3]), 2)},
        "stages_median_us": {k: round(float(v), 2) for k, v in zip(("hash", "gather", "proj", "fuse"),
                                                                    stage_med_us)},
        "gather": {"bound": "hbm", "achieved": round(gather_gbs, 1), "peak": HBM_PEAK_GBS,
                   "unit": "GB/s", "frac": round(gather_gbs / HBM_PEAK_GBS, 4),
                   "bytes_per_launch": gather_bytes, "lookups_per_launch": lookups,
                   "unique_rows_per_launch": unique_rows,
                   "traffic": recorded_traffic(gather_name, name)},
        "gather_cold": None if cold_us is None else {
            "avg_us": round(float(cold_us[1]), 2), "achieved": round(gather_bytes / (cold_us[1] * 1e-6) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gather_bytes / (cold_us[1] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "stages_us": {k: round(float(v), 2) for k, v in zip(("hash", "gather", "proj", "fuse"), cold_us)}},
        "proj": {"kernel": proj_name, "bound": "mfma", "achieved": round(proj_tflops, 2),
                 "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(proj_tflops / BF16_PEAK_TFLOPS, 4)},
        "fuse": {"bound": "hbm", "achieved": round(fuse_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(fuse_gbs / HBM_PEAK_GBS, 4)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and h0 is not None:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, name, W, cw, h0, args.cpu_budget, args.layout)
    elif not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        h0 = wl.hidden(0)
        result["cpu_baseline"] = cpu_baseline(wl, name, W, cw, h0, args.cpu_budget, args.layout)
    if args.copy_calibration:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE of this dispatch
        # calibrate the per-kernel counters to bytes
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 1 << 30
    if args.copy_ceiling:
        nbytes = int(tokens_per_call) * 2560 * 2
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        sink = torch.empty(12, dtype=torch.uint8, device=dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(12)]
        for k in range(12):
            torch.amax(flush, dim=0, out=sink[k])
            ev[k][0].record()
            dst.copy_(src)
            ev[k][1].record()
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in ev[2:]]
        avg = sum(us) / len(us)
        result["copy_ceiling"] = {"bytes": 2 * nbytes, "avg_us": round(avg, 2),
                                  "achieved": round(2 * nbytes / avg * 1e-3, 1), "unit": "GB/s",
                                  "kernel": "torch copy_ (uint8, contiguous)"}
        del src, dst, flush, sink
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
