#!/usr/bin/env python3
"""Throughput of the PLE n-gram embedding path on one MI355X.

A step is one ple_forward over one batch of the workload (n-gram IDs ->
gather/dequant from the 51.2 GB FP8 table in HBM -> projection -> gate /
short conv / residual add). The headline workload is the 32,768-token Zipf
prefill, the one the gather roofline target is stated for; --workload picks
another (tiny, decode, ragged, long). Inputs are resident in HBM before the
timed region; the timed region is K back-to-back steps between two device
synchronizations.

Printed: one JSON line with the step throughput (tokens/s), the roofline of
the dominant kernel measured with HIP events in the same run, per-stage
durations, the other four workloads measured the same way (per_config), and
the CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "PLE fused tokens/s (hash+gather+dequant+proj+fuse); gather HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
D = 2560

# Algorithmic bytes / flop per unit (one token, or one distinct table row).
#  gather: per distinct row read 2560 B of codes + 4 B scale (a row looked up
#          twice needs to come from HBM once); per token 8 B of row ids read
#          and 5120 B of bf16 x written
#  proj:   2 * 2560 * 2560 flop per token; W (13,107,200 B) read once per call
#  fuse:   per token h 5120 B + e 5120 B read, out 5120 B written
#  hash:   per token 4 B token read (+ history), 8 B ids written
GATHER_BYTES_PER_ROW = 2560 + 4
GATHER_BYTES_PER_TOKEN = 8 + 2 * D
# 16-lookup layout: per distinct (head, row) 160 B of codes + 4 B scale; per
# token 64 B of row ids and 5120 B of bf16 x
HEADS_BYTES_PER_ROW = 160 + 4
HEADS_BYTES_PER_TOKEN = 64 + 2 * D
# NVFP4 table: per distinct row 1280 B of E2M1 codes + 160 B of E4M3 block
# scales + 4 B row scale; per token as the FP8 table
NVFP4_BYTES_PER_ROW = D // 2 + D // 16 + 4
PROJ_FLOP_PER_TOKEN = 2 * D * D
W_BYTES = D * D * 2
FUSE_BYTES_PER_TOKEN = 3 * 2 * D
STATE_BYTES_PER_SEQ = 3 * D * 4   # the carried conv state of one sequence (fp32)

# the other workloads of the same run: (name, timed steps, warm-up steps)
PER_CONFIG = (("tiny", 50, 10), ("decode", 64, 8), ("ragged", 20, 5), ("long", 4, 1))

_CSRC = "sparse_memory_gather_amd/csrc/"
_PROJ_SRC = [_CSRC + f for f in ("ple_proj.hip", "ple_fragments.h", "ple_kernels.h")]
_GATHER_SRC = [_CSRC + f for f in ("ple_gather.hip", "ple_dequant.h", "ple_ngram.h", "ple_kernels.h")]
_FUSE_SRC = [_CSRC + f for f in ("ple_fuse.hip", "ple_fuse_common.h", "ple_ngram.h", "ple_kernels.h")]
_DECODE_SRC = [_CSRC + f for f in ("ple_decode.hip", "ple_dequant.h", "ple_fragments.h", "ple_fuse_common.h",
                                   "ple_ngram.h", "ple_kernels.h")]
# every file a kernel is compiled from: a recorded traffic figure holds only
# while their contents are unchanged
KERNEL_SOURCES = {
    "proj_kernel": _PROJ_SRC, "proj_w320_kernel": _PROJ_SRC,
    "gather_kernel": _GATHER_SRC, "gather_heads_kernel": _GATHER_SRC, "gather_nvfp4_kernel": _GATHER_SRC,
    "fuse_stream_kernel": _FUSE_SRC, "decode_step_kernel": _DECODE_SRC,
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


def mem_available_gib():
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable"):
                    return int(line.split()[1]) / 2 ** 20
    except OSError:
        pass
    return 0.0


def cpu_baseline(wl, name, W, cw, h0, budget_s=12.0, layout="two", dev_table=None):
    """The CPU oracle (as it stands) on the first N tokens of the workload's
    first chunk, N sized so that the run takes about `budget_s` seconds.
    With dev_table (the FP8 table and scales in HBM) and enough host memory,
    the oracle reads its rows from a host-resident copy of the table's bytes
    (copied before timing); otherwise the CPU generator rebuilds the rows a
    call needs inside the call."""
    import oracle
    from gen import table

    toks, cu = wl.chunks[0]
    S = len(cu) - 1
    row_source, source = table.rows_cpu, "table rows rebuilt on demand by the CPU generator inside the call"
    host = None
    if layout == "two" and dev_table is not None:
        nbytes = dev_table[0].numel() + 4 * dev_table[1].numel()
        if mem_available_gib() * 2 ** 30 > 1.5 * nbytes:
            print(f"[bench] copying the {nbytes / 1e9:.1f} GB table to host memory", file=sys.stderr, flush=True)
            host = (dev_table[0].cpu().numpy(), dev_table[1].cpu().numpy())
            row_source = lambda ids: (host[0][ids], host[1][ids])
            source = f"rows read from a host-resident copy of the {nbytes / 1e9:.1f} GB table"

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
            oracle.forward(toks[:n], cut, h0[:n], W, cw, wl.R, row_source,
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
                        f"({dt:.1f} s); {source}"}
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
    del host
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


class Context:
    """Device, weights and tables shared by the workloads of one run; the
    51.2 GB table is generated once."""

    def __init__(self, dev):
        import torch

        from gen import inputs
        self.dev = dev
        self.W, self.cw = inputs.weights()

        def bf16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        self.bf16 = bf16
        self.Wd, self.cwd = bf16(self.W), bf16(self.cw)
        self._tables = {}
        self.hev = HipEvents()

    def table(self, R, layout):
        """(table, scales, nvfp4 blocks or None) for R rows in the layout."""
        from gen import table
        key = (R, layout)
        if key not in self._tables:
            print(f"[bench] generating the {R:,}-row {layout} table", file=sys.stderr, flush=True)
            if layout == "nvfp4":
                codes, blocks, sc = table.nvfp4_gpu(R, device=self.dev)
                self._tables[key] = (codes, sc, blocks)
            elif layout == "heads":
                tab, _, _ = self.table(R, "two")
                self._tables[key] = (tab, table.head_scales_gpu(R, device=self.dev), None)
            else:
                tab, sc = table.table_gpu(R, device=self.dev)
                self._tables[key] = (tab, sc, None)
        return self._tables[key]

    def drop_tables(self, keep_R):
        import torch
        for k in [k for k in self._tables if k[0] != keep_R]:
            del self._tables[k]
        torch.cuda.empty_cache()


def measure(ctx, name, layout, steps, warmup, overlap=False, graph=False, cold=True, warmup_ms=100.0,
            inplace=False, staged=False):
    """Time `steps` steps of workload `name` after `warmup` steps. Returns the
    workload's figures: tokens/s from wall time and from events around the
    timed loop, per-stage averages and medians from a second pass with
    events around each kernel, the gather's bytes, and (cold) the same
    stages with the caches flushed before each step."""
    import torch

    import sparse_memory_gather_amd as ple
    from gen import inputs

    dev, hev = ctx.dev, ctx.hev
    wl = inputs.make_workload(name, decode_steps=max(1, steps + warmup))
    n_batches = len(wl.chunks)
    heads, nvfp4 = layout == "heads", layout == "nvfp4"
    tab, sc, blocks = ctx.table(wl.R, layout)
    Wd, cwd, bf16 = ctx.Wd, ctx.cwd, ctx.bf16
    ws = ple.Workspace(dev)

    # batches, all resident on the device before timing
    print(f"[bench] {name}: inputs", file=sys.stderr, flush=True)
    batches = []
    if name in ("long", "decode"):
        for i, (t, c) in enumerate(wl.chunks):
            batches.append((torch.from_numpy(t).to(dev), torch.from_numpy(c).to(dev), bf16(wl.hidden(i))))
    else:
        t, c = wl.chunks[0]
        batches.append((torch.from_numpy(t).to(dev), torch.from_numpy(c).to(dev), bf16(wl.hidden(0))))
    state = ple.State(wl.S, dev)
    if name == "decode":
        hist = wl.history[0]
        hh = bf16(wl.history_hidden(hist.size))
        cu_h = torch.arange(0, hist.size + 1, hist.shape[1], dtype=torch.int32, device=dev)
        ple.ple_forward(torch.from_numpy(hist.reshape(-1)).to(dev), cu_h, tab, sc, Wd, cwd, hh, state,
                        workspace=ws, heads=heads, nvfp4_blocks=blocks)
        del hh
    outs = [torch.empty_like(b[2]) for b in batches]
    for b in batches:
        ws.get(b[0].numel(), b[1].numel() - 1, heads)
    n_calls = len(batches) if name == "long" else 1
    tokens_per_step = sum(b[0].numel() for b in batches) if name == "long" else batches[0][0].numel()
    stream = torch.cuda.current_stream().cuda_stream

    # one prepared call per fixed set of buffers (each long chunk, each decode
    # step's batch, the single prefill/ragged/tiny batch): the argument
    # checks and marshalling happen once, outside the timing
    # (inplace: out == h; staged: every stage its own launch, also for the
    # short calls ple_forward runs as one)
    calls = [ple.Forward(t, c, tab, sc, Wd, cwd, h, state, out=h if inplace else o, workspace=ws, heads=heads,
                         nvfp4_blocks=blocks, staged=staged) for (t, c, h), o in zip(batches, outs)]

    def eager_step(k, events=None):
        if name == "long":
            for j, call in enumerate(calls):
                call(events=None if events is None else events[j])
        else:
            calls[k % len(calls)](events=None if events is None else events[0])

    if name == "long" and overlap:
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

        def step(k):
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
    elif graph:
        # each step's calls captured once into a HIP graph and replayed (the
        # forward records no memset and allocates nothing)
        eager_step(0)
        torch.cuda.synchronize()
        graphs = []
        for k in range(len(calls) if name != "long" else 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                eager_step(k)
            graphs.append(g)
        torch.cuda.synchronize()

        def step(k):
            graphs[k % len(graphs)].replay()
    else:
        def step(k):
            eager_step(k)

    # warm-up: at least `warmup` steps, and at least warmup_ms of GPU work
    # since the last idle period: from idle the clocks take some 10-20 ms to
    # ramp up, and a timed loop started earlier measures the ramp
    n_warm, t_warm = 0, time.perf_counter()
    while n_warm < warmup or (time.perf_counter() - t_warm) * 1e3 < warmup_ms:
        for _ in range(max(warmup, 1)):
            step(n_warm)
            n_warm += 1
        torch.cuda.synchronize()
    warmup = n_warm
    print(f"[bench] {name}: {warmup} warm-up steps, timing {steps} steps", file=sys.stderr, flush=True)
    loop_ev = hev.create(2)
    t0 = time.perf_counter()
    hev.record(loop_ev[0], stream)
    for k in range(steps):
        step(warmup + k)
    hev.record(loop_ev[1], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = hev.elapsed_ms(loop_ev[0], loop_ev[1])
    res = {"name": name, "layout": layout, "steps": steps, "warmup": warmup, "n_batches": n_batches,
           "tokens_per_step": tokens_per_step, "ms_per_step": 1e3 * wall / steps,
           "value": tokens_per_step * steps / wall, "gpu_ms_per_step": gpu_ms / steps,
           "workload": describe(name, wl, layout), "S": wl.S, "R": wl.R, "graph": graph}
    if graph or overlap or inplace or staged:
        return res

    # per-kernel durations inside the real forward: events around each kernel
    # (a second pass of the same steps, so that the event records do not
    # perturb the timed loop)
    ev = [[hev.create(5) for _ in range(n_calls)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        eager_step(warmup + k, events=ev[k])
    torch.cuda.synchronize()
    per_launch = np.array([[hev.elapsed_ms(e[i], e[i + 1]) for i in range(4)] for es in ev for e in es])
    res["stage_us"] = 1e3 * per_launch.mean(axis=0)
    res["stage_med_us"] = 1e3 * np.median(per_launch, axis=0)
    res["stage_min_us"] = 1e3 * per_launch.min(axis=0)
    res["stage_max_us"] = 1e3 * per_launch.max(axis=0)

    # the same kernels cold: before each call a 1 GiB buffer is read (a max,
    # so no dirty lines are left to write back and nothing is converted),
    # which evicts the L2s and the 256 MB Infinity Cache, so no table row can
    # be served from a cache filled by the previous step
    if cold:
        flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        n_cold = min(steps, 8) if name == "long" else steps
        sink = torch.zeros(n_cold * n_calls, dtype=torch.uint8, device=dev)
        ev_cold = [[hev.create(5) for _ in range(n_calls)] for _ in range(n_cold)]
        torch.cuda.synchronize()
        for k in range(n_cold):
            if name == "long":
                for j, call in enumerate(calls):
                    torch.amax(flush, dim=0, out=sink[k * n_calls + j])
                    call(events=ev_cold[k][j])
            else:
                torch.amax(flush, dim=0, out=sink[k])
                calls[(warmup + k) % len(calls)](events=ev_cold[k][0])
        torch.cuda.synchronize()
        cold = np.array([[hev.elapsed_ms(e[i], e[i + 1]) for i in range(4)] for es in ev_cold for e in es])
        res["cold_stage_us"] = 1e3 * cold.mean(axis=0)
        assert int(sink.sum().item()) == n_cold * n_calls
        del flush, sink

    # lookups and distinct rows per call (the gather's algorithmic bytes),
    # each call with the history it runs with
    lookups, uniq = [], []
    for i, (t, c, _) in enumerate(batches if name == "long" else batches[:1]):
        S = wl.S
        if name == "decode":
            hid = torch.from_numpy(wl.history[0][:, -2:].astype(np.int32)).to(dev)
            hl = torch.full((S,), 2, dtype=torch.int32, device=dev)
        elif name == "long" and i > 0:
            hid = torch.from_numpy(wl.chunks[i - 1][0][-2:].reshape(1, 2).astype(np.int32)).to(dev)
            hl = torch.full((1,), 2, dtype=torch.int32, device=dev)
        else:
            hid = torch.zeros((S, 2), dtype=torch.int32, device=dev)
            hl = torch.zeros((S,), dtype=torch.int32, device=dev)
        rid = ple.ple_hash(t, c, hid, hl, wl.R, heads=heads)
        valid = rid >= 0
        lookups.append(int(valid.sum().item()))
        key = rid.to(torch.int64)
        if heads:   # distinct (head, row) pairs
            key = key + torch.arange(16, device=dev, dtype=torch.int64)[None, :] * wl.R
        uniq.append(int(torch.unique(key[valid]).numel()))
    res["lookups_per_call"] = float(np.mean(lookups))
    res["distinct_rows_per_call"] = float(np.mean(uniq))
    res["tokens_per_call"] = tokens_per_step / n_calls
    res["proj_kernel"] = ple.proj_tiling(int(res["tokens_per_call"]))
    if layout == "two" and ple.one_launch(int(res["tokens_per_call"]), wl.S):
        # the whole path is one kernel, timed in the projection stage
        res["proj_kernel"] = "decode_step_kernel"
    del calls, batches, outs, ws, state
    torch.cuda.empty_cache()
    return res


def gather_stream(ctx, name, layout, batches=20):
    """The gather kernel over `batches` different batches of the workload's
    own shape and generator (the long workload: its 16 chunks), launched
    back to back after one untimed pass, with events around the loop only.
    A batch's rows are not those of the batch before, so for uniform tokens
    no row is served from a cache filled by an earlier launch; Zipf batches
    still share their most frequent rows. Bytes count each batch's distinct
    rows once. None for the short workloads (no gather of their own to
    time this way: a tiny table, or the rows read inside the one-launch
    decode kernel)."""
    import torch

    import sparse_memory_gather_amd as ple
    from gen import inputs

    if name not in ("prefill", "ragged", "long"):
        return None
    dev = ctx.dev
    heads, nvfp4 = layout == "heads", layout == "nvfp4"
    wl = inputs.make_workload(name)
    tab, sc, blocks = ctx.table(wl.R, layout)
    if name == "long":
        toks = [t for t, _ in wl.chunks]
        cu = wl.chunks[0][1]
    else:
        cu = wl.chunks[0][1]
        T = int(cu[-1])
        rng = np.random.Generator(np.random.PCG64([wl.seed, 0x5354]))
        gen = inputs.zipf_tokens if name == "prefill" else inputs.uniform_tokens
        toks = [gen(rng, T) for _ in range(batches)]
    S = len(cu) - 1
    per_row = HEADS_BYTES_PER_ROW if heads else NVFP4_BYTES_PER_ROW if nvfp4 else GATHER_BYTES_PER_ROW
    per_tok = HEADS_BYTES_PER_TOKEN if heads else GATHER_BYTES_PER_TOKEN
    cu_d = torch.from_numpy(cu).to(dev)
    rids, total = [], 0
    for i, t in enumerate(toks):
        if name == "long" and i > 0:
            hid = torch.from_numpy(toks[i - 1][-2:].reshape(1, 2).astype(np.int32)).to(dev)
            hl = torch.full((1,), 2, dtype=torch.int32, device=dev)
        else:
            hid = torch.zeros((S, 2), dtype=torch.int32, device=dev)
            hl = torch.zeros((S,), dtype=torch.int32, device=dev)
        rid = ple.ple_hash(torch.from_numpy(t).to(dev), cu_d, hid, hl, wl.R, heads=heads)
        valid = rid >= 0
        key = rid.to(torch.int64)
        if heads:
            key = key + torch.arange(16, device=dev, dtype=torch.int64)[None, :] * wl.R
        total += int(torch.unique(key[valid]).numel()) * per_row + len(t) * per_tok
        rids.append(rid)
    x = torch.empty((len(toks[0]), D), dtype=torch.bfloat16, device=dev)

    def run():
        for rid in rids:
            if nvfp4:
                ple.ple_lookup_nvfp4(rid, tab, blocks, sc, x=x)
            else:
                ple.ple_lookup(rid, tab, sc, x=x, heads=heads)

    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    run()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / len(rids)
    bytes_per = total / len(rids)
    return {"batches": len(rids), "avg_us": round(us, 2), "bytes_per_launch": int(bytes_per),
            "achieved": round(bytes_per / us * 1e-3, 1), "unit": "GB/s",
            "frac": round(bytes_per / us * 1e-3 / HBM_PEAK_GBS, 4),
            "timing": "events around back-to-back launches over different batches"}


def copy_ceiling(dev, total_bytes, reps=12):
    """A plain device copy moving `total_bytes` (half read, half written),
    timed like the gather: a 1 GiB read before each copy evicts the caches,
    and events bracket the one launch. The like-for-like ceiling for an
    HBM-bound kernel of that size measured that way."""
    import torch
    n = max(1, int(total_bytes) // 2)
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(reps, dtype=torch.uint8, device=dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for k in range(reps):
        torch.amax(flush, dim=0, out=sink[k])
        ev[k][0].record()
        dst.copy_(src)
        ev[k][1].record()
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1e3 for a, b in ev[2:]]
    avg = sum(us) / len(us)
    del src, dst, flush, sink
    return {"bytes": 2 * n, "avg_us": round(avg, 2), "achieved": round(2 * n / avg * 1e-3, 1), "unit": "GB/s",
            "frac": round(2 * n / avg * 1e-3 / HBM_PEAK_GBS, 4), "kernel": "torch copy_ (uint8, contiguous)"}


def vendor_gemm(dev, T, reps=20):
    """The projection's product through torch (hipBLASLt on ROCm): bf16
    x [T][2560] times W^T as a contiguous [2560][2560] operand, bf16 out,
    events around each call, after a warm-up. A reference point for the MFMA
    kernel on the same shape, not part of the path."""
    import torch
    g = torch.Generator(device=dev).manual_seed(7)
    x = torch.randn((T, D), device=dev, generator=g).to(torch.bfloat16)
    wt = (torch.randn((D, D), device=dev, generator=g) * D ** -0.5).to(torch.bfloat16).contiguous()
    out = torch.empty((T, D), dtype=torch.bfloat16, device=dev)
    for _ in range(5):
        torch.mm(x, wt, out=out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        torch.mm(x, wt, out=out)
        b.record()
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    avg = sum(us) / len(us)
    tf = T * PROJ_FLOP_PER_TOKEN / avg * 1e-6
    del x, wt, out
    return {"op": "torch.mm bf16 (hipBLASLt)", "tokens": T, "avg_us": round(avg, 2),
            "median_us": round(us[len(us) // 2], 2), "achieved": round(tf, 2), "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4)}


def stage_table(res, key="stage_us"):
    """Per-stage durations (us) of a measure() result; a one-launch step has
    one stage, timed by the events around its timed loop."""
    if res["proj_kernel"] == "decode_step_kernel":
        return {"decode_step_kernel": round(1e3 * res["gpu_ms_per_step"], 2)}
    return {k: round(float(v), 2) for k, v in zip(("hash", "gather", "proj", "fuse"), res[key])}


def figures(res, layout):
    """Rooflines and rates from a measure() result."""
    tpc = res["tokens_per_call"]
    st = res["stage_us"]
    if layout == "heads":
        per_row, per_tok, gname = HEADS_BYTES_PER_ROW, HEADS_BYTES_PER_TOKEN, "gather_heads_kernel"
    elif layout == "nvfp4":
        per_row, per_tok, gname = NVFP4_BYTES_PER_ROW, GATHER_BYTES_PER_TOKEN, "gather_nvfp4_kernel"
    else:
        per_row, per_tok, gname = GATHER_BYTES_PER_ROW, GATHER_BYTES_PER_TOKEN, "gather_kernel"
    g_bytes = res["distinct_rows_per_call"] * per_row + tpc * per_tok
    g_bytes_all = res["lookups_per_call"] * per_row + tpc * per_tok
    gather = {"kernel": gname, "bound": "hbm", "achieved": round(g_bytes / st[1] * 1e-3, 1), "peak": HBM_PEAK_GBS,
              "unit": "GB/s", "frac": round(g_bytes / st[1] * 1e-3 / HBM_PEAK_GBS, 4),
              "bytes_per_launch": int(g_bytes), "avg_us": round(float(st[1]), 2),
              "median_us": round(float(res["stage_med_us"][1]), 2),
              "distinct_rows_per_launch": res["distinct_rows_per_call"],
              "lookups_per_launch": res["lookups_per_call"],
              "achieved_counting_every_lookup": round(g_bytes_all / st[1] * 1e-3, 1),
              "note": "bytes count each distinct row once; achieved_counting_every_lookup counts repeated "
                      "rows again (those can be served from L2 or the Infinity Cache)"}
    if "cold_stage_us" in res:
        c = res["cold_stage_us"][1]
        gather["cold"] = {"avg_us": round(float(c), 2), "achieved": round(g_bytes / c * 1e-3, 1),
                          "frac": round(g_bytes / c * 1e-3 / HBM_PEAK_GBS, 4)}
    if res["proj_kernel"] == "decode_step_kernel":
        # no gather kernel: the rows are read inside the one launch, whose
        # time the projection stage carries (the gather stage's events
        # bracket nothing but their own records)
        gather = {"kernel": None, "note": "rows read inside decode_step_kernel (one launch)",
                  "distinct_rows_per_launch": res["distinct_rows_per_call"],
                  "lookups_per_launch": res["lookups_per_call"]}
    flop = tpc * PROJ_FLOP_PER_TOKEN
    if res["proj_kernel"] == "decode_step_kernel":
        # one launch for the whole path: W once, the distinct rows, and per
        # token h in, out, and the carried conv state read and rewritten. A
        # step is that one launch, so the events around the timed loop give
        # its duration (launch gaps included); events around a single launch
        # would add their own records' cost to a ~20 us kernel
        pb = W_BYTES + res["distinct_rows_per_call"] * per_row + tpc * (4 * D + 2 * STATE_BYTES_PER_SEQ)
        us = 1e3 * res["gpu_ms_per_step"]
        proj = {"kernel": res["proj_kernel"], "bound": "hbm", "achieved": round(pb / us * 1e-3, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(pb / us * 1e-3 / HBM_PEAK_GBS, 4),
                "bytes_per_launch": int(pb), "avg_us": round(us, 2),
                "timing": "events around the timed loop of one-launch steps",
                "events_around_one_launch_us": round(float(st[2]), 2)}
    elif res["proj_kernel"] == "proj_small_kernel":
        # a few tokens: the kernel streams W once; its bound is HBM
        pb = W_BYTES + tpc * 4 * D
        proj = {"kernel": res["proj_kernel"], "bound": "hbm", "achieved": round(pb / st[2] * 1e-3, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(pb / st[2] * 1e-3 / HBM_PEAK_GBS, 4),
                "bytes_per_launch": int(pb), "avg_us": round(float(st[2]), 2),
                "median_us": round(float(res["stage_med_us"][2]), 2)}
    else:
        tf = flop / st[2] * 1e-6
        tf_med = flop / res["stage_med_us"][2] * 1e-6
        proj = {"kernel": res["proj_kernel"], "bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4), "flop_per_launch": int(flop),
                "avg_us": round(float(st[2]), 2), "median_us": round(float(res["stage_med_us"][2]), 2),
                "frac_of_median": round(tf_med / BF16_PEAK_TFLOPS, 4),
                "min_us": round(float(res["stage_min_us"][2]), 2),
                "max_us": round(float(res["stage_max_us"][2]), 2)}
    fb = tpc * FUSE_BYTES_PER_TOKEN
    fuse = {"bound": "hbm", "achieved": round(fb / st[3] * 1e-3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(fb / st[3] * 1e-3 / HBM_PEAK_GBS, 4), "bytes_per_launch": int(fb),
            "avg_us": round(float(st[3]), 2), "median_us": round(float(res["stage_med_us"][3]), 2)}
    if res["proj_kernel"] == "decode_step_kernel":
        fuse = {"kernel": None, "note": "gate, conv and residual add inside decode_step_kernel (one launch)"}
        roofline = dict(proj)
        roofline["stage"] = "whole step"
        return gather, proj, fuse, roofline
    dominant = int(np.argmax(st[1:])) + 1
    roofline = dict([gather, proj, fuse][dominant - 1])
    roofline["stage"] = ["gather", "proj", "fuse"][dominant - 1]
    return gather, proj, fuse, roofline


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps before the timed loop (at least; see --warmup-ms)")
    ap.add_argument("--warmup-ms", type=float, default=100.0,
                    help="keep warming up until this much GPU work has run, so that the clocks have ramped up")
    ap.add_argument("--workload", default="prefill", choices=["tiny", "decode", "prefill", "ragged", "long"])
    ap.add_argument("--overlap", action="store_true",
                    help="long workload: IDs and rows of the next chunk on a second stream (ple_forward_x)")
    ap.add_argument("--graph", action="store_true",
                    help="capture each step's calls into a HIP graph once and time graph replays")
    ap.add_argument("--layout", default="two", choices=["two", "heads", "nvfp4"],
                    help="two: 2 lookups of 2560-byte FP8 rows per token; heads: 16 lookups of 160-byte "
                         "rows; nvfp4: 2 lookups of NVFP4 rows (E2M1 codes, E4M3 scale per 16 elements)")
    ap.add_argument("--no-per-config", action="store_true", help="time only the selected workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.exit("bench.py measures one GPU: the path runs on a single MI355X (how it would shard "
                 "across GPUs is described, not implemented), so --gpus must be 1")

    import torch

    import sparse_memory_gather_amd as ple
    from gen import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ple.load_library()
    ctx = Context(dev)
    name = args.workload
    head = measure(ctx, name, args.layout, args.steps, args.warmup, overlap=args.overlap, graph=args.graph,
                   warmup_ms=args.warmup_ms)
    result = {
        "metric": METRIC, "value": round(head["value"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": head["warmup"], "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": head["workload"] + (
                       "; IDs and rows of the next chunk gathered on a second stream during the current one"
                       if args.overlap and name == "long" else "") + (
                       "; each step replayed from a captured HIP graph" if args.graph else ""),
                   "name": name, "layout": args.layout, "tokens_per_step": head["tokens_per_step"],
                   "sequences": head["S"], "table_rows": head["R"],
                   "table_bytes": head["R"] * (NVFP4_BYTES_PER_ROW if args.layout == "nvfp4"
                                               else D + (64 if args.layout == "heads" else 4))},
        "gpu_ms_per_step": round(head["gpu_ms_per_step"], 4),
    }
    if "stage_us" in head:
        gather, proj, fuse, roofline = figures(head, args.layout)
        roofline["traffic"] = recorded_traffic(roofline["kernel"], name)
        gather["traffic"] = recorded_traffic(gather["kernel"], name)
        result["roofline"] = roofline
        result["stages_us"] = stage_table(head)
        result["stages_median_us"] = stage_table(head, "stage_med_us")
        if gather.get("kernel"):
            gather["copy_same_bytes"] = copy_ceiling(dev, gather["bytes_per_launch"])
            gather["stream"] = gather_stream(ctx, name, args.layout)
        if proj.get("bound") == "mfma":
            proj["vendor_gemm_same_shape"] = vendor_gemm(dev, int(head["tokens_per_call"]))
        result["gather"], result["proj"], result["fuse"] = gather, proj, fuse
    result["cpu_baseline"] = None

    if not args.no_per_config and name == "prefill" and not args.graph and not args.overlap:
        # the other workloads in the same run, each with its own timed loop
        per = {}
        for wname, st, wu in PER_CONFIG:
            r = measure(ctx, wname, args.layout, st, wu, warmup_ms=args.warmup_ms)
            g, p, f, rf = figures(r, args.layout)
            per[wname] = {"value": round(r["value"], 1), "unit": "tokens/s", "ms_per_step": round(r["ms_per_step"], 4),
                          "gpu_ms_per_step": round(r["gpu_ms_per_step"], 4), "steps": st, "warmup": r["warmup"],
                          "tokens_per_step": r["tokens_per_step"], "workload": r["workload"],
                          "dominant": dict({k: rf[k] for k in ("stage", "kernel", "bound", "achieved", "peak",
                                                               "unit", "frac") if k in rf},
                                           traffic=recorded_traffic(rf["kernel"], wname)),
                          "stages_us": stage_table(r),
                          "gather": {k: g[k] for k in ("achieved", "frac", "cold", "distinct_rows_per_launch",
                                                       "lookups_per_launch", "achieved_counting_every_lookup",
                                                       "note") if k in g}}
            if g.get("kernel"):
                per[wname]["gather"]["copy_same_bytes"] = copy_ceiling(dev, g["bytes_per_launch"])
                per[wname]["gather"]["stream"] = gather_stream(ctx, wname, args.layout)
            if wname == "decode":
                rg = measure(ctx, "decode", args.layout, st, wu, graph=True, warmup_ms=args.warmup_ms)
                per[wname]["graph_replay"] = {"ms_per_step": round(rg["ms_per_step"], 4),
                                              "gpu_ms_per_step": round(rg["gpu_ms_per_step"], 4),
                                              "value": round(rg["value"], 1)}
                # the same steps in place (out == h), one launch as well; and
                # as three launches (ple_forward_staged: IDs in the gather,
                # small-T projection, one-token fuse)
                for key, kw in (("in_place", {"inplace": True}), ("three_launches", {"staged": True})):
                    r3 = measure(ctx, "decode", args.layout, st, wu, warmup_ms=args.warmup_ms, **kw)
                    per[wname][key] = {"ms_per_step": round(r3["ms_per_step"], 4),
                                       "gpu_ms_per_step": round(r3["gpu_ms_per_step"], 4),
                                       "value": round(r3["value"], 1)}
            ctx.drop_tables(inputs.R_FULL)
        result["per_config"] = per

    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        wl = inputs.make_workload(name, decode_steps=1)
        dev_table = ctx.table(wl.R, "two")[:2] if args.layout == "two" else None
        result["cpu_baseline"] = cpu_baseline(wl, name, ctx.W, ctx.cw, wl.hidden(0), args.cpu_budget, args.layout,
                                              dev_table)
    if args.copy_calibration:
        # a plain copy of known size: FETCH_SIZE / WRITE_SIZE of this dispatch
        # calibrate the per-kernel counters to bytes
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 1 << 30
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
