#!/usr/bin/env python3
"""Packed mixed-bit GEMV benchmark on one MI355X.

Default workload: the 9B-class decoder stack at batch 1 -- 32 layers of
{q 4096x4096, k 1024x4096, v 1024x4096, o 4096x4096, gate 14336x4096,
up 14336x4096, down 4096x14336} plus an LM head 128256x4096. Widths per
64-weight group are drawn with p{1:.69, 2:.15, 4:.12, 8:.04} (LM head
p{1:.92, 2:.07, 4:.01}), W ~ N(0, 0.02^2) quantised on the GPU by vbq_pack,
x ~ N(0,1) in fp16, one x per projection (the stack is not chained).

One step = one decode token's worth of GEMVs: one batched launch per layer
(its 7 projections) and one launch for the LM head. Inputs are resident in
HBM when the timed region starts; the stack (2.1 GB) is far larger than the
on-chip caches, so every launch streams its weights from HBM.

Prints one JSON line (see the fields below).

Profiling helpers (same file, so every profile is made by committed code):
  --copy-calibration   after the measurement, run a plain device copy of
                       known size a few times; its FETCH_SIZE/WRITE_SIZE
                       readings calibrate the GEMV's counters.
  --summarize-trace D  (CPU only) summarise a rocprofv3 --kernel-trace run.
  --summarize-pmc F W  (CPU only) summarise a FETCH_SIZE run F and a
                       WRITE_SIZE run W into HBM bytes per GEMV launch.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "packed-weight GEMV: achieved HBM GB/s (% of peak) + µs/layer at batch 1"
PEAK_HBM_GBS = 8000.0          # MI355X published HBM3E bandwidth, decimal GB/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
KERNEL = "k_gemv"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(sizes, N, K, B, resid=False):
    """Bytes the method must move for one GEMV: packed codes (b bits per
    weight), fp16 scale + fp16 offset per group, the 2-bit width per group,
    x (fp16) and y (fp32), plus the fp16 residual when served."""
    groups = N * (K // 64)
    b = sizes.code_bits / 8 + 4 * groups + groups / 4 + 2 * B * K + 4 * B * N
    if resid:
        b += 2 * N * K
    return float(b)


class Stack:
    """Packed matrices of the 9B-class stack, their x and y buffers, and plans.
    The step's launches are vbq_gemv_batched_static calls (every k-tile of
    the 14336-wide down projection gets a workgroup); `batched_plans` holds
    the same launches through vbq_gemv_batched. With recipe=True the same
    weights are also packed with the structured recipe's widths
    (`recipe_plans`)."""

    def __init__(self, layers: int, B: int, recipe: bool = False):
        import torch

        import packed_decode_gemv_amd as vbq
        import synth
        self.vbq = vbq
        self.layers, self.B = layers, B
        self.plans, self.batched_plans, self.launch_bytes, self.launch_names = [], [], [], []
        self.recipe_plans, self.recipe_bytes, self.recipe_mats = [], [], {}
        self.mats = {}
        t0 = time.time()
        dev = torch.device("cuda")
        wl = synth.C3
        for layer in range(layers + 1):
            projs = [wl.head] if layer == layers else wl.projs
            lid = -1 if layer == layers else layer
            pms, xs, ys, rpms, rys = [], [], [], [], []
            nbytes, rbytes = 0.0, 0.0
            for pi, proj in enumerate(projs):
                key = synth.proj_key(3, lid, pi)
                W = torch.from_numpy(synth.weights(synth.SEED, key, proj.n, proj.k)).to(dev)
                pm = vbq.vbq_pack(W, synth.widths(synth.SEED, key, proj.n, proj.k // 64, proj.mix), check=False)
                x = torch.from_numpy(synth.x_f16(synth.SEED, key, B, proj.k).view(np.float16)).to(dev)
                y = torch.empty(B, proj.n, dtype=torch.float32, device=dev)
                pms.append(pm)
                xs.append(x)
                ys.append(y)
                nbytes += algorithmic_bytes(pm.sizes, proj.n, proj.k, B)
                self.mats[(lid, pi)] = (pm, x, y)
                if recipe:
                    rpm = vbq.vbq_pack(W, synth.recipe_widths(lid, pi, proj, layers), check=False)
                    ry = torch.empty(B, proj.n, dtype=torch.float32, device=dev)
                    rpms.append(rpm)
                    rys.append(ry)
                    rbytes += algorithmic_bytes(rpm.sizes, proj.n, proj.k, B)
                    self.recipe_mats[(lid, pi)] = (rpm, x, ry)
                del W
            self.plans.append(vbq.GemvPlan(pms, xs, ys, static=True))
            self.batched_plans.append(vbq.GemvPlan(pms, xs, ys))
            self.launch_bytes.append(nbytes)
            self.launch_names.append("lm_head" if lid < 0 else f"layer{layer}")
            if recipe:
                self.recipe_plans.append(vbq.GemvPlan(rpms, xs, rys, static=True))
                self.recipe_bytes.append(rbytes)
            if layer % 8 == 7:
                log(f"  packed {layer + 1}/{layers} layers ({time.time() - t0:.0f} s)")
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0
        self.weight_bytes = sum(pm.nbytes for (pm, _, _) in self.mats.values())
        self.weights = sum(pm.N * pm.K for (pm, _, _) in self.mats.values())
        self.code_bits = sum(pm.sizes.code_bits for (pm, _, _) in self.mats.values())

    def check_packed(self):
        import ctypes as C
        for (pm, _, _) in list(self.mats.values()) + list(self.recipe_mats.values()):
            st = self.vbq.lib.vbq_matrix_check(C.byref(pm.desc), self.vbq._stream())
            if st != 0:
                raise RuntimeError(f"packed layout check failed: status {st}")

    def step(self, stream_handle, plans=None):
        for p in (self.plans if plans is None else plans):
            p.launch(stream_handle)


def time_steps(stack, steps, warmup):
    """Warm up, then time exactly `steps` steps with HIP events recorded on the
    stream the kernels are launched on (torch's current stream, which is the
    stream every launch below is given). Returns ms per step."""
    import torch
    sh = stack.vbq._stream()
    for _ in range(warmup):
        stack.step(sh)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        stack.step(sh)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def capture(fn, n):
    """A HIP graph of n calls fn(0) .. fn(n-1), captured on a stream of our
    own (fn takes the current stream itself). The library allocates nothing,
    so no call has to run on that stream before the capture."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(n):
            fn(i)
    return g


def time_graph(g, reps, warmup=2):
    """us per replay of graph g, HIP events around exactly `reps` replays."""
    import torch
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def time_steps_graph(stack, steps, warmup, plans=None, mats=None):
    """One step (all launches of `plans`, default the headline's) captured as
    a HIP graph, warmed up, then exactly `steps` replays timed with HIP
    events. Returns (ms per step, graph). The replayed outputs (of `mats`)
    are checked bit for bit against an eager step."""
    import torch
    vbq = stack.vbq
    mats = list((stack.mats if mats is None else mats).values())
    stack.step(vbq._stream(), plans)   # an eager step, the reference for the replays
    torch.cuda.synchronize()
    watch = mats[:8] + mats[-1:]
    eager = [y.clone() for (_, _, y) in watch]
    g = capture(lambda i: stack.step(vbq._stream(), plans), 1)
    us = time_graph(g, steps, warmup)
    for (_, _, y), ref in zip(watch, eager):
        if not torch.equal(y, ref):
            raise RuntimeError("graph replay differs from the eager step")
    return us / 1e3, g


def time_launches(stack, reps):
    """Per-launch durations (us) from an event pair around every launch, after
    the timed region: splits a step into its layer and LM-head launches."""
    import torch
    sh = stack.vbq._stream()
    n = len(stack.plans)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
           for _ in range(reps)]
    torch.cuda.synchronize()
    for r in range(reps):
        for i, p in enumerate(stack.plans):
            evs[r][i][0].record()
            p.launch(sh)
            evs[r][i][1].record()
    torch.cuda.synchronize()
    d = np.array([[a.elapsed_time(b) * 1e3 for (a, b) in row] for row in evs])
    return d.mean(axis=0)


COPY_CAL_BYTES = 1 << 30      # bytes read (and written) by one calibration copy
COPY_CAL_REPS = 4


def copy_calibration():
    """A plain device-to-device copy of COPY_CAL_BYTES, COPY_CAL_REPS times:
    the reference whose counter readings convert FETCH_SIZE / WRITE_SIZE into
    HBM bytes. torch.neg keeps the kernel distinct from the runtime's own
    copy kernels (it reads and writes each fp32 element once)."""
    import torch
    n = COPY_CAL_BYTES // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(COPY_CAL_REPS):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    log(f"copy calibration: {COPY_CAL_REPS} x torch.neg over {COPY_CAL_BYTES} B")


def stream_ceilings():
    """Practical HBM ceilings measured in the same run, next to the 8 TB/s
    specification: a read-only pass (row sums of 2 GiB of fp32 in rows of 1024:
    reads each byte once, writes 1/1024 as much; the fastest read-only torch
    kernel found) and a copy (torch.neg over 1 GiB: reads and writes each byte
    once), each the best of a few timed repetitions."""
    import torch
    a = torch.ones((2 << 30) // 4, dtype=torch.float32, device="cuda")
    c = a[: (1 << 30) // 4]
    d = torch.empty_like(c)
    out = {}
    for name, fn, nbytes in (("read_gbs", lambda: a.view(-1, 1024).sum(1), 2 << 30),
                             ("copy_gbs", lambda: torch.neg(c, out=d), 2 << 30)):
        fn()
        best = None
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            t = e0.elapsed_time(e1) * 1e-3
            best = t if best is None else min(best, t)
        out[name] = round(nbytes / best / 1e9, 1)
    del a, c, d
    out["kernels"] = "row sums of 2 GiB fp32, rows of 1024 (read); torch.neg over 1 GiB fp32 (read + write)"
    return out


# ---------------------------------------------------------------------------
# rocprofv3 result summaries (CPU only; read the SQLite result files)

def _db_files(path):
    import glob
    if os.path.isfile(path):
        return [path]
    return sorted(glob.glob(os.path.join(path, "**", "*_results.db"), recursive=True))


def _short(name):
    name = name.replace("(anonymous namespace)::", "").split("(")[0]
    return name.replace("void ", "")


def _kernel_rows(path):
    import sqlite3
    out = []
    for f in _db_files(path):
        c = sqlite3.connect(f)
        out += c.execute("select name, duration, grid_x / workgroup_x, workgroup_x, lds_size, vgpr_count, "
                         "sgpr_count from kernels").fetchall()
    return out


def _pmc_rows(path, counter):
    import sqlite3
    out = []
    for f in _db_files(path):
        c = sqlite3.connect(f)
        out += c.execute("select dispatch_id, kernel_name, sum(value) from counters_collection "
                         "where counter_name = ? group by dispatch_id, kernel_name", (counter,)).fetchall()
    return out


def _pmc_max_rows(path, counter):
    """Per dispatch, the largest value of `counter` over its instances (a
    counter kept once per XCD, such as GRBM_GUI_ACTIVE, is the time the
    busiest XCD was active, not the sum over XCDs)."""
    import sqlite3
    out = []
    for f in _db_files(path):
        c = sqlite3.connect(f)
        out += c.execute("select K.dispatch_id, max(E.value), K.end - K.start from rocpd_pmc_event E "
                         "join rocpd_info_pmc I on I.id = E.pmc_id and I.guid = E.guid "
                         "join rocpd_kernel_dispatch K on K.event_id = E.event_id and K.guid = E.guid "
                         "where I.name = ? group by E.guid, K.dispatch_id", (counter,)).fetchall()
    return out


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES",
                 "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE")
SIMDS = 256 * 4                # MI355X: 256 compute units of 4 SIMDs


def summarize_mfma(path, command, flops_per_call):
    """Markdown summary of one --pmc pass over the GEMM: MFMA utilisation
    (busy cycles of the matrix units over 1024 SIMDs x the active cycles of
    the busiest XCD), counted bf16 flops against 2 M N K, co-issue of vector
    work beside the MFMAs, and the clock those cycles imply."""
    per = {}
    for counter in MFMA_COUNTERS:
        if counter == "GRBM_GUI_ACTIVE":
            rows = [(d, v, dur) for (d, v, dur) in _pmc_max_rows(path, counter)]
        else:
            rows = [(d, v, None) for (d, k, v) in _pmc_rows(path, counter) if "k_gemm" in k]
        per[counter] = {d: (v, dur) for (d, v, dur) in rows}
    ids = sorted(per["SQ_VALU_MFMA_BUSY_CYCLES"])
    if not ids:
        raise SystemExit("no k_gemm dispatches with MFMA counters")

    def mean(counter):
        return float(np.mean([per[counter][d][0] for d in ids]))
    gui = mean("GRBM_GUI_ACTIVE")
    dur_ns = float(np.mean([per["GRBM_GUI_ACTIVE"][d][1] for d in ids]))
    busy = mean("SQ_VALU_MFMA_BUSY_CYCLES")
    mops = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16")
    rows = [
        ("k_gemm dispatches", f"{len(ids)}"),
        ("dispatch duration (kernel trace, under counters)", f"{dur_ns / 1e3:.2f} us"),
        ("GRBM_GUI_ACTIVE, busiest XCD", f"{gui:.0f} cycles ({gui / dur_ns:.2f} GHz over the duration)"),
        ("SQ_VALU_MFMA_BUSY_CYCLES, sum over SIMDs", f"{busy:.0f}"),
        ("**MFMA utilisation** = busy / (1024 SIMDs x GUI_ACTIVE)", f"**{100 * busy / (SIMDS * gui):.1f} %**"),
        ("SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512", f"{mops * 512:.4g} flop (2 M N K = {flops_per_call:.4g})"),
        ("SQ_INSTS_MFMA", f"{mean('SQ_INSTS_MFMA'):.0f}"),
        ("SQ_INSTS_VALU (includes the MFMAs)", f"{mean('SQ_INSTS_VALU'):.0f}"),
        ("SQ_VALU_MFMA_COEXEC_CYCLES / busy", f"{100 * mean('SQ_VALU_MFMA_COEXEC_CYCLES') / busy:.1f} %"),
        ("SQ_BUSY_CU_CYCLES / (256 CUs x GUI_ACTIVE): CUs holding work", f"{100 * mean('SQ_BUSY_CU_CYCLES') / (256 * gui):.1f} %"),
        ("bf16 flop/s over the duration", f"{flops_per_call / (dur_ns * 1e-9) / 1e12:.1f} TFLOP/s "
                                           f"({100 * flops_per_call / (dur_ns * 1e-9) / 1e12 / PEAK_BF16_TFLOPS:.1f} % "
                                           f"of {PEAK_BF16_TFLOPS:.0f})"),
    ]
    text = ["# rocprofv3 MFMA counters: k_gemm", "",
            "Command (from the repository root, on an MI355X):", "", "```", command, "```", "",
            "| quantity | value |", "|---|---|"]
    text += [f"| {a} | {b} |" for a, b in rows]
    return "\n".join(text) + "\n"


def summarize_trace(path, command):
    """Markdown table of dispatch counts and durations per kernel, with the
    GEMV split by launch shape (workgroups) since layers and the LM head differ."""
    import collections
    by = collections.defaultdict(list)
    for name, dur, wgs, wgsize, lds, vgpr, sgpr in _kernel_rows(path):
        k = _short(name)
        key = (k, wgs, wgsize, lds, vgpr, sgpr) if "k_gemv" in k else (k, None, wgsize, lds, vgpr, sgpr)
        by[key].append(dur / 1e3)
    lines = ["# rocprofv3 kernel trace", "", "Command (from the repository root, on an MI355X):", "",
             "```", command, "```", "",
             "| kernel | workgroups | threads/WG | LDS B | VGPR | SGPR | calls | avg us | min us | max us | total us |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for key, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        k, wgs, wgsize, lds, vgpr, sgpr = key
        a = np.array(v)
        lines.append(f"| `{k}` | {wgs if wgs is not None else 'various'} | {wgsize} | {lds} | {vgpr} | {sgpr} | "
                     f"{len(a)} | {a.mean():.2f} | {a.min():.2f} | {a.max():.2f} | {a.sum():.1f} |")
    gem = [d / 1e3 for (n, d, *_) in _kernel_rows(path) if "k_gemv" in n]
    if gem:
        lines += ["", f"All `k_gemv` dispatches: {len(gem)} calls, average {np.mean(gem):.2f} us."]
    return "\n".join(lines) + "\n"


def summarize_counters(path, kernel, command):
    """Markdown table of every counter in one --pmc pass, averaged over the
    dispatches of `kernel` (summed over a counter's instances; GRBM_GUI_ACTIVE
    taken from the busiest XCD), split by launch shape (workgroups)."""
    import collections
    import sqlite3
    shape = {}
    for f in _db_files(path):
        c = sqlite3.connect(f)
        for did, grid, wg in c.execute("select dispatch_id, grid_size, workgroup_size from counters_collection "
                                       "where kernel_name like ? group by dispatch_id", (f"%{kernel}%",)):
            shape[did] = grid // max(wg, 1)
        names = [r[0] for r in c.execute("select distinct counter_name from counters_collection")]
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for n in names:
        if n == "GRBM_GUI_ACTIVE":
            rows = [(d, v) for (d, v, _) in _pmc_max_rows(path, n) if d in shape]
        else:
            rows = [(d, v) for (d, k, v) in _pmc_rows(path, n) if kernel in k]
        for d, v in rows:
            vals[shape[d]][n].append(v)
    lines = [f"# rocprofv3 counters: {kernel}", "", "Command (from the repository root, on an MI355X):", "",
             "```", command, "```", ""]
    for wgs in sorted(vals):
        lines += [f"Launches of {wgs} workgroups ({len(next(iter(vals[wgs].values())))} dispatches), "
                  "average per dispatch:", "", "| counter | value |", "|---|---|"]
        lines += [f"| {n} | {np.mean(v):.4g} |" for n, v in sorted(vals[wgs].items())]
        lines.append("")
    return "\n".join(lines)


def summarize_pmc(fetch_path, write_path):
    """HBM bytes per k_gemv dispatch from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by the reading of the calibration copy, which moves
    exactly COPY_CAL_BYTES in each direction."""
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_path), ("WRITE_SIZE", write_path)):
        rows = _pmc_rows(path, counter)
        cal = [v for (_, k, v) in rows if "neg" in k]
        gem = [v for (_, k, v) in rows if "k_gemv" in k]
        if not cal or not gem:
            raise SystemExit(f"{counter}: no calibration copy ({len(cal)}) or k_gemv ({len(gem)}) dispatches")
        factor = COPY_CAL_BYTES / (float(np.mean(cal)) * 1024.0)
        res[counter] = dict(kib_per_gemv_dispatch=float(np.mean(gem)), gemv_dispatches=len(gem),
                            kib_per_copy_dispatch=float(np.mean(cal)), copy_dispatches=len(cal),
                            copy_factor=factor,
                            bytes_per_gemv_dispatch=float(np.mean(gem)) * 1024.0 * factor)
    return res


def kernel_source_sha() -> str:
    """Hash of the GEMV kernel sources; counter readings are valid only for it."""
    import hashlib
    h = hashlib.sha256()
    for f in ("gemv.hip", "vbq_common.h"):
        h.update(open(os.path.join(ROOT, "packed_decode_gemv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic_gemv_9b_stack_b1.json")


def read_traffic(layers, batch):
    """HBM bytes per GEMV launch from the committed counter summary, or None
    when it is missing, for another workload, or for other kernel sources."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    try:
        t = json.load(open(TRAFFIC_JSON))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    if t.get("layers") != layers or t.get("batch") != batch:
        return None
    return t.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# The other workloads: one line each in the JSON's "workloads" list

POOL_BYTES = 600 << 20     # rotate over more than the 256 MB last-level cache


def _events_time(fn, calls, warmup=3, reps=3):
    """Average us per call of fn(i): after an eager warm-up, `calls` calls are
    captured into one HIP graph and replayed `reps` times between HIP events
    (so the time is the device's, not the host launch path's). fn takes the
    current stream itself."""
    for i in range(warmup):
        fn(i)
    g = capture(fn, calls)
    return time_graph(g, reps) / calls


def _pool(pm, extra_bytes=0):
    n = max(1, POOL_BYTES // max(1, pm.nbytes + extra_bytes))
    return [pm] + [pm.clone() for _ in range(n - 1)]


def _gemv_line(name, us, nbytes, extra=None):
    d = dict(workload=name, us_per_call=round(us, 3), gb_per_s=round(nbytes / (us * 1e-6) / 1e9, 1),
             roofline_frac=round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), bound="hbm",
             algorithmic_bytes=nbytes)
    d.update(extra or {})
    return d


def measure_workloads(stack, calls, outputs=None):
    """Timed lines for the other workloads (weights and inputs resident in HBM,
    rotated over a pool larger than the caches where they would fit):
    131M-class projection, 1.0B-class layer at batch 1 and 4, the 9B-class
    stack at batch 4, the in-cell update
    (residual GEMV, re-quantisation check, drift bound), the GEMV over recurrent
    residual levels and the batched GEMM on
    MFMA. The GPU outputs of the timed calls go to ``outputs`` (host copies
    with what regenerates their inputs) for the same-run parity check."""
    import torch

    import synth
    vbq = stack.vbq
    dev = torch.device("cuda")
    out = []

    def packed(cid, layer, pi, proj):
        key = synth.proj_key(cid, layer, pi)
        widths = synth.widths(synth.SEED, key, proj.n, proj.k // 64, proj.mix)
        W = torch.from_numpy(synth.weights(synth.SEED, key, proj.n, proj.k)).to(dev)
        pm = vbq.vbq_pack(W, widths)
        return pm, W, key

    def xf16(key, B, K):
        return torch.from_numpy(synth.x_f16(synth.SEED, key, B, K).view(np.float16)).to(dev)

    # 131M-class projection 768 x 768, batch 1
    proj = synth.C0.projs[0]
    pm, _, key = packed(0, 0, 0, proj)
    x = xf16(key, 1, proj.k)
    y = torch.empty(1, proj.n, dtype=torch.float32, device=dev)
    pool = _pool(pm)
    us = _events_time(lambda i: vbq.vbq_gemv(pool[i % len(pool)], x, out=y), calls)
    out.append(_gemv_line(f"131M-class projection {proj.n}x{proj.k}, batch 1", us,
                          algorithmic_bytes(pm.sizes, proj.n, proj.k, 1)))
    keep = outputs.append if outputs is not None else (lambda _: None)
    keep(dict(name="131M-class projection", kind="gemv", cid=0, layer=0, pi=0, proj=proj, B=1,
              y=y.cpu().numpy()))

    # 1.0B-class layer (5 projections in one launch), batch 1 and 4
    mats = [packed(1, 0, pi, p) for pi, p in enumerate(synth.C1.projs)]
    layer_bytes = sum(m.nbytes for m, _, _ in mats)
    n_copies = max(1, POOL_BYTES // layer_bytes)
    layers = [[m for m, _, _ in mats]] + [[m.clone() for m, _, _ in mats] for _ in range(n_copies - 1)]
    for B in (1, 4):
        xs = [xf16(k, B, p.k) for (_, _, k), p in zip(mats, synth.C1.projs)]
        ys = [torch.empty(B, p.n, dtype=torch.float32, device=dev) for p in synth.C1.projs]
        plans = [vbq.GemvPlan(L, xs, ys, static=True) for L in layers]
        us = _events_time(lambda i: plans[i % len(plans)].launch(vbq._stream()), calls)
        for pi, p in enumerate(synth.C1.projs):
            keep(dict(name=f"1.0B-class layer {p.name}, batch {B}", kind="gemv", cid=1, layer=0, pi=pi, proj=p,
                      B=B, y=ys[pi].cpu().numpy()))
        nb = sum(algorithmic_bytes(m.sizes, p.n, p.k, B) for (m, _, _), p in zip(mats, synth.C1.projs))
        out.append(_gemv_line(f"1.0B-class layer (qkv 6144x2048, o 2048x2048, up/gate 8192x2048, "
                              f"down 2048x8192), one vbq_gemv_batched_static launch, batch {B}", us, nb))
    del mats, layers, plans

    # The whole 9B-class step in as few launches as the ABI allows (32 matrices
    # each): the 225 matrices in 8 vbq_gemv_batched_static calls, so later
    # workgroups start while earlier ones stream (no layer order kept)
    mats = list(stack.mats.values())
    wplans = [vbq.GemvPlan([m[0] for m in mats[i:i + 32]], [m[1] for m in mats[i:i + 32]],
                           [m[2] for m in mats[i:i + 32]], static=True) for i in range(0, len(mats), 32)]

    def whole_step(i):
        sh = vbq._stream()
        for p in wplans:
            p.launch(sh)
    us = _events_time(whole_step, 1, reps=max(3, calls // 20))
    out.append(_gemv_line(f"9B-class stack ({stack.layers} layers + LM head), batch 1, all {len(mats)} matrices "
                          f"in {len(wplans)} batched launches (no layer order), one step", us,
                          float(sum(stack.launch_bytes))))
    del wplans

    # 9B-class stack at batch 4: the same packed weights, batch-4 activations
    B = 4
    plans, nb = [], 0.0
    for layer in range(stack.layers):
        pms, xs, ys = [], [], []
        for pi, p in enumerate(synth.C3.projs):
            pmx = stack.mats[(layer, pi)][0]
            pms.append(pmx)
            xs.append(xf16(synth.proj_key(3, layer, pi), B, p.k))
            ys.append(torch.empty(B, p.n, dtype=torch.float32, device=dev))
            nb += algorithmic_bytes(pmx.sizes, p.n, p.k, B)
        plans.append(vbq.GemvPlan(pms, xs, ys, static=True))
    pmh = stack.mats[(-1, 0)][0]
    hx = xf16(synth.proj_key(3, -1, 0), B, synth.C3.head.k)
    plans.append(vbq.GemvPlan([pmh], [hx], [torch.empty(B, synth.C3.head.n, dtype=torch.float32, device=dev)]))
    nb += algorithmic_bytes(pmh.sizes, synth.C3.head.n, synth.C3.head.k, B)

    def stack_step(i):
        sh = vbq._stream()
        for p in plans:
            p.launch(sh)
    us = _events_time(stack_step, 1, reps=max(3, calls // 20))
    out.append(_gemv_line(f"9B-class stack ({stack.layers} layers + LM head), batch 4, one step", us, nb,
                          {"us_per_layer": round((us) / (stack.layers + 1), 3)}))
    del plans

    # In-cell update on a 4-bit release 14336 x 4096. The update is drawn as
    # compact fraction bytes f (uniform in [-127, 127]); the fp16 residual
    # r = fp16(s f / 256) is decoded on the device from the packed scales, so
    # both residual forms stand for the same in-cell update.
    proj = synth.C2.projs[0]
    pm, W, key = packed(2, 0, 0, proj)
    del W
    N, K = proj.n, proj.k
    f8 = torch.from_numpy(synth.cell_f(synth.SEED, key, N, K)).to(dev)
    resid = vbq.cell8_decode(pm, f8)
    x = xf16(key, 1, K)
    y = torch.empty(1, N, dtype=torch.float32, device=dev)
    rbytes = resid.numel() * 2
    n_copies = max(1, POOL_BYTES // (pm.nbytes + rbytes + f8.numel()))
    pool = [(pm, resid, f8)] + [(pm.clone(), resid.clone(), f8.clone()) for _ in range(n_copies - 1)]
    us = _events_time(lambda i: vbq.vbq_gemv(pool[i % len(pool)][0], x, residual=pool[i % len(pool)][1], out=y),
                      calls)
    nb = algorithmic_bytes(pm.sizes, N, K, 1, resid=True)
    out.append(_gemv_line(f"in-cell update {N}x{K} (all 4-bit) + fp16 residual, residual GEMV, batch 1", us, nb))
    keep(dict(name="in-cell fp16 residual GEMV", kind="resid16", cid=2, layer=0, pi=0, proj=proj, B=1,
              y=y.cpu().numpy()))
    # the same update as one signed byte per weight (vbq_gemv_cell8)
    us = _events_time(lambda i: vbq.vbq_gemv_cell8(pool[i % len(pool)][0], x, pool[i % len(pool)][2], out=y),
                      calls)
    nb8 = algorithmic_bytes(pm.sizes, N, K, 1) + N * K
    out.append(_gemv_line(f"in-cell update {N}x{K} (all 4-bit) + compact residual (int8 cell fraction), "
                          "residual GEMV, batch 1", us, nb8))
    keep(dict(name="in-cell compact residual GEMV", kind="cell8", cid=2, layer=0, pi=0, proj=proj, B=1,
              y=y.cpu().numpy()))
    # encoding an fp16 residual into fraction bytes: reads r (2 B/weight), the
    # scale of every group and the width map, writes f (1 B/weight)
    f_out = torch.empty_like(f8)
    us = _events_time(lambda i: vbq.cell8_encode(pool[i % len(pool)][0], pool[i % len(pool)][1], out=f_out), calls)
    groups = N * (K // 64)
    nbe = 3.0 * N * K + 4 * groups + groups / 4
    out.append(_gemv_line(f"in-cell update {N}x{K}: encoding the fp16 residual to fraction bytes (cell8_encode)",
                          us, nbe, {"matches_drawn_bytes": bool(torch.equal(f_out, pool[(calls - 1) % len(pool)][2]))}))
    res = torch.empty(3, dtype=torch.int64, device=dev)
    import ctypes as C

    def verify(i):
        pmv, rv, _ = pool[i % len(pool)]
        st = vbq.lib.cell_requant_verify(C.byref(pmv.desc), C.c_void_p(rv.data_ptr()), C.c_void_p(res.data_ptr()),
                                         None, vbq._stream())
        if st != 0:
            raise RuntimeError(f"cell_requant_verify status {st}")
    us = _events_time(verify, calls)
    counts = res.cpu().numpy().view(np.uint64)
    nbv = algorithmic_bytes(pm.sizes, N, K, 1, resid=True) - 2 * K - 4 * N + 24
    out.append(_gemv_line(f"in-cell update {N}x{K}: re-quantisation check (cell_requant_verify)", us, nbv,
                          {"mismatches": int(counts[0]), "out_of_cell": int(counts[1])}))
    # Drift bound of the update: scale/offset (4 B) and the 2-bit width of
    # every group, x, one float per row; the codes are not read.
    bound = torch.empty(1, N, dtype=torch.float32, device=dev)
    us = _events_time(lambda i: vbq.cell_drift_bound(pool[i % len(pool)][0], x, out=bound), calls)
    nbd = N * (K // 64) * (4 + 0.25) + 2 * K + 4 * N
    out.append(_gemv_line(f"in-cell update {N}x{K}: drift bound (cell_drift_bound), batch 1", us, nbd))
    del pool

    # Recurrent residual levels of the same shape: a 2-bit base and three
    # 2-bit residual levels (8 effective bits), GEMV over all four at batch 1.
    Wr = torch.from_numpy(synth.weights(synth.SEED, key, N, K)).to(dev)
    levels = vbq.rrq_pack(Wr, 4)
    del Wr
    lv_bytes = sum(pm_.nbytes for pm_ in levels)
    pool = [levels] + [[pm_.clone() for pm_ in levels] for _ in range(max(1, POOL_BYTES // lv_bytes) - 1)]
    us = _events_time(lambda i: vbq.vbq_gemv_levels(pool[i % len(pool)], x, out=y), calls)
    groups = N * (K // 64)
    nbr = sum(pm_.sizes.code_bits / 8 + 4 * groups + groups / 4 for pm_ in levels) + 2 * K + 4 * N
    out.append(_gemv_line(f"recurrent residual levels {N}x{K}: 2-bit base + 3 levels (8 effective bits), "
                          "GEMV over the levels, batch 1", us, nbr))
    keep(dict(name="recurrent residual levels", kind="levels", cid=2, layer=0, pi=0, proj=proj, B=1,
              y=y.cpu().numpy()))
    del pool, levels

    out.append(gemm_workload(vbq, calls, outputs))
    return out


def recipe_line(stack, steps, warmup):
    """The 9B-class stack with the structured recipe's widths (same weights
    and activations): one step replayed as a HIP graph, plus the spread of
    its per-launch times (event pairs around each launch)."""
    import torch
    ms, _ = time_steps_graph(stack, steps, warmup, plans=stack.recipe_plans, mats=stack.recipe_mats)
    nb = float(sum(stack.recipe_bytes))
    sh = stack.vbq._stream()
    reps = 5
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in stack.recipe_plans] for _ in range(reps)]
    torch.cuda.synchronize()
    for r in range(reps):
        for i, p in enumerate(stack.recipe_plans):
            evs[r][i][0].record()
            p.launch(sh)
            evs[r][i][1].record()
    torch.cuda.synchronize()
    d = np.array([[a.elapsed_time(b) * 1e3 for (a, b) in row] for row in evs]).mean(axis=0)
    per_layer = [nbl / (t * 1e-6) / 1e9 for nbl, t in zip(stack.recipe_bytes[:-1], d[:-1])]
    mats = stack.recipe_mats.values()
    weights = sum(pm.N * pm.K for (pm, _, _) in mats)
    code_bits = sum(pm.sizes.code_bits for (pm, _, _) in mats)
    return _gemv_line(
        f"9B-class stack ({stack.layers} layers + LM head), structured recipe: first MLP block 2.5 bits, "
        f"SLQ-style per-layer mixes (ends widest), LM head 1.1 bits, wide groups on hot rows and input "
        f"channels; batch {stack.B}, one step", ms * 1e3, nb,
        {"mean_code_bits": round(code_bits / weights, 4),
         "layer0_us": round(float(d[0]), 3), "layer15_us": round(float(d[15]), 3) if len(d) > 16 else None,
         "lm_head_us": round(float(d[-1]), 3),
         "layer_gb_per_s_min": round(min(per_layer), 1), "layer_gb_per_s_max": round(max(per_layer), 1)})


def gemm_workload(vbq, calls, outputs=None):
    """The batched GEMM on MFMA: M = 256 tokens, K = 4096, N = 14336, default
    width mix; one timed line."""
    import torch

    import synth
    dev = torch.device("cuda")
    proj = synth.C4.projs[0]
    M = synth.C4.gemm_m
    key = synth.proj_key(4, 0, 0)
    widths = synth.widths(synth.SEED, key, proj.n, proj.k // 64, proj.mix)
    pm = vbq.vbq_pack(torch.from_numpy(synth.weights(synth.SEED, key, proj.n, proj.k)).to(dev), widths)
    xb = torch.from_numpy(synth.x_bf16(synth.SEED, key, M, proj.k).view(np.int16)).to(dev).view(torch.bfloat16)
    yg = torch.empty(M, proj.n, dtype=torch.float32, device=dev)
    us = _events_time(lambda i: vbq.vbq_gemm(pm, xb, out=yg), calls)
    if outputs is not None:
        outputs.append(dict(name=f"batched GEMM M={M}", kind="gemm", cid=4, layer=0, pi=0, proj=proj, B=M,
                            y=yg.cpu().numpy()))
    flops = 2.0 * M * proj.n * proj.k
    tf = flops / (us * 1e-6) / 1e12
    return dict(workload=f"batched GEMM M={M} K={proj.k} N={proj.n} (bf16 MFMA)", us_per_call=round(us, 3),
                tflop_per_s=round(tf, 1), roofline_frac=round(tf / PEAK_BF16_TFLOPS, 4), bound="mfma",
                peak_tflop_per_s=PEAK_BF16_TFLOPS, flops=flops, M=M, K=proj.k, N=proj.n)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(stack, budget_s):
    """The CPU oracle (as it stands) on a bounded sample of the same workload:
    whole projections of the first layers, then LM head rows, until about
    budget_s seconds of wall time. The oracle packs the same synthetic W
    itself (untimed); the timed part is its GEMV from the packed layout
    (unpack, fp64 dequantise, fp64 dot), run on every core this process may
    use: the rows of a matrix are cut into slices and each worker thread
    calls the oracle on its slice (the oracle runs in C and releases the
    interpreter lock). Its outputs double as a sampled parity check of the GPU
    results."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import synth
    wl = synth.C3
    B = stack.B
    cores = sorted(os.sched_getaffinity(0))
    n_threads = len(cores)
    spent, done_bytes, done_w = 0.0, 0.0, 0
    worst, checked = 0.0, []
    order = [(layer, pi, proj) for layer in range(stack.layers) for pi, proj in enumerate(wl.projs)]
    order.insert(7, (-1, 0, wl.head))
    first = None
    with ThreadPoolExecutor(n_threads) as ex:
        for (layer, pi, proj) in order:
            if spent >= budget_s:
                break
            key = synth.proj_key(3, layer, pi)
            rows = proj.n
            if layer == -1:
                rows = min(proj.n, 16384 * max(1, n_threads // 8))
            G = proj.k // 64
            widths = synth.widths(synth.SEED, key, proj.n, G, proj.mix, rows=np.arange(rows))
            W = synth.weights(synth.SEED, key, proj.n, proj.k, rows=np.arange(rows))
            x = synth.x_f16(synth.SEED, key, B, proj.k)
            lay = oracle.pack(W, widths)
            slices = np.array_split(np.arange(rows, dtype=np.int64), 4 * n_threads)

            def run(sl, lay=lay, x=x):
                q, s_, o, _ = oracle.unpack(lay, rows=sl)
                return oracle.gemv(q, s_, o, x)

            t0 = time.perf_counter()
            parts = list(ex.map(run, slices))
            dt = time.perf_counter() - t0
            y = np.concatenate(parts, axis=1)
            spent += dt
            sizes = stack.vbq.pack_query(widths)
            if first is None:
                first = (lay, x, rows, proj.k, sizes)
            done_bytes += algorithmic_bytes(sizes, rows, proj.k, B)
            done_w += rows * proj.k
            yg = stack.mats[(layer, pi)][2].cpu().numpy()[:, :rows].astype(np.float64)
            rel = float(np.linalg.norm(yg - y) / np.linalg.norm(y))
            worst = max(worst, rel)
            checked.append(f"{'lm_head' if layer < 0 else f'L{layer}.{proj.name}'}[{rows}x{proj.k}]")
    # The same oracle on one thread (the calling one), over row slices of the
    # first matrix, for about a tenth of the budget.
    one_thread = None
    if first is not None:
        lay0, x0, rows0, k0, sizes0 = first
        t0, n1 = time.perf_counter(), 0
        for sl in np.array_split(np.arange(rows0, dtype=np.int64), 64):
            q, s_, o, _ = oracle.unpack(lay0, rows=sl)
            oracle.gemv(q, s_, o, x0)
            n1 += len(sl)
            if time.perf_counter() - t0 >= budget_s / 10:
                break
        dt1 = time.perf_counter() - t0
        one_thread = dict(value=algorithmic_bytes(sizes0, rows0, k0, B) * n1 / rows0 / dt1 / 1e9, unit="GB/s",
                          rows=n1, seconds=round(dt1, 2))
    return dict(value=done_bytes / spent / 1e9, unit="GB/s", cores=n_threads, kind="oracle",
                one_thread=one_thread,
                cpu=cpu_model(), threads="one oracle call per row slice on every core of the process's affinity",
                sample=f"{len(checked)} matrices ({done_w / 1e6:.0f}M weights, batch {B}): "
                       + ", ".join(checked[:4]) + (" ..." if len(checked) > 4 else ""),
                seconds=round(spent, 2)), dict(max_rel_l2=worst, matrices=len(checked), tol=2e-3)


def workload_parity(outputs, max_rows=1024):
    """Same-run parity of the other workloads' GPU outputs against the CPU
    oracle (part of the CPU-baseline leg): for each output, the oracle
    quantises the same synthetic rows (every row up to max_rows, else an even
    sample of max_rows rows) and forms its fp64 result; the figure is the
    rel-L2 distance over those rows. Widths, weights, activations and residual
    bytes are regenerated from the seeded draws, row by row."""
    import oracle
    import synth
    res = {}
    for o in outputs:
        p = o["proj"]
        key = synth.proj_key(o["cid"], o["layer"], o["pi"])
        rows = np.arange(p.n) if p.n <= max_rows else np.unique(np.linspace(0, p.n - 1, max_rows).astype(np.int64))
        widths = synth.widths(synth.SEED, key, p.n, p.k // 64, p.mix, rows=rows)
        W = synth.weights(synth.SEED, key, p.n, p.k, rows=rows)
        if o["kind"] == "levels":
            levels, _ = oracle.rrq_levels(W, 4)
            ref = oracle.rrq_gemv(levels, synth.x_f16(synth.SEED, key, 1, p.k))
        else:
            q, s16, o16 = oracle.quantize_matrix(W, widths)
            if o["kind"] == "gemm":
                ref = oracle.gemm_bf16_weights(q, s16, o16, synth.x_bf16(synth.SEED, key, o["B"], p.k))
            else:
                x = synth.x_f16(synth.SEED, key, o["B"], p.k)
                if o["kind"] == "gemv":
                    ref = oracle.gemv(q, s16, o16, x)
                else:
                    f = synth.cell_f(synth.SEED, key, p.n, p.k, rows=rows)
                    ref = (oracle.gemv(q, s16, o16, x, resid=oracle.cell8_decode(f, s16)) if o["kind"] == "resid16"
                           else oracle.gemv_cell8(q, s16, o16, x, f))
        y = o["y"][:, rows].astype(np.float64)
        res[o["name"]] = dict(rel_l2=float(np.linalg.norm(y - ref) / np.linalg.norm(ref)), rows=int(len(rows)))
    return dict(max_rel_l2=max((v["rel_l2"] for v in res.values()), default=0.0), tol=2e-3, outputs=res)


def workload_name(layers, B):
    return (f"9B-class stack: {layers} layers x (q 4096x4096, k 1024x4096, v 1024x4096, o 4096x4096, "
            f"gate 14336x4096, up 14336x4096, down 4096x14336) + LM head 128256x4096, "
            f"64-weight groups of 1/2/4/8 bits, batch {B}")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--launch-reps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="only the headline stack")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the step through vbq_gemv_batched (profiles of the headline launches only)")
    ap.add_argument("--workload-calls", type=int, default=100)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-trace", metavar="RESULTS")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_RESULTS", "WRITE_RESULTS"))
    ap.add_argument("--summarize-mfma", metavar="RESULTS", help="MFMA counters of a --gemm-only run")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("RESULTS", "KERNEL"),
                    help="every counter of a --pmc pass, averaged over one kernel's dispatches")
    ap.add_argument("--gemm-only", action="store_true", help="time only the batched GEMM and print its line")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    ap.add_argument("--out", help="summary file to write")
    args = ap.parse_args(argv)

    if args.summarize_trace:
        text = summarize_trace(args.summarize_trace, args.command)
        open(args.out, "w").write(text) if args.out else sys.stdout.write(text)
        return 0
    if args.summarize_counters:
        text = summarize_counters(*args.summarize_counters, args.command)
        open(args.out, "w").write(text) if args.out else sys.stdout.write(text)
        return 0
    if args.summarize_mfma:
        import synth
        p = synth.C4.projs[0]
        text = summarize_mfma(args.summarize_mfma, args.command, 2.0 * synth.C4.gemm_m * p.n * p.k)
        open(args.out, "w").write(text) if args.out else sys.stdout.write(text)
        return 0
    if args.summarize_pmc:
        res = summarize_pmc(*args.summarize_pmc)
        traffic = res["FETCH_SIZE"]["bytes_per_gemv_dispatch"] + res["WRITE_SIZE"]["bytes_per_gemv_dispatch"]
        doc = dict(kernel=KERNEL, workload=workload_name(args.layers, args.batch), layers=args.layers,
                   batch=args.batch, kernel_source_sha=kernel_source_sha(), bytes_per_launch=traffic,
                   counters=res, command=args.command)
        out = args.out or TRAFFIC_JSON
        json.dump(doc, open(out, "w"), indent=1)
        print(json.dumps(doc, indent=1))
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the packed GEMV here runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.gemm_only:
        import packed_decode_gemv_amd as vbq
        print(json.dumps(gemm_workload(vbq, args.workload_calls)), flush=True)
        return 0
    log(f"building the 9B-class stack: {args.layers} layers + LM head, batch {args.batch}")
    stack = Stack(args.layers, args.batch, recipe=not args.no_workloads)
    stack.check_packed()
    log(f"  setup {stack.setup_s:.1f} s, packed weights {stack.weight_bytes / 1e9:.3f} GB")

    ms_eager = time_steps(stack, args.steps, args.warmup)
    ms, _ = time_steps_graph(stack, args.steps, args.warmup)
    ms_batched = None
    if not args.no_compare:
        ms_batched, _ = time_steps_graph(stack, args.steps, args.warmup, plans=stack.batched_plans)
    log(f"  eager launches {ms_eager * 1e3:.1f} us/step, graph replay {ms * 1e3:.1f} us/step "
        f"(vbq_gemv_batched launches: {ms_batched and round(ms_batched * 1e3, 1)} us/step)")
    n_launch = len(stack.plans)
    step_bytes = float(sum(stack.launch_bytes))
    value = step_bytes / (ms * 1e-3) / 1e9
    # The dominant kernel is k_gemv: every launch of a step is one. Its average
    # launch duration is the timed region's event time over its launches.
    launch_avg_us = ms * 1e3 / n_launch
    bytes_per_launch = step_bytes / n_launch
    achieved = bytes_per_launch / (launch_avg_us * 1e-6) / 1e9
    log(f"  {ms * 1e3:.1f} us/step, {value:.0f} GB/s, {launch_avg_us:.2f} us per launch")

    d = time_launches(stack, args.launch_reps)
    head_us = float(d[-1])
    layer_us = (ms * 1e3 - head_us) / args.layers
    log(f"  event pair per launch: layer {d[:-1].mean():.2f} us, lm_head {head_us:.2f} us")

    ceilings = stream_ceilings()
    log(f"  measured ceilings: read {ceilings['read_gbs']:.0f} GB/s, copy {ceilings['copy_gbs']:.0f} GB/s")

    workloads, outputs = None, []
    if not args.no_workloads:
        log("structured recipe stack")
        workloads = [recipe_line(stack, args.steps, args.warmup)]
        log("other workloads")
        workloads += measure_workloads(stack, args.workload_calls, outputs)
        for w in workloads:
            log(f"  {w['workload']}: {w['us_per_call']:.2f} us, frac {w['roofline_frac']:.3f}")

    if args.copy_calibration:
        copy_calibration()

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on a bounded sample (~{args.cpu_seconds:.0f} s)")
        cpu, parity = cpu_baseline(stack, args.cpu_seconds)
        log(f"  oracle {cpu['value']:.4f} GB/s; sampled parity max rel-L2 {parity['max_rel_l2']:.2e}")
        if outputs:
            parity["workloads"] = workload_parity(outputs)
            log(f"  other workloads: max rel-L2 {parity['workloads']['max_rel_l2']:.2e}")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_eager_launches": round(ms_eager, 4),
        "ms_per_step_vbq_gemv_batched": None if ms_batched is None else round(ms_batched, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": workload_name(args.layers, args.batch),
            "batch": args.batch,
            "layers": args.layers,
            "launches_per_step": n_launch,
            "launch": "one vbq_gemv_batched_static launch per layer (its 7 projections; every k-tile of the "
                      "down projection a workgroup of its own) + one for the LM head; a step's launches "
                      "replayed as one HIP graph",
            "algorithmic_bytes_per_step": step_bytes,
            "packed_bytes_resident": stack.weight_bytes,
            "weights": stack.weights,
            "mean_code_bits": round(stack.code_bits / stack.weights, 4),
            "algorithmic_bits_read_per_weight": round(8 * step_bytes / stack.weights, 4),
            "stream_bits_per_weight": round(8 * stack.weight_bytes / stack.weights, 4),
        },
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "us_per_layer": round(layer_us, 3),
        "us_lm_head": round(head_us, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": read_traffic(args.layers, args.batch),
            "kernel": KERNEL,
            "avg_launch_us": round(launch_avg_us, 3),
            "algorithmic_bytes_per_launch": bytes_per_launch,
            "measured_ceilings": ceilings,
        },
        "cpu_baseline": cpu,
        "parity": parity,
        "workloads": workloads,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
