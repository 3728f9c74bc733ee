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

Prints one JSON line (see the fields below). Other workloads are available
with --workload for reporting; they are not the headline line.
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
    """Packed matrices of the 9B-class stack, their x and y buffers, and plans."""

    def __init__(self, layers: int, B: int):
        import torch

        import packed_decode_gemv_amd as vbq
        import synth
        self.vbq = vbq
        self.layers, self.B = layers, B
        self.plans, self.launch_bytes, self.launch_names = [], [], []
        self.mats = {}
        t0 = time.time()
        dev = torch.device("cuda")
        wl = synth.C3
        for layer in range(layers):
            pms, xs, ys = [], [], []
            nbytes = 0.0
            for pi, proj in enumerate(wl.projs):
                pm, x, y, nb = self._make(3, layer, pi, proj, B, dev)
                pms.append(pm)
                xs.append(x)
                ys.append(y)
                nbytes += nb
                self.mats[(layer, pi)] = (pm, x, y)
            self.plans.append(vbq.GemvPlan(pms, xs, ys))
            self.launch_bytes.append(nbytes)
            self.launch_names.append(f"layer{layer}")
            if layer % 8 == 7:
                log(f"  packed {layer + 1}/{layers} layers ({time.time() - t0:.0f} s)")
        pm, x, y, nb = self._make(3, -1, 0, wl.head, B, dev)
        self.mats[(-1, 0)] = (pm, x, y)
        self.plans.append(vbq.GemvPlan([pm], [x], [y]))
        self.launch_bytes.append(nb)
        self.launch_names.append("lm_head")
        torch.cuda.synchronize()
        self.setup_s = time.time() - t0
        self.weight_bytes = sum(pm.nbytes for (pm, _, _) in self.mats.values())

    def _make(self, cid, layer, pi, proj, B, dev):
        import torch

        import synth
        key = synth.proj_key(cid, layer, pi)
        G = proj.k // 64
        widths = synth.widths(synth.SEED, key, proj.n, G, proj.mix)
        W = torch.from_numpy(synth.weights(synth.SEED, key, proj.n, proj.k)).to(dev)
        pm = self.vbq.vbq_pack(W, widths, check=False)
        del W
        x = torch.from_numpy(synth.x_f16(synth.SEED, key, B, proj.k).view(np.float16)).to(dev)
        y = torch.empty(B, proj.n, dtype=torch.float32, device=dev)
        nb = algorithmic_bytes(pm.sizes, proj.n, proj.k, B)
        return pm, x, y, nb

    def check_packed(self):
        import ctypes as C
        for (pm, _, _) in self.mats.values():
            st = self.vbq.lib.vbq_matrix_check(C.byref(pm.desc), self.vbq._stream())
            if st != 0:
                raise RuntimeError(f"packed layout check failed: status {st}")

    def step(self, stream_handle):
        for p in self.plans:
            p.launch(stream_handle)


def time_steps(stack, steps, warmup):
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
    return e0.elapsed_time(e1) / steps   # ms per step


def time_launches(stack, reps):
    """Per-launch durations from HIP events around every launch (same stream)."""
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
    d = np.array([[a.elapsed_time(b) * 1e3 for (a, b) in row] for row in evs])   # us
    return d.mean(axis=0)


def cpu_baseline(stack, budget_s):
    """The CPU oracle (single-threaded, as it stands) on a bounded sample of the
    same workload: whole projections of the first layers, then LM head rows,
    until about budget_s seconds of oracle GEMV time. The oracle packs the
    same synthetic W itself (untimed); the timed part is its GEMV from the
    packed layout: unpack, fp64 dequantise, fp64 dot. Its outputs double as a
    sampled parity check of the GPU results."""
    import oracle
    import synth
    wl = synth.C3
    B = stack.B
    spent, done_bytes, done_w = 0.0, 0.0, 0
    worst, checked = 0.0, []
    order = [(layer, pi, proj) for layer in range(stack.layers) for pi, proj in enumerate(wl.projs)]
    order.insert(7, (-1, 0, wl.head))
    for (layer, pi, proj) in order:
        if spent >= budget_s:
            break
        key = synth.proj_key(3, layer, pi)
        rows = proj.n
        if layer == -1:
            rows = min(proj.n, 16384)
        G = proj.k // 64
        widths = synth.widths(synth.SEED, key, proj.n, G, proj.mix, rows=np.arange(rows))
        W = synth.weights(synth.SEED, key, proj.n, proj.k, rows=np.arange(rows))
        x = synth.x_f16(synth.SEED, key, B, proj.k)
        lay = oracle.pack(W, widths)
        t0 = time.perf_counter()
        q, s, o, _ = oracle.unpack(lay)
        y = oracle.gemv(q, s, o, x)
        dt = time.perf_counter() - t0
        spent += dt
        sizes = stack.vbq.pack_query(widths)
        done_bytes += algorithmic_bytes(sizes, rows, proj.k, B)
        done_w += rows * proj.k
        yg = stack.mats[(layer, pi)][2].cpu().numpy()[:, :rows].astype(np.float64)
        rel = float(np.linalg.norm(yg - y) / np.linalg.norm(y))
        worst = max(worst, rel)
        checked.append(f"{'lm_head' if layer < 0 else f'L{layer}.{proj.name}'}[{rows}x{proj.k}]")
    return dict(value=done_bytes / spent / 1e9, unit="GB/s", cores=1, kind="oracle",
                sample=f"{len(checked)} matrices ({done_w / 1e6:.0f}M weights, batch {B}): "
                       + ", ".join(checked[:4]) + (" ..." if len(checked) > 4 else ""),
                seconds=round(spent, 2)), dict(max_rel_l2=worst, matrices=len(checked), tol=2e-3)


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
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build runs the packed GEMV on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus}).", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    log(f"building the 9B-class stack: {args.layers} layers + LM head, batch {args.batch}")
    stack = Stack(args.layers, args.batch)
    stack.check_packed()
    log(f"  setup {stack.setup_s:.1f} s, packed weights {stack.weight_bytes / 1e9:.3f} GB")

    ms = time_steps(stack, args.steps, args.warmup)
    step_bytes = float(sum(stack.launch_bytes))
    value = step_bytes / (ms * 1e-3) / 1e9
    log(f"  {ms * 1e3:.1f} us/step, {value:.0f} GB/s")

    d = time_launches(stack, args.launch_reps)
    layer_us = d[:-1]
    head_us = float(d[-1])
    kernel_avg_us = float(d.mean())
    achieved = (step_bytes / len(d)) / (kernel_avg_us * 1e-6) / 1e9
    log(f"  per launch: layer {layer_us.mean():.2f} us, lm_head {head_us:.2f} us, avg {kernel_avg_us:.2f} us")

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic_gemv_9b_stack_b1.json")
    if os.path.exists(tpath):
        try:
            t = json.load(open(tpath))
            if t.get("kernel_source_sha") == kernel_source_sha():
                traffic = t.get("bytes_per_launch")
        except Exception:
            traffic = None

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on a bounded sample (~{args.cpu_seconds:.0f} s)")
        cpu, parity = cpu_baseline(stack, args.cpu_seconds)
        cpu["cores"] = 1
        log(f"  oracle {cpu['value']:.4f} GB/s; sampled parity max rel-L2 {parity['max_rel_l2']:.2e}")

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": f"9B-class stack: {args.layers} layers x (q,k,v,o 4096-wide; gate,up,down 14336-wide) "
                        f"+ LM head 128256x4096, mixed 1/2/4/8-bit 64-weight groups, batch {args.batch}",
            "batch": args.batch,
            "layers": args.layers,
            "launches_per_step": len(d),
            "launch": "one vbq_gemv_batched launch per layer (7 projections) + one for the LM head",
            "algorithmic_bytes_per_step": step_bytes,
            "packed_bytes_resident": stack.weight_bytes,
        },
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "us_per_layer": round(float(layer_us.mean()), 3),
        "us_lm_head": round(head_us, 3),
        "us_per_layer_wall": round((ms * 1e3 - head_us) / args.layers, 3),
        "roofline": {
            "bound": "hbm",
            "kernel": KERNEL,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(kernel_avg_us, 3),
            "algorithmic_bytes_per_launch": step_bytes / len(d),
        },
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(out), flush=True)
    return 0


def kernel_source_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("gemv.hip", "vbq_common.h"):
        h.update(open(os.path.join(ROOT, "packed_decode_gemv_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
