#!/usr/bin/env python3
"""Throughput of VGGT global attention on one MI355X, through the C ABI of libvggt_attn.so.

A step is one vggt_attn_forward of the workload: the gather/pack stage (index set S, packed K/V
tiles, per-frame mean K/V) followed by the MFMA attention kernel, on inputs already resident in
HBM.  Default workload: 800 frames x 1374 tokens (37x37 patches + 5 special), 16 heads, d = 64,
bf16 in / fp32 out, SGA sigma = 6 (2x3 windows) with frame 0 and the specials dense and the
diagonal + per-frame mean terms on.

Prints one JSON line.  value = attended queries/s (query tokens, each over all heads, per second
of step time).  roofline = the attention kernel against the bf16 dense matrix-core peak, its
duration taken from HIP events on the launch stream.  cpu_baseline = the float64 oracle timed
on a bounded sample of query rows of the same workload on this host's cores (a reported
baseline, not a target); the same rows double as a parity check of this run's output.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak (vendor figure)
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
# float32 vector FMA rate without packed (two-wide) instructions, which this library does not use:
# 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz (the published 157.3 TFLOP/s counts packed FP32)
FP32_VECTOR_PEAK_TFLOPS = 78.6

METRIC = "global-attn attended queries/s + TFLOP/s (% bf16 MFMA peak), 800 frames sigma=6"

# name -> (plan/oracle descriptor, human description)
WORKLOADS = {
    "sga6-800f": (dict(frames=800, grid_h=37, grid_w=37, heads=16, sigma=6, diag=True, mean=True),
                  "800 frames x 1374 tokens (37x37 patches + 5 special), 16 heads, d=64, bf16 in / fp32 out, "
                  "SGA sigma=6 (2x3), frame 0 + specials dense, diagonal + per-frame mean K/V (unit weight)"),
    "dense-32f": (dict(frames=32, grid_h=37, grid_w=37, heads=16, sigma=1),
                  "32 frames x 1374 tokens, 16 heads, d=64, bf16 in / fp32 out, dense global attention"),
    "sga4-100f": (dict(frames=100, grid_h=37, grid_w=37, heads=16, sigma=4, diag=True, mean=True),
                  "100 frames x 1374 tokens, 16 heads, d=64, bf16 in / fp32 out, SGA sigma=4 (2x2), diag + mean"),
    "g2f-200f": (dict(frames=200, grid_h=37, grid_w=37, heads=16, g2f=True),
                 "200 frames x 1374 tokens, 16 heads, d=64, bf16 in / fp32 out, Global-to-Frame (3200 batches of 1374x1374)"),
    "sga9-200f": (dict(frames=200, grid_h=37, grid_w=37, heads=16, sigma=9, diag=True, mean=True),
                  "200 frames x 1374 tokens, 16 heads, d=64, bf16 in / fp32 out, SGA sigma=9 (3x3), diag + mean"),
    "sga6-800f-phase": (dict(frames=800, grid_h=37, grid_w=37, heads=16, sigma=6, diag=True, mean=True, phase_shift=True),
                        "800 frames x 1374 tokens, 16 heads, d=64, bf16 in / fp32 out, SGA sigma=6 (2x3) on a "
                        "phase-shifted grid (offsets cycle over 6 frames), frame 0 + specials dense, diag + per-frame mean"),
    "sga9-200f-phase-global": (dict(frames=200, grid_h=37, grid_w=37, heads=16, sigma=9, diag=True, mean=True,
                                    mean_count=True, mean_global=True, phase_shift=True),
                               "200 frames x 1374 tokens, 16 heads, d=64, bf16 in / fp32 out, SGA sigma=9 (3x3) on a "
                               "phase-shifted grid, diag + one global mean K/V with the log-count bias"),
    "sga6-800f-sized": (dict(frames=800, grid_h=37, grid_w=37, heads=16, sigma=6, diag=True, log_size=True),
                        "800 frames x 1374 tokens, 16 heads, d=64, bf16 in / fp32 out, SGA sigma=6 (2x3) with the "
                        "diagonal term and size-aware keys (seeded group sizes 1..4, + ln g on every key's logit)"),
    "g2m-32f": (dict(frames=32, grid_h=37, grid_w=37, heads=16, g2m=True),
                "32 frames x 1374 tokens, 16 heads, d=64, bf16 in / fp32 out, Global-to-Mean (one mean K/V token)"),
}
# The f16 score form (PRESCALE_Q) of a workload: packed keys f16(k * 2^-e_h), Q * tau * log2(e) *
# 2^e_h rounded to f16 once, QK^T on the f16 matrix cores (same peak as bf16), PV on bf16.
for _n in ("sga6-800f", "dense-32f", "g2f-200f", "sga9-200f"):
    _d, _t = WORKLOADS[_n]
    WORKLOADS[_n + "-f16"] = (dict(_d, prescale_q=True), _t + "; f16 score form (Q*tau*log2e rounded to f16 once)")

# Reported beside the headline workload (same run, fewer steps).  Each group shares one set of
# tensors and its step is the sum of its plans' forwards.  "g2f+sga9-200f" is the early/middle
# layer split of the 200-frame workload: one G2F call, then enhanced SGA sigma 9, on the same
# tensors.  "sweep-200f" runs every form at one N (200 frames) so that their measured times can be
# set beside their FLOP ratios and sigma ("AVGGT" notes, 关键设计 1 and 2: G2F turns O((NL)^2)
# into O(N L^2), SGA cuts global attention by about sigma).
_D200 = dict(frames=200, grid_h=37, grid_w=37, heads=16)
SWEEP_200 = [dict(_D200, sigma=1)] + [
    dict(_D200, sigma=s, **enh) for s in (2, 4, 6, 9) for enh in ({}, dict(diag=True, mean=True))] + [
    dict(_D200, g2f=True)]
EXTRA_GROUPS = [
    ("tiny-fp32", [dict(frames=4, grid_h=8, grid_w=8, heads=2, sigma=4, diag=True, mean=True)], "fp32"),
    # The float32 path (one lane per query on the VALU, no matrix cores) at a mid-size geometry, so
    # that its cost beyond the tiny workload is on record.
    ("sga4-32f-fp32", [dict(frames=32, grid_h=37, grid_w=37, heads=16, sigma=4, diag=True, mean=True)], "fp32"),
    ("dense+g2m-32f", [WORKLOADS["dense-32f"][0], WORKLOADS["dense-32f-f16"][0], WORKLOADS["g2m-32f"][0]], "bf16"),
    ("sga4-100f", [WORKLOADS["sga4-100f"][0]], "bf16"),
    ("g2f+sga9-200f", [WORKLOADS["g2f-200f"][0], WORKLOADS["sga9-200f"][0]], "bf16"),
    ("f16+phase-200f", [WORKLOADS["g2f-200f-f16"][0], WORKLOADS["sga9-200f-f16"][0],
                        WORKLOADS["sga9-200f-phase-global"][0]], "bf16"),
    ("sweep-200f", SWEEP_200, "bf16"),
]
# Run on the headline workload's own tensors (same geometry), before they are released.
SAME_TENSOR_EXTRAS = {"sga6-800f": ["sga6-800f-f16", "sga6-800f-phase", "sga6-800f-sized"],
                      "sga6-800f-phase": ["sga6-800f"], "sga6-800f-f16": ["sga6-800f"]}


def form_name(d) -> str:
    if d.get("g2f"):
        return "g2f-f16" if d.get("prescale_q") else "g2f"
    if d.get("g2m"):
        return "g2m"
    name = f"sigma{d.get('sigma', 1)}"
    if d.get("phase_shift"):
        name += "-phase"
    if d.get("mean_global"):
        name += "-globalmean"
    if d.get("log_size"):
        name += "-sized"
    if d.get("prescale_q"):
        name += "-f16"
    return name


class Sized:
    """Wraps a LOG_SIZE plan so that time_calls can call pack/forward without log sizes."""

    def __init__(self, plan, log_g):
        self.plan, self.log_g = plan, log_g

    def __getattr__(self, name):
        return getattr(self.plan, name)

    def forward(self, q, k, v, out, ws):
        self.plan.forward_sized(q, k, v, self.log_g, out, ws)

    def pack(self, k, v, ws):
        self.plan.pack_sized(k, v, self.log_g, ws)

KERNEL_SOURCES = ("vggt_global_attention_attn_amd/csrc/attn.hip", "vggt_global_attention_attn_amd/csrc/device_common.h",
                  "vggt_global_attention_attn_amd/csrc/plan.h")
TRAFFIC_FILE = "profiles/attn_{workload}_hbm_traffic.txt"
CLOCK_FILE = "profiles/attn_{workload}_clock.txt"
MFMA_BF16_FLOP_PER_CLK_CU = 4096  # 16x16x32 bf16 MFMA: 16384 flop per 16 cycles per SIMD, 4 SIMDs per CU


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 of the attention kernel's code: its sources without // comments, blank lines and
    surrounding whitespace, so that a comment edit keeps a traffic record while any code change
    voids it."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def profile_record(template: str, workload: str):
    """The JSON record of a committed rocprofv3 summary, if it was taken on the current kernel
    source; else None."""
    path = os.path.join(ROOT, template.format(workload=workload))
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("{") and '"source_sha256"' in line:
                rec = json.loads(line)
    if not rec or rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec


def measured_traffic(workload: str):
    """HBM bytes per attention launch from the committed PMC summary (FETCH_SIZE, WRITE_SIZE)."""
    rec = profile_record(TRAFFIC_FILE, workload)
    return rec.get("hbm_bytes_per_launch") if rec else None


def measured_clock(workload: str):
    """Sustained shader clock (GHz) of the attention kernel from the committed GRBM_GUI_ACTIVE
    summary of the same workload."""
    rec = profile_record(CLOCK_FILE, workload)
    return rec.get("gfx_clock_ghz") if rec else None


def clock_fields(flops: float, workload: str, cus: int) -> dict:
    """The bf16 matrix-core peak at the clock the kernel sustains, and the fraction of it reached,
    both from the committed GRBM_GUI_ACTIVE run (its own clock and kernel duration: the clock
    differs from box to box, so this run's time is not divided by another run's clock)."""
    rec = profile_record(CLOCK_FILE, workload)
    if rec is None:
        return {"clock_ghz": None, "peak_at_clock": None, "frac_at_clock": None}
    ghz = rec["gfx_clock_ghz"]
    peak = cus * MFMA_BF16_FLOP_PER_CLK_CU * ghz * 1e9 / 1e12
    return {"clock_ghz": ghz, "peak_at_clock": peak, "frac_at_clock": flops / rec["duration_s"] / 1e12 / peak,
            "clock_source": CLOCK_FILE.format(workload=workload)}


def gather_bytes(desc, c) -> int:
    """Algorithmic bytes of the gather/pack stage (bf16): read the K/V rows of S and the dropped
    rows that feed the means, write the packed K/V rows (padding included) and S."""
    H, d, e = desc["heads"], 64, 2
    L = 5 + desc["grid_h"] * desc["grid_w"]
    T = desc["frames"] * L
    if desc.get("g2f"):
        rows_read = T
        rows_written = desc["frames"] * ((L + 63) // 64) * 64
        index = 0
    else:
        n_drop_read = c["n_mean"] and (T - c["n_kv"])  # every dropped token feeds a mean
        rows_read = c["n_kv"] + (n_drop_read or 0)
        rows_written = (c["n_kv"] + c["n_mean"] + 63) // 64 * 64
        index = 4 * c["n_kv"]
    return int(H * (rows_read + rows_written) * d * e * 2 + index)


def time_calls(plans, tensors, outs, wss, steps, warmup):
    """Average seconds per step (all plans' forwards) and per plan's attention launch."""
    import torch
    for _ in range(warmup):
        for p, o, w in zip(plans, outs, wss):
            p.forward(*tensors, o, w)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in plans] for _ in range(steps)]
    t0 = time.perf_counter()
    for row in ev:
        for (e0, e1, e2), p, o, w in zip(row, plans, outs, wss):
            e0.record()
            p.pack(tensors[1], tensors[2], w)
            e1.record()
            p.attend(*tensors, o, w)
            e2.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    attn = [sum(row[i][1].elapsed_time(row[i][2]) for row in ev) / steps * 1e-3 for i in range(len(plans))]
    return wall, attn


def attention_entry(d, secs, flops, plan) -> dict:
    """One form's attention-stage time against its roofline: the bf16 MFMA peak, or for G2M (a
    broadcast of the mean value: out = v-bar, nothing to multiply) HBM bandwidth on its output
    writes, or for float32 plans the float32 vector ALU rate."""
    e = {"form": form_name(d), "ms": secs * 1e3, "kv_tokens": plan.counts()["n_kv"],
         "tflops": flops / secs / 1e12, "frac_bf16_peak": flops / secs / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    if plan.in_dtype == "fp32":
        e.update({"bound": "alu", "peak_fp32_tflops": FP32_VECTOR_PEAK_TFLOPS,
                  "frac_fp32_peak": flops / secs / 1e12 / FP32_VECTOR_PEAK_TFLOPS})
    if d.get("g2m"):
        out_bytes = plan.T * d["heads"] * 64 * 4
        e.update({"bound": "hbm", "out_bytes": out_bytes, "GB/s": out_bytes / secs / 1e9,
                  "frac_hbm_peak": out_bytes / secs / 1e9 / HBM_PEAK_GBS})
    return e


def sweep_ratios(descs, attn, flops) -> list:
    """Each form's attention time and algorithmic FLOPs as fractions of the dense form's (the
    group's sigma = 1 plan), beside its sigma: SGA's FLOPs fall about sigma times, so a
    time ratio near its FLOP ratio means the kernel keeps its efficiency on the smaller key set."""
    i0 = next(i for i, d in enumerate(descs) if d.get("sigma", 1) == 1 and not d.get("g2f") and not d.get("g2m"))
    return [{"form": form_name(d) + ("-enh" if d.get("diag") else ""), "sigma": d.get("sigma", 1),
             "ms": a * 1e3, "time_ratio_to_dense": a / attn[i0], "flop_ratio_to_dense": f / flops[i0],
             "dense_over_form": attn[i0] / a}
            for d, a, f in zip(descs, attn, flops)]


def timed_group(dev, name, descs, dtype, tensors, steps):
    """Time the forwards of one group of plans on shared tensors; one result entry."""
    import torch

    import vggt_global_attention_attn_amd as va

    plans = [va.Plan(**d, in_dtype=dtype, out_dtype="fp32") for d in descs]
    if any(d.get("log_size") for d in descs):
        from synth import make_log_sizes
        d0 = descs[0]
        _, lg = make_log_sizes(d0["frames"], d0["grid_h"], d0["grid_w"], 5, seed=5)
        lg = torch.from_numpy(lg).to(dev)
        plans = [Sized(p, lg) if d.get("log_size") else p for p, d in zip(plans, descs)]
    outs = [p.new_output(dev) for p in plans]
    wss = [p.new_workspace(dev) for p in plans]
    wall, attn = time_calls(plans, tensors, outs, wss, steps, warmup=1)
    flops = [p.counts()["flops"] for p in plans]
    T = plans[0].T
    entry = {"name": name, "ms_per_step": wall * 1e3, "queries_per_s": T / wall,
             "tflops": sum(flops) / wall / 1e12, "pct_bf16_peak": 100 * sum(flops) / wall / 1e12 / MFMA_BF16_PEAK_TFLOPS,
             "attention": [attention_entry(d, a, f, p) for d, a, f, p in zip(descs, attn, flops, plans)]}
    if name.startswith("sweep"):
        entry["ratios_to_dense"] = sweep_ratios(descs, attn, flops)
        for r in entry["ratios_to_dense"]:
            log(f"  {r['form']:>14s}: {r['ms']:8.3f} ms, time {r['time_ratio_to_dense']:.4f} of dense, "
                f"FLOPs {r['flop_ratio_to_dense']:.4f} of dense (sigma {r['sigma']})")
    log(f"extra {name}: {wall * 1e3:.3f} ms/step, {entry['tflops']:.1f} TFLOP/s")
    del outs, wss
    torch.cuda.empty_cache()
    return entry


def scheduled_pass(dev, frames: int, sigma: int, steps: int, qkv, model: str = "vggt") -> dict:
    """One pass over the 24 global layers of `model` under AVGGT's schedule ("AVGGT" notes,
    整体框架: G2F below t_early -- 9 for VGGT, 10 for pi^3 --, enhanced SGA sigma in the middle,
    dense for layers 20-23), each layer a full forward (pack + attend) on the given device Q/K/V
    of `frames` frames; beside it, 24 times the measured time of a dense layer, the cost of the
    same 24 layers without the schedule."""
    import torch

    import vggt_global_attention_attn_amd as va

    sl = va.ScheduledLayers(frames, 37, 37, 16, model=model, sigma=sigma, device=dev)
    qd, kd, vd = qkv
    outs = [p.new_output(dev) for p in sl.plans]
    for layer in range(va.GLOBAL_LAYERS):  # warm-up pass (also allocates the workspaces)
        sl.forward(layer, qd, kd, vd, outs[sl.index[layer]])
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(va.GLOBAL_LAYERS)] for _ in range(steps)]
    w0 = time.perf_counter()
    for row in ev:
        for layer, (e0, e1) in enumerate(row):
            e0.record()
            sl.forward(layer, qd, kd, vd, outs[sl.index[layer]])
            e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - w0) / steps
    per_layer = [sum(row[layer][0].elapsed_time(row[layer][1]) for row in ev) / steps for layer in range(24)]
    kinds = va.layer_schedule(model, sigma)
    by_form = {}
    for layer, kw in enumerate(kinds):
        name = "g2f" if kw["g2f"] else (f"sigma{kw['sigma']}-enh" if kw["sigma"] > 1 else "dense")
        by_form.setdefault(name, []).append(per_layer[layer])
    forms = {n: {"layers": len(t), "ms_per_layer": sum(t) / len(t)} for n, t in by_form.items()}
    dense_ms = forms["dense"]["ms_per_layer"]
    entry = {"name": f"avggt{sigma}-24layers-{frames}f" + ("" if model == "vggt" else f"-{model}"), "model": model, "sigma": sigma, "frames": frames,
             "ms_per_pass": wall * 1e3, "sum_of_layer_ms": sum(per_layer), "tflops": sl.flops() / wall / 1e12,
             "forms": forms, "dense_24_layers_ms": 24 * dense_ms,
             "speedup_vs_24_dense_layers": 24 * dense_ms / (wall * 1e3)}
    log(f"extra {entry['name']}: {wall * 1e3:.1f} ms per 24-layer pass, 24 dense layers {24 * dense_ms:.1f} ms "
        f"({entry['speedup_vs_24_dense_layers']:.2f}x); " + ", ".join(
            f"{n} {f['layers']} x {f['ms_per_layer']:.2f} ms" for n, f in forms.items()))
    del outs, sl
    torch.cuda.empty_cache()
    return entry


def extra_workloads(dev, steps: int):
    import numpy as np
    import torch

    from synth import make_qkv

    results = []
    shared = {}  # one set of device tensors per geometry and dtype, kept while groups use it
    for gi, (name, descs, dtype) in enumerate(EXTRA_GROUPS):
        d0 = descs[0]
        key = (d0["frames"], d0["grid_h"], d0["grid_w"], d0["heads"], dtype)
        if key not in shared:
            shared.clear()
            torch.cuda.empty_cache()
            q, k, v = make_qkv(d0["frames"], d0["grid_h"], d0["grid_w"], 5, d0["heads"], 64, dtype, seed=0)
            if dtype == "bf16":
                up = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
            else:
                up = lambda x: torch.from_numpy(x).to(dev)
            shared[key] = (up(q), up(k), up(v))
            del q, k, v
        results.append(timed_group(dev, name, descs, dtype, shared[key], steps))
    shared.clear()
    torch.cuda.empty_cache()
    q, k, v = make_qkv(100, 37, 37, 5, 16, 64, "bf16", seed=0)
    up = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    qkv = (up(q), up(k), up(v))
    del q, k, v
    for model in ("vggt", "pi3"):
        results.append(scheduled_pass(dev, 100, 9, steps=2, qkv=qkv, model=model))
    del qkv
    torch.cuda.empty_cache()
    return results


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sga6-800f", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024, help="query rows in the timed oracle sample (cpu_baseline)")
    ap.add_argument("--parity-rows", type=int, default=4096,
                    help="seeded sampled query rows checked against the oracle (the timed sample plus the rest)")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (PMC scale calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import vggt_global_attention_attn_amd as va
    from synth import host_threads, make_qkv, sample_rows

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    desc, description = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    plan = va.Plan(**desc, in_dtype="bf16", out_dtype="fp32")
    log_g = None
    if desc.get("log_size"):
        from synth import make_log_sizes
        _, log_g = make_log_sizes(desc["frames"], desc["grid_h"], desc["grid_w"], 5, seed=5)
        plan = Sized(plan, torch.from_numpy(log_g).to(dev))
    counts = plan.counts()
    T, H = plan.T, plan.heads

    log(f"workload {args.workload}: T={T} heads={H} |S|={counts['n_kv']} M={counts['n_mean']} "
        f"n_diag={counts['n_diag']} flops={counts['flops']:.4e}")
    t0 = time.time()
    q, k, v = make_qkv(desc["frames"], desc["grid_h"], desc["grid_w"], 5, H, 64, "bf16", seed=0)
    log(f"inputs drawn in {time.time() - t0:.1f} s")

    def up(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    qd, kd, vd = up(q), up(k), up(v)
    if args.no_cpu_baseline:
        del q, k, v
    out = plan.new_output(dev)
    ws = plan.new_workspace(dev)
    torch.cuda.synchronize()

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy of {args.calib_copy_mib} MiB done")

    for i in range(args.warmup):
        plan.forward(qd, kd, vd, out, ws)
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup}")

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record()
        plan.pack(kd, vd, ws)
        e1.record()
        plan.attend(qd, kd, vd, out, ws)
        e2.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    t_gather = sum(e0.elapsed_time(e1) for e0, e1, _ in ev) / len(ev) * 1e-3
    t_attn = sum(e1.elapsed_time(e2) for _, e1, e2 in ev) / len(ev) * 1e-3
    fwd_ms = sorted(e0.elapsed_time(e2) for e0, _, e2 in ev)
    t_fwd_median = fwd_ms[len(fwd_ms) // 2] * 1e-3
    step_s = wall / args.steps
    log(f"timed {args.steps} steps: {step_s * 1e3:.3f} ms/step (gather {t_gather * 1e3:.3f} ms, attention {t_attn * 1e3:.3f} ms)")

    flops = counts["flops"]
    achieved = flops / t_attn / 1e12
    if not args.no_cpu_baseline:  # keep the sampled rows of this run's output for the parity check
        # 4096 seeded rows (the forced coverage set and PCG64(1) draws); the oracle is timed on an
        # evenly spaced 1024 of them (cpu_baseline) and then computes the rest for parity only.
        rows_all = sample_rows(desc["frames"], desc["grid_h"], desc["grid_w"], 5, count=args.parity_rows, seed=1)
        step = max(1, rows_all.size // args.cpu_rows)
        timed_sel = np.zeros(rows_all.size, dtype=bool)
        timed_sel[::step] = True
        timed_sel[np.flatnonzero(timed_sel)[args.cpu_rows:]] = False
        rows = rows_all[timed_sel]
        rest = rows_all[~timed_sel]
        out_rows = out[:, torch.from_numpy(rows).to(dev)].double().cpu().numpy()
        out_rest = out[:, torch.from_numpy(rest).to(dev)].double().cpu().numpy() if rest.size else None
    traffic = measured_traffic(args.workload)
    gbytes = gather_bytes(desc, counts)
    result = {
        "metric": METRIC,
        "value": T / step_s,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": description, "name": args.workload, "form": form_name(desc), "frames": desc["frames"],
                   "tokens": T, "heads": H, "head_dim": 64, "sigma": desc.get("sigma", 1), "kv_tokens": counts["n_kv"],
                   "mean_tokens": counts["n_mean"], "diag_queries": counts["n_diag"]},
        "query_heads_per_s": H * T / step_s,
        "tflops": flops / step_s / 1e12,
        "pct_bf16_peak": 100.0 * flops / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "t_gather_ms": t_gather * 1e3,
        "t_attn_ms": t_attn * 1e3,
        "t_fwd_median_ms": t_fwd_median * 1e3,
        "gather": {"bytes": gbytes, "GB/s": gbytes / t_gather / 1e9, "frac_hbm_peak": gbytes / t_gather / 1e9 / HBM_PEAK_GBS},
        "roofline": {"bound": "mfma", "kernel": "attn_bf16_kernel", "achieved": achieved,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": traffic, "algorithmic_flops_per_launch": flops,
                     **clock_fields(flops, args.workload, torch.cuda.get_device_properties(dev).multi_processor_count)},
        "device": torch.cuda.get_device_name(dev),
        "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count,
        "hip_version": torch.version.hip,
    }

    if not args.no_extra:
        del out, ws
        torch.cuda.empty_cache()
        same = [timed_group(dev, n, [WORKLOADS[n][0]], "bf16", (qd, kd, vd), steps=3)
                for n in SAME_TENSOR_EXTRAS.get(args.workload, [])]
        del qd, kd, vd
        torch.cuda.empty_cache()
        result["other_workloads"] = same + extra_workloads(dev, steps=3)
        # The same attention kernel in the f16 score form on the headline tensors (opt-in flag).
        for e in same:
            if e["name"] == args.workload + "-f16":
                a = e["attention"][0]
                result["roofline_f16_score_form"] = {
                    "bound": "mfma", "kernel": "attn_bf16_kernel (PRESCALE_Q)", "achieved": a["tflops"],
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": a["frac_bf16_peak"],
                    "traffic": measured_traffic(e["name"]),
                    **clock_fields(flops, e["name"], torch.cuda.get_device_properties(dev).multi_processor_count),
                    "note": "QK^T on f16 matrix cores (same dense peak as bf16), PV on bf16"}

    if not args.no_cpu_baseline:
        import oracle
        from oracle import Desc
        odesc = Desc(**{k: v for k, v in desc.items() if k != "prescale_q"})
        cores = host_threads()
        log(f"oracle on {rows.size} rows x {H} heads with {cores} threads")
        c0 = time.perf_counter()
        ref = oracle.attention(q, k, v, odesc, rows=rows, workers=cores, log_g=log_g)
        c_s = time.perf_counter() - c0
        got, refs = [out_rows], [ref]
        if out_rest is not None:
            log(f"oracle on the other {rest.size} parity rows")
            refs.append(oracle.attention(q, k, v, odesc, rows=rest, workers=cores, log_g=log_g))
            got.append(out_rest)
        got, ref = np.concatenate(got, axis=1), np.concatenate(refs, axis=1)
        diff = got - ref
        oflops = flops * rows.size / T  # the same formula restricted to the sampled rows
        result["cpu_baseline"] = {
            "value": rows.size / c_s, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "gflops": oflops / c_s / 1e9,
            "sample": f"{rows.size} seeded query rows (all {H} heads) of the same workload, float64 NumPy, "
                      f"{c_s:.1f} s including its own index-set and mean computation",
            "seconds": c_s,
        }
        result["parity_sample"] = {"rows": int(ref.shape[1]), "max_abs": float(np.abs(diff).max()),
                                   "rel_l2": float(np.linalg.norm(diff) / np.linalg.norm(ref)),
                                   "bar": {"max_abs": 2e-2, "rel_l2": 5e-3},
                                   "within_bar": bool(np.abs(diff).max() <= 2e-2 and
                                                      np.linalg.norm(diff) / np.linalg.norm(ref) <= 5e-3)}
        log(f"oracle {c_s:.1f} s; parity max-abs {result['parity_sample']['max_abs']:.3e} "
            f"rel-L2 {result['parity_sample']['rel_l2']:.3e}")

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
