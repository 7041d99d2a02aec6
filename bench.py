#!/usr/bin/env python3
"""Muon optimizer step benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload moe1b]

A step is one whole Muon step over every hidden 2-D matrix of the workload
(by default the MoE model with 1B parameters in total: 4288 matrices, 3.03 G
elements, the largest full model of the workloads):
momentum/Nesterov head, 5 Newton-Schulz iterations, scale/decay/update tail,
issued as ONE grouped launch sequence (muon_step_grouped) on inputs already
resident in HBM (the 2k-hidden stress set, whose whole-model workspace would
not fit beside its 189 GB of W, G and M, as a few calls over even chunks of
its groups, --max-workspace-gb).  Without --warmup, the untimed warmup runs
as many steps as take 0.25 s (at least 3): on the GPU the first ten or so
steps run up to 20 % slower while its clocks ramp up.  Prints one JSON line:

  value       optimizer steps per second (whole job = one GPU)
  roofline    the dominant kernel (the Newton-Schulz update GEMM) against
              the roof its arithmetic intensity puts it under (HBM below the
              ridge point, MFMA above): algorithmic bytes or flops per launch
              over its average launch time, timed live with HIP events on the
              launch stream; both views are given
  ns / head / tail   phase figures: NS TFLOP/s vs the bf16 MFMA peak and the
              elementwise phases' GB/s vs HBM peak
  cpu_baseline  the fp64 oracle on the host cores on a bounded sample of the
              same matrices, extrapolated to the full workload
  aux_adamw   the other half of the hybrid optimizer, timed separately (not
              part of `value`): one grouped AdamW call over the model's
              embedding, head and gains, its GB/s against HBM peak
  workloads   the other workloads, each timed the same way after the main
              one in the same run (not part of `value`): GPT-160M, GPT-400M
              (Muon and MuonGS), the 2k-hidden stress set (fewer steps) and
              the single fp32 256x512 matrix (latency)
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

METRIC = "Muon optimizer steps/sec (full model) + NS TFLOP/s as % of bf16 MFMA peak"
PEAK_MFMA = {"bf16": 2.5e15, "f32": 157.3e12}   # dense, published MI355X figures
PEAK_HBM = 8.0e12
HP = dict(lr=0.02, momentum=0.95, weight_decay=0.1, ns_steps=5)
NS_COEFFS = (3.4445, -4.7750, 2.0315)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps (default: as many as take 0.25 s, at least 3: "
                         "the GPU's clocks ramp up over the first tens of milliseconds)")
    ap.add_argument("--workload", default="moe1b")
    ap.add_argument("--variant", default="muon", choices=["muon", "muongs", "muonh", "normuon", "meqmuon"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time for the oracle baseline sample")
    ap.add_argument("--max-workspace-gb", type=float, default=32.0,
                    help="workspace budget; a model whose step needs more runs as several "
                         "grouped calls per step (2k-hidden stress set)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-phase-profile", action="store_true")
    ap.add_argument("--no-aux", action="store_true", help="skip the AdamW-side measurement")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only --workload (not the other workloads after it)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy three times (the reference "
                         "kernel for scaling FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
# Committed counter summaries, one per workload: profiles/ns_update_<workload>_hbm_traffic.md
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ns_update_{}_hbm_traffic.md")
# The sources the update kernel is built from: traffic counters are only
# reported while these are unchanged since the counters were taken.
KERNEL_SOURCES = ("muon_step_03_amd/csrc/k_ns_bf16.hip", "muon_step_03_amd/csrc/muon_internal.h")
COPY_BYTES = 256 * 1024 * 1024


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per update launch from the committed counter summary, or
    None if there is none for this workload or the kernel has changed."""
    path = TRAFFIC_FILE.format(workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and line.split(":", 1)[0].strip() in (
                    "traffic_bytes_per_launch", "kernel_source_sha256"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}), flush=True)


def matrix_work(groups, dtype_bytes):
    """Algorithmic work per step, from the true (unpadded) shapes."""
    gram = poly = upd = 0.0
    elems = 0
    for g in groups:
        p, q = min(g.rows, g.cols), max(g.rows, g.cols)
        gram += g.count * p * p * q            # symmetric X X^T: half of 2p^2q
        poly += g.count * p ** 3               # symmetric A A^T: half of 2p^3
        upd += g.count * 2.0 * p * p * q       # B X
        elems += g.count * g.rows * g.cols
    es = dtype_bytes
    upd_bytes = sum(g.count * (min(g.rows, g.cols) ** 2 + 2 * g.rows * g.cols) * dtype_bytes
                    for g in groups)                      # B r, X r, X' w
    return dict(gram=gram, poly=poly, update=upd, elems=elems, update_bytes=upd_bytes,
                head_bytes=elems * (es + 4 + 4 + es),   # G r, M r+w, X0 w
                tail_bytes=elems * (es + es + es))      # W r, O r, W w


def cpu_baseline(w, Ws, Gs, Ms, seconds):
    """The oracle, untuned, on the workload's own inputs (copied from the
    device before the GPU's first step), one whole matrix at a time in layer
    order (round-robin over the shape groups) until about `seconds` of CPU
    time, extrapolated per shape to the full matrix count."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()
                       if t.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    per_shape = {}
    order = []
    for k in range(max(g.count for g in w.groups)):
        for gi, g in enumerate(w.groups):
            if k < g.count:
                order.append((gi, k))
    spent = 0.0
    done = 0
    # cycle over the model until about `seconds` (at most 4 passes)
    for gi, k in order * 4:
        g = w.groups[gi]
        Wd = Ws[gi][k].double().cpu().numpy()
        Gd = Gs[gi][k].double().cpu().numpy()
        Md = Ms[gi][k].double().cpu().numpy()
        t0 = time.perf_counter()
        oracle.muon_step(Wd, Gd, Md, **HP)
        dt = time.perf_counter() - t0
        per_shape.setdefault((g.rows, g.cols), []).append(dt)
        spent += dt
        done += 1
        if spent >= seconds and len(per_shape) == len(w.groups):
            break
    total = sum(g.count * (sum(per_shape[(g.rows, g.cols)]) / len(per_shape[(g.rows, g.cols)]))
                for g in w.groups)
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:  # pragma: no cover
        pass
    return {"value": 1.0 / total, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} matrix steps over the {w.n_matrices} matrices (the GPU's own "
                      f"inputs, round-robin over the shape groups), {spent:.1f} s of fp64 NumPy; "
                      f"seconds/step = per-shape mean x count",
            "seconds_per_step": total, "host_cpus": os.cpu_count(), "cpu_model": model}


def aux_adamw(args, wl, dev, stream, muon_ms):
    """AdamW over the workload's embedding, head and gains (bf16 parameters and
    gradients, float32 moments): one grouped call per step, K timed calls
    after W warm-up calls, each launch timed with HIP events."""
    import torch
    from muon_step_03_amd import AUX_LR, _lib, adamw_step_grouped, adamw_tensor
    name = args.workload
    Ps = wl.make_aux_params(name, dev)
    Gs = wl.make_aux_grads(name, 1, dev)
    mv = wl.make_aux_moments(name, dev)
    roles = [t.role for t in wl.AUX_SETS[name]]
    descs = [adamw_tensor(P, G, m, v, lr=AUX_LR[r]) for P, G, (m, v), r in zip(Ps, Gs, mv, roles)]
    elems = sum(P.numel() for P in Ps)
    state = {"t": 0}

    def call():
        state["t"] += 1
        adamw_step_grouped(descs, torch.bfloat16, step=state["t"], stream=stream)

    for _ in range(args.warmup or 3):
        call()
    torch.cuda.synchronize()
    L = _lib.lib()
    L.muon_profile_enable(1)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    L.muon_profile_enable(0)
    n = _lib.MUON_NUM_PHASES
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    assert L.muon_profile_read(ms, cnt, n) == 0
    k = [L.muon_phase_name(i).decode() for i in range(n)].index("adamw")
    launch_ms = ms[k] / cnt[k]
    call_ms = ms[k] / args.steps
    nbytes = elems * (2 + 2 + 2 + 4 + 4 + 4 + 4)   # P r+w, G r, m r+w, v r+w
    return {"tensors": len(Ps), "elements": elems, "launches_per_step": cnt[k] / args.steps,
            "ms_per_step": call_ms, "wall_ms_per_step": wall_ms,
            "avg_launch_ms": launch_ms, "alg_bytes_per_step": nbytes,
            "gbps": nbytes / (call_ms * 1e-3) / 1e9,
            "frac_of_hbm": nbytes / (call_ms * 1e-3) / PEAK_HBM,
            "hybrid_ms_per_step": muon_ms + call_ms,
            "hyper": {"betas": [0.8, 0.95], "eps": 1e-10, "weight_decay": 1e-3, "lr": AUX_LR}}


def roofline(flops, nbytes, seconds, peak_flops, peak_bw=PEAK_HBM):
    """One launch against the roof its arithmetic intensity puts it under:
    HBM below the ridge point (peak flops / peak bandwidth), MFMA above it;
    both views are kept."""
    intensity, ridge = flops / nbytes, peak_flops / peak_bw
    mfma_view = {"achieved": flops / seconds / 1e12, "peak": peak_flops / 1e12,
                 "unit": "TFLOP/s", "frac": flops / seconds / peak_flops,
                 "alg_flops_per_launch": flops}
    hbm_view = {"achieved": nbytes / seconds / 1e9, "peak": peak_bw / 1e9, "unit": "GB/s",
                "frac": nbytes / seconds / peak_bw, "alg_bytes_per_launch": nbytes}
    main = hbm_view if intensity < ridge else mfma_view
    return {"bound": "hbm" if intensity < ridge else "mfma", "achieved": main["achieved"],
            "peak": main["peak"], "unit": main["unit"], "frac": main["frac"],
            "alg_flops_per_launch": flops, "alg_bytes_per_launch": nbytes,
            "flop_per_byte": intensity, "ridge_flop_per_byte": ridge,
            "mfma_view": mfma_view, "hbm_view": hbm_view}


def phase_profile(L, step, steps, w, es):
    """Per-launch kernel times (HIP events on the launch stream, recorded by
    the library around every launch) over `steps` more steps: the roofline
    of the update launch, the Newton-Schulz phase and the head/tail GB/s."""
    from muon_step_03_amd import _lib
    import torch
    L.muon_profile_enable(1)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    L.muon_profile_enable(0)
    n = _lib.MUON_NUM_PHASES
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    assert L.muon_profile_read(ms, cnt, n) == 0
    names = [L.muon_phase_name(i).decode() for i in range(n)]
    avg = {names[i]: (ms[i] / cnt[i] if cnt[i] else 0.0) for i in range(n)}
    per_step = {names[i]: ms[i] / steps for i in range(n)}
    per = {names[i]: cnt[i] / steps for i in range(n)}
    work = matrix_work(w.groups, es)
    peak = PEAK_MFMA[w.dtype]
    out = {}
    # Algorithmic flops per "update" launch: the update work of every
    # iteration timed in this phase (the last one is timed apart when it
    # also applies the step), spread over its launches (two per iteration
    # when a phase runs both tile sizes, more when the model is split over
    # several calls).
    upd_iters = HP["ns_steps"] - (1 if per["update_tail"] > 0 else 0)
    if per["update"] > 0:
        upd_flops = work["update"] * upd_iters / per["update"]
        # The launch's algorithmic bytes (B and X read once, X' written once,
        # unpadded shapes) and its arithmetic intensity decide which roof
        # bounds it: below the ridge point (dense peak / HBM peak) the HBM
        # roof is the lower one (the MoE experts: short side 512), above it
        # the MFMA roof.  Both fractions are reported.
        upd_bytes = work["update_bytes"] * upd_iters / per["update"]
        out["roofline"] = dict(
            {"kernel": "ns_update (X' = BX, B = aI + bA + cA^2)" if w.dtype == "bf16"
                       else "ns_update (X' = aX + BX)"},
            **roofline(upd_flops, upd_bytes, avg["update"] * 1e-3, peak),
            traffic=measured_traffic(w.name), avg_launch_ms=avg["update"])
    ns_ms = per_step["gram"] + per_step["poly"] + per_step["update"] + per_step["update_tail"]
    ns_flops = HP["ns_steps"] * (work["gram"] + work["poly"] + work["update"])
    out["ns"] = {"ms_per_step": ns_ms, "tflops": ns_flops / (ns_ms * 1e-3) / 1e12,
                 "frac_of_peak": ns_flops / (ns_ms * 1e-3) / peak,
                 "alg_tflop_per_step": ns_flops / 1e12,
                 "avg_launch_ms": {k: avg[k] for k in ("gram", "poly", "update")}}
    if per_step["update_tail"] > 0:
        out["ns"]["last_update_with_step_ms"] = avg["update_tail"]
    # per step: a model split over several calls has one head launch per call
    out["head"] = {"ms": per_step["head"],
                   "gbps": work["head_bytes"] / (per_step["head"] * 1e-3) / 1e9,
                   "frac_of_hbm": work["head_bytes"] / (per_step["head"] * 1e-3) / PEAK_HBM}
    tail_ms = per_step["tail_apply"] + per_step["tail_reduce"] + per_step["tail_finalize"]
    if tail_ms > 0:
        out["tail"] = {"ms": tail_ms, "gbps": work["tail_bytes"] / (tail_ms * 1e-3) / 1e9,
                       "frac_of_hbm": work["tail_bytes"] / (tail_ms * 1e-3) / PEAK_HBM}
    else:
        out["tail"] = {"ms": 0.0, "fused_into_last_update": True}
    out["phase_ms_per_step"] = per_step
    return out


def measure(name, variant, steps, warmup, args, cpu_seconds=None, main=False):
    """Times exactly `steps` whole steps of workload `name` (after `warmup`
    untimed ones, or 0.25 s of them when None), then the same number again
    with one event pair per step, then the phase profile.  Inputs are drawn
    on the device and stay resident; they are freed on return."""
    import torch
    from muon_step_03_amd import _lib, muon_step_grouped, stacked_chunks
    from muon_step_03_amd import workloads as wl

    w = wl.WORKLOADS[name]
    dev = torch.device("cuda", 0)
    tdtype = wl.torch_dtype(w.dtype)
    es = 2 if w.dtype == wl.BF16 else 4
    torch.cuda.empty_cache()
    Ws = wl.make_weights(w, dev)
    Gs = wl.make_grads(w, 0, dev)
    Ms = wl.make_momentum(w, dev)
    torch.cuda.empty_cache()   # the generators' float32 temporaries
    out = {}
    if cpu_seconds:
        # the oracle on the GPU's own inputs, before the first GPU step
        out["cpu_baseline"] = cpu_baseline(w, Ws, Gs, Ms, cpu_seconds)
    # One grouped call over the whole model when its workspace fits the
    # budget (every workload but the 2k-hidden stress set), else the fewest
    # calls over even chunks of every group.
    calls, ws_bytes = stacked_chunks(zip(Ws, Gs, Ms), tdtype, int(args.max_workspace_gb * 2**30))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    hp = dict(HP, ns_coefficients=NS_COEFFS, variant=variant)

    def step():
        for groups in calls:
            muon_step_grouped(groups, tdtype, workspace=ws, device=dev, stream=stream, **hp)

    if warmup is None:
        # by time: at least 3 steps and 0.25 s of work
        torch.cuda.synchronize()
        t_w, n_w = time.perf_counter(), 0
        while n_w < 3 or time.perf_counter() - t_w < 0.25:
            step()
            n_w += 1
            if n_w % 8 == 0:
                torch.cuda.synchronize()
        warmup = n_w
    else:
        for _ in range(warmup):
            step()
    torch.cuda.synchronize()
    print(f"# {name} {variant}: warmup done ({warmup} steps)", file=sys.stderr, flush=True)

    # ---- timed region: exactly `steps` steps, synchronised on both sides
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ev_ms = start.elapsed_time(stop)
    ms_per_step = max(ev_ms, wall_ms) / steps
    print(f"# {name} {variant}: timed {steps} steps: {ms_per_step:.4f} ms/step",
          file=sys.stderr, flush=True)

    # ---- per-step distribution: the same number of steps again, one event pair each
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    per_step_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)

    def pct(q):
        return per_step_ms[min(len(per_step_ms) - 1, int(q * (len(per_step_ms) - 1) + 0.5))]

    out.update({
        "value": 1e3 / ms_per_step, "ms_per_step": ms_per_step, "steps": steps, "warmup": warmup,
        "dtype": w.dtype,
        "config": {"workload": w.name, "description": w.description, "matrices": w.n_matrices,
                   "elements": w.n_elements, "variant": variant, "ns_steps": HP["ns_steps"],
                   "lr": HP["lr"], "momentum": HP["momentum"],
                   "weight_decay": HP["weight_decay"],
                   "launch": ("muon_step_grouped, one launch sequence per step" if len(calls) == 1
                              else f"muon_step_grouped, {len(calls)} calls per step over "
                                   f"chunks of {calls[0][0].count} matrices per shape"),
                   "workspace_bytes": ws_bytes},
        "step_ms": {"p10": pct(0.1), "median": pct(0.5), "p90": pct(0.9),
                    "note": "a second pass of the same number of steps, one event pair per step"},
    })
    if not args.no_phase_profile:
        out.update(phase_profile(_lib.lib(), step, steps, w, es))
    if main and not args.no_aux and name in wl.AUX_SETS:
        out["aux_adamw"] = aux_adamw(args, wl, dev, stream, ms_per_step)
    del Ws, Gs, Ms, ws, calls
    torch.cuda.empty_cache()
    return out


# The other workloads timed after the main one: (name, variant, steps, warmup);
# None takes --steps / --warmup.  The stress set moves 189 GB of W, G and M per
# step (about a second): two timed steps after one warm-up.
EXTRAS = (("gpt160m", "muon", None, None), ("gpt400m", "muon", None, None),
          ("gpt400m", "muongs", None, None), ("moe1b", "muongs", None, None),
          ("stress2k", "muon", 2, 1), ("fp32_256x512", "muon", None, None))


def summary(r):
    """The figures of one extra workload kept in the JSON line."""
    keys = ("value", "ms_per_step", "steps", "warmup", "dtype", "config", "step_ms")
    out = {k: r[k] for k in keys if k in r}
    out["unit"] = "steps/s"
    if "roofline" in r:
        out["roofline_update"] = {k: r["roofline"][k] for k in
                                  ("bound", "achieved", "unit", "frac", "avg_launch_ms",
                                   "traffic", "flop_per_byte")}
        out["roofline_update"]["mfma_frac"] = r["roofline"]["mfma_view"]["frac"]
        out["roofline_update"]["hbm_frac"] = r["roofline"]["hbm_view"]["frac"]
    for k in ("ns", "head", "tail", "phase_ms_per_step"):
        if k in r:
            out[k] = r[k]
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): this build has no multi-GPU path; each GPU would run the same "
              "step on its own share of the matrices.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    from muon_step_03_amd import workloads as wl

    torch.cuda.set_device(torch.device("cuda", 0))
    w = wl.WORKLOADS[args.workload]
    main_r = measure(args.workload, args.variant, args.steps, args.warmup, args,
                     cpu_seconds=None if args.no_cpu_baseline else args.cpu_seconds, main=True)
    result = {
        "metric": METRIC, "value": main_r["value"], "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": main_r["warmup"], "ms_per_step": main_r["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian W ~ N(0, 0.02^2), G ~ N(0, 1e-3^2), M = 0)",
        "config": main_r["config"], "step_ms": main_r["step_ms"],
    }
    for k in ("roofline", "ns", "head", "tail", "phase_ms_per_step", "aux_adamw", "cpu_baseline"):
        if k in main_r:
            result[k] = main_r[k]
    if not args.no_extras:
        result["workloads"] = {}
        for name, variant, steps, warmup in EXTRAS:
            if (name, variant) == (args.workload, args.variant):
                continue
            r = measure(name, variant, steps or args.steps,
                        warmup if steps else args.warmup, args)
            result["workloads"][f"{name}/{variant}"] = summary(r)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
