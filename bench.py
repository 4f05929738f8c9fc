"""Throughput of the owner-rank Muon step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--publish]
    python bench.py --route adamw [--workload adamw_stream|adamw_llama_norms]

A step is one Muon step over every matrix of the workload
(momentum, per-slice normalisation, k = 5 quintic Newton–Schulz iterations,
decoupled decay + lr-scaled update), with all inputs already resident in HBM.
Prints one JSON line.  ``value`` is matrices stepped per second; the line also
carries the effective TFLOP/s (Σ k·(4m²n + 2m³) per step), its share of the bf16
dense matrix-core peak, a roofline entry for the dominant kernel and the fp64 CPU
oracle timed on a bounded sample of the same workload.

A step is prepared once (``dmuon_muon_step_prepare`` writes the tables for the
workload's tensors into the workspace) and every timed step is one
``dmuon_muon_step_run``.  The step is timed twice.  The first timed pass gives
``value``: the library's own launch configuration (it may split the tensors into
concurrent stream groups on side streams), no per-launch events.  The second pass
runs the same kernels on one stream (``stream_groups`` = 1) with HIP events
around every launch on that stream;
the roofline and the per-phase times come from it, because the duration of a
launch that shares the GPU with another stream's kernels says nothing about
the kernel itself.  ``--stream-groups N`` fixes the group count of the first
pass (``--stream-groups 1`` makes both passes alike, which is the configuration
the committed rocprofv3 kernel summaries are taken on).  ``--publish`` also writes the
bf16 published copy of every updated master inside the step.

After the two passes the line's ``mfma_ceiling`` times the probe library's
matrix-core-only waves (v_mfma_f32_16x16x32_bf16 on random register operands,
the bf16 contraction kernels' instruction) for 3 s under the same board power
limit; ``roofline.frac_of_mfma_ceiling`` is the dominant kernel's rate over
that ceiling.  ``--mfma-probe`` prints the ceiling of both instruction shapes on
random and zero operands.

``--graph`` captures the prepared step of the first pass into a HIP graph and
times its replays instead (one graph launch per step), which shows what the
launches themselves cost on small workloads.

``--route adamw`` measures the ``adamw`` route instead: one ``dmuon_adamw_step``
over the workload's 1-D parameters per step; ``value`` is elements per second
and the roofline is HBM bandwidth against algorithmic bytes (gradient read,
parameter and both moments read and written, plus the bf16 copy).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)
DEFAULT_WORKLOAD = "mlp_moe_large"
METRIC = "Muon NS step matrices/s + TFLOP/s and % bf16 MFMA peak, 1\u00d7MI355X"
ADAMW_METRIC = "adamw route elements/s (owner 1-D parameters), 1\u00d7MI355X"
ADAMW_DEFAULT_WORKLOAD = "adamw_stream"
# sources that decide what a launch does: the kernels and the planner (grouping, tiling)
KERNELS_SRC = [os.path.join(ROOT, "matrix_optimizer_muon_amd", "csrc", f) for f in ("kernels.hip", "abi.cpp")]
PROFILES = os.path.join(ROOT, "profiles")


def kernels_sha256():
    import hashlib
    h = hashlib.sha256()
    for path in KERNELS_SRC:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel, workload_name):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter summary.

    The summary records FETCH_SIZE and WRITE_SIZE per dispatch, calibrated by the
    same counters on a plain device copy of known size, and the sha256 of the
    kernel and planner sources they were taken on; a different source gives None.
    """
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload_name}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and line.strip().startswith("- "):
                k, v = line.strip()[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernels_sha256") != kernels_sha256():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measured_mfma_busy(workload_name):
    """Per-kernel matrix-core busy share and clock from the committed rocprofv3
    counter summary (GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES), or None when the
    summary is missing or was taken on other kernel sources."""
    path = os.path.join(PROFILES, f"mfma_busy_{workload_name}.md")
    if not os.path.exists(path):
        return None
    out, sha = {}, None
    with open(path) as f:
        for line in f:
            if line.strip().startswith("- kernels_sha256:"):
                sha = line.split(":", 1)[1].strip().strip("`")
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if len(cells) == 6 and cells[3].replace(".", "", 1).isdigit() and cells[4].endswith("%"):
                out[cells[0].replace("\u2212", "-")] = {"clock_ghz": float(cells[3]),
                                                        "mfma_busy": round(float(cells[4][:-1]) / 100, 4)}
    if sha != kernels_sha256() or not out:
        return None
    return {"source": os.path.relpath(path, ROOT), "kernels": out,
            "note": "mfma_busy is the share of the dispatch's cycles the matrix cores are busy; "
                    "under the board's power limit a cheaper instruction raises the clock and "
                    "lowers this share while the kernel gets faster"}


def peak_clock_mhz(device_index):
    """The device's peak shader clock (hipDeviceGetAttribute with
    hipDeviceAttributeClockRate, value 5 in ROCm 7's hip_runtime_api.h, in kHz),
    read through the HIP runtime torch has already loaded (same soname)."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
    except OSError:
        return None
    v = ctypes.c_int(0)
    if hip.hipDeviceGetAttribute(ctypes.byref(v), ctypes.c_int(5), ctypes.c_int(device_index)) != 0:
        return None
    return round(v.value / 1000.0, 1)


def copy_probe(nbytes):
    """A plain device-to-device copy of known size (counter calibration)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}), flush=True)


def mfma_ceiling(shape=32, operands=0, seconds=3.0, settle=1.0):
    """What the matrix cores sustain on their own: the probe library's waves issue
    only bf16 MFMAs (32×32×16 or 16×16×32) on register operands, back to back,
    for ``settle`` seconds and then ``seconds`` timed with HIP events on the
    launch stream, while a thread samples the board power and shader clock the
    driver reports (torch.cuda.power_draw / clock_rate, amd-smi's readings).
    With random operands this is the ceiling the board's power limit sets; with
    zero operands (operands=1) it is the unloaded bound."""
    import threading
    import torch
    from matrix_optimizer_muon_amd import probe

    blocks, iters = 2048, 20000
    sink = torch.empty(blocks * probe.THREADS, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    launch = lambda: probe.probe_mfma(shape, operands, blocks, iters, sink.data_ptr(), st.cuda_stream)
    t_end = time.perf_counter() + settle
    while time.perf_counter() < t_end:
        launch()
        torch.cuda.synchronize()
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                samples.append((float(torch.cuda.power_draw()), float(torch.cuda.clock_rate())))
            except Exception:
                return
            time.sleep(0.05)

    th = threading.Thread(target=sample)
    th.start()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    ev0.record(st)
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(4):
            launch()
        n += 4
        torch.cuda.synchronize()
    ev1.record(st)
    torch.cuda.synchronize()
    stop.set()
    th.join()
    ms = ev0.elapsed_time(ev1) / n
    tflops = probe.flops_per_launch(blocks, iters) / (ms * 1e-3) / 1e12
    out = {"instruction": f"v_mfma_f32_{shape}x{shape}x{512 // shape}_bf16",
           "operands": "random bf16" if operands == 0 else "zero",
           "tflops": round(tflops, 1), "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
           "launches": n, "ms_per_launch": round(ms, 3), "power_w": None, "clock_mhz": None}
    if samples:
        out["power_w"] = round(sum(p for p, _ in samples) / len(samples), 1)
        out["clock_mhz"] = round(sum(c for _, c in samples) / len(samples), 1)
    return out


def mfma_probe():
    """--mfma-probe: the matrix-core ceiling for both instruction shapes, random
    and zero operands, one JSON line each."""
    for shape in (32, 16):
        for operands in (0, 1):
            print(json.dumps(mfma_ceiling(shape, operands)), flush=True)


def copy_ceiling_gbs(nbytes=1 << 30, reps=10):
    """Bytes per second (read + write) of a plain 1 GiB device-to-device copy,
    timed with HIP events: the practical ceiling of a kernel that writes as
    much as it reads."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def ingest_bytes_per_elem(grad_dtype, precision):
    """(algorithmic, moved) HBM bytes per element of the momentum kernel: the
    gradient read, the momentum read and written; it also writes the first
    iteration's operand copy of B (bf16, or fp32 in both orientations on the
    fp32 path)."""
    alg = (2 if grad_dtype == "bf16" else 4) + 8
    return alg, alg + (2 if precision == "bf16" else 8)


def matrices_of(wl, share=None):
    """(rows, cols, batch) of every stepped slice group."""
    ts = wl.tensors if share is None else [wl.tensors[i] for i in share]
    return ts


def ns_flops(ts, steps):
    tot = 0
    for t in ts:
        b = t.shape[0] if len(t.shape) == 3 else 1
        r, c = t.shape[-2:]
        m, n = min(r, c), max(r, c)
        tot += b * steps * (4 * m * m * n + 2 * m ** 3)
    return tot


def phase_flops(ts):
    """Algorithmic flops of one launch of each contraction phase (all slices)."""
    g = s = a = 0
    for t in ts:
        b = t.shape[0] if len(t.shape) == 3 else 1
        r, c = t.shape[-2:]
        m, n = min(r, c), max(r, c)
        g += b * 2 * m * m * n
        s += b * 2 * m ** 3
        a += b * 2 * m * m * n
    return {"gram": g, "square": s, "apply": a}


def n_slices(ts):
    return sum(t.shape[0] if len(t.shape) == 3 else 1 for t in ts)


def select_share(wl_name):
    """The stepped tensors of a workload (one owner slot's LPT share for the 32-layer model)."""
    from matrix_optimizer_muon_amd import lpt_assign
    from matrix_optimizer_muon_amd.workloads import workload
    wl = workload(wl_name)
    if wl_name != "llama_d4096":
        return wl, None
    rows = [t.shape[0] for t in wl.tensors]
    cols = [t.shape[1] for t in wl.tensors]
    res = lpt_assign(rows, cols, [1] * len(rows), [t.layer for t in wl.tensors], 8, owner_slot=0)
    return wl, [int(i) for i in res["owner_order"]]


def lpt_summary(wl_name):
    """The LPT partition behind a workload's owner share (None when it is stepped
    whole): slot count, the owner's slot and matrix count, every slot's load in
    elements and the max/mean balance."""
    if wl_name != "llama_d4096":
        return None
    from matrix_optimizer_muon_amd import lpt_assign
    from matrix_optimizer_muon_amd.workloads import workload
    wl = workload(wl_name)
    rows = [t.shape[0] for t in wl.tensors]
    cols = [t.shape[1] for t in wl.tensors]
    res = lpt_assign(rows, cols, [1] * len(rows), [t.layer for t in wl.tensors], 8, owner_slot=0)
    loads = [int(v) for v in res["slot_load"]]
    return {"slots": 8, "owner_slot": 0, "owned_matrices": int(len(res["owner_order"])),
            "slot_loads_elements": loads, "max_over_mean": round(max(loads) * len(loads) / sum(loads), 4)}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()
                    if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def slice_shapes(ts):
    """Distinct (rows, cols, grad dtype) of the stepped 2-D slices, with counts,
    in workload order, each with the first tensor holding it."""
    out = {}
    for t in ts:
        key = (tuple(t.shape[-2:]), t.grad_dtype)
        b = t.shape[0] if len(t.shape) == 3 else 1
        if key not in out:
            out[key] = [t, 0]
        out[key][1] += b
    return [(key, spec, count) for key, (spec, count) in out.items()]


def cpu_baseline(wl, ts, budget_s=25.0, min_s=10.0, max_passes=64, est_rate=4.0e11):
    """fp64 oracle on one 2-D slice of every distinct slice shape, scaled by count.

    Each slice gets one full step (momentum, normalisation, k Newton–Schulz
    iterations, decay + update) of the oracle as it stands.  A slice whose step
    is estimated (at ``est_rate`` flop/s) above its share of ``budget_s`` is
    instead stepped at k = 0 and at k = 1 and its k-step time taken as
    t0 + k·(t1 − t0) (the iterations all cost the same).  Whole-step slices are
    repeated until ``min_s`` of measured time (at most ``max_passes``).  The
    workload's step time is Σ count·t_slice; the value is its slices per second."""
    import numpy as np
    import oracle
    from matrix_optimizer_muon_amd.workloads import HYPER, make_tensor

    k = HYPER["steps"]
    hp = dict(lr=HYPER["lr"], mu=HYPER["mu"], wd=HYPER["wd"], eps=HYPER["eps"], a=HYPER["a"],
              b=HYPER["b"], c=HYPER["c"])
    groups = slice_shapes(ts)
    per_shape = budget_s / len(groups)

    def one(td, steps):
        t1 = time.perf_counter()
        oracle.muon_step(td.grad, td.momentum, td.master, steps=steps, **hp)
        return time.perf_counter() - t1

    parts, est_total, measured = [], 0.0, 0.0
    for (shape, dtype), spec, count in groups:
        td = make_tensor(wl, spec)
        if len(spec.shape) == 3:        # the first slice of a 3-D tensor, as its own 2-D tensor
            td.grad, td.momentum, td.master = (np.ascontiguousarray(a[0]) for a in
                                               (td.grad, td.momentum, td.master))
        f = ns_flops([type(spec)(spec.index, spec.name, shape, dtype)], k)
        if f / est_rate <= per_shape:
            tot, passes = 0.0, 0
            while passes < max_passes and (passes == 0 or tot < min_s / len(groups)):
                tot += one(td, k)
                passes += 1
            t_slice = tot / passes
            measured += tot
            how = f"{shape[0]}x{shape[1]}: full step x{passes}"
        else:
            t0 = one(td, 0)
            t1 = one(td, 1)
            measured += t0 + t1
            t_slice = t0 + k * (t1 - t0)
            how = (f"{shape[0]}x{shape[1]}: step at k=0 ({t0:.2f} s) and k=1 ({t1:.2f} s), "
                   f"extrapolated to k={k}")
        est_total += count * t_slice
        parts.append(f"{how}, {t_slice:.3f} s per slice, x{count} slices")
        del td
    slices = sum(c for _, _, c in groups)
    return {"value": slices / est_total, "unit": "matrices/s", "cores": int(blas_threads()),
            "kind": "oracle",
            "sample": "one 2-D slice of each distinct slice shape of the workload, fp64 numpy oracle; "
                      + "; ".join(parts) + f"; step time = sum over shapes = {est_total:.1f} s; "
                      f"{measured:.1f} s of oracle time measured",
            "seconds_per_step": est_total, "seconds_measured": measured,
            "gflops_fp64": ns_flops(ts, k) / est_total / 1e9}


def adamw_bytes_per_elem(grad_dtype, publish):
    """Algorithmic HBM bytes per element of one AdamW step."""
    return (2 if grad_dtype == "bf16" else 4) + 3 * 8 + (2 if publish else 0)


def cpu_baseline_adamw(wl, budget_elems=1 << 24, min_s=10.0, max_passes=64):
    """fp64 AdamW oracle on whole tensors of the workload up to ~16 Mi elements,
    in passes over them until min_s of measured time (at most max_passes)."""
    import oracle
    from matrix_optimizer_muon_amd.workloads import make_adamw
    threads = blas_threads()
    chosen, n_el = [], 0
    for t in wl.tensors:
        if chosen and n_el + t.shape[0] > budget_elems:
            break
        chosen.append(t)
        n_el += t.shape[0]
    total, passes = 0.0, 0
    while passes < max_passes and (passes == 0 or total < min_s):
        for t in chosen:
            ad = make_adamw(wl, t)
            t1 = time.perf_counter()
            oracle.adamw_step(ad.param, ad.grad, ad.exp_avg, ad.exp_avg_sq, lr=1e-3, beta1=0.9,
                              beta2=0.999, eps=1e-8, wd=0.01, step=10)
            total += time.perf_counter() - t1
        passes += 1
    return {"value": n_el * passes / total, "unit": "elements/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(chosen)} of {len(wl.tensors)} tensors ({n_el} elements), one step each in fp64 "
                      f"numpy, {passes} pass(es), {total:.3f} s", "seconds": total}


def bench_adamw(args):
    import numpy as np
    import torch
    import matrix_optimizer_muon_amd as mm
    from matrix_optimizer_muon_amd.workloads import make_adamw, workload

    name = args.workload if args.workload != DEFAULT_WORKLOAD else ADAMW_DEFAULT_WORKLOAD
    wl = workload(name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    P, G, M, V, PUB = [], [], [], [], []
    for t in wl.tensors:
        ad = make_adamw(wl, t)
        P.append(torch.from_numpy(ad.param).to(dev))
        if ad.grad_bits is not None:
            G.append(torch.from_numpy(ad.grad_bits.view(np.int16)).view(torch.bfloat16).to(dev))
        else:
            G.append(torch.from_numpy(ad.grad).to(dev))
        M.append(torch.from_numpy(ad.exp_avg).to(dev))
        V.append(torch.from_numpy(ad.exp_avg_sq).to(dev))
        PUB.append(torch.empty(t.shape, dtype=torch.int16, device=dev))
    pubs = PUB if args.publish else None
    numel = sum(int(p.numel()) for p in P)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    k = [10]
    prepared = mm.AdamwStep(P, G, M, V, param_outs=pubs, workspace=ws)

    def step():
        prepared(k[0], stream)
        k[0] += 1

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if not args.no_phase_timing:
        mm.phase_timing(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    mm.phase_timing(False)
    phases = mm.phase_timing_read()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    bpe = adamw_bytes_per_elem(wl.tensors[0].grad_dtype, args.publish)
    roof = None
    ms_tot, cnt = phases["adamw"]
    if cnt:
        avg_ms = ms_tot / cnt
        ach = numel * bpe / (avg_ms * 1e-3) / 1e9
        roof = {"kernel": "adamw", "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic("adamw", name), "avg_launch_ms": round(avg_ms, 4),
                "bytes_per_launch": numel * bpe, "bytes_per_element": bpe, "launches": cnt}
    cpu = None if args.no_cpu_baseline else cpu_baseline_adamw(wl)
    line = {
        "metric": ADAMW_METRIC, "value": round(numel / (ms_step * 1e-3), 1), "unit": "elements/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "tensors": len(wl.tensors), "elements": numel,
                   "grad_dtype": wl.tensors[0].grad_dtype, "publish": bool(args.publish)},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--precision", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-phase-timing", action="store_true")
    ap.add_argument("--route", default="muon", choices=["muon", "adamw"])
    ap.add_argument("--publish", action="store_true",
                    help="also write the bf16 published copy of the updated parameters")
    ap.add_argument("--stream-groups", type=int, default=0,
                    help="concurrent stream groups of the value pass (0: the library's choice)")
    ap.add_argument("--graph", action="store_true",
                    help="value pass: capture one prepared step into a HIP graph and time its replays")
    ap.add_argument("--mfma-probe", action="store_true",
                    help="only measure the matrix-core ceiling (probe library), both shapes")
    ap.add_argument("--no-mfma-ceiling", action="store_true",
                    help="skip the 3 s matrix-core ceiling measurement of the main line")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.mfma_probe:
        mfma_probe()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the owner-rank step has no cross-GPU work on its "
              "hot path (each GPU steps its own LPT share); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.route == "adamw":
        bench_adamw(args)
        return

    import numpy as np
    import torch
    import matrix_optimizer_muon_amd as mm
    from matrix_optimizer_muon_amd.workloads import HYPER, make_tensor

    wl, share = select_share(args.workload)
    ts = matrices_of(wl, share)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    grads, moms, masters, pubs = [], [], [], []
    for t in ts:
        td = make_tensor(wl, t)
        if td.grad_bits is not None:
            g = torch.from_numpy(td.grad_bits.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            g = torch.from_numpy(td.grad).to(dev)
        grads.append(g)
        moms.append(torch.from_numpy(td.momentum).to(dev))
        masters.append(torch.from_numpy(td.master).to(dev))
        if args.publish:
            pubs.append(torch.empty(t.shape, dtype=torch.int16, device=dev))
        del td
    stream = torch.cuda.current_stream()

    def prepare(groups):
        return mm.MuonStep(grads, moms, masters, precision=args.precision, stream_groups=groups,
                           param_outs=pubs if args.publish else None, stream=stream)

    def timed(prepared, events):
        for _ in range(args.warmup):
            prepared(stream)
        torch.cuda.synchronize()
        if events:
            mm.phase_timing(True)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            prepared(stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        mm.phase_timing(False)
        return ev0.elapsed_time(ev1) / args.steps, wall, mm.phase_timing_read()

    def graphed(prepared):
        # the step's launches (side streams included) recorded once, replayed
        # as one graph launch per step on the stream
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            prepared()
        torch.cuda.synchronize()
        return lambda st: graph.replay()

    # pass 1: throughput in the library's launch configuration
    first = prepare(args.stream_groups)
    groups_used = first.groups
    ms_step, wall, _ = timed(graphed(first) if args.graph else first, False)
    del first
    slices = n_slices(ts)
    flops = ns_flops(ts, HYPER["steps"])
    tflops = flops / (ms_step * 1e-3) / 1e12

    # pass 2: every launch alone on one stream, timed with HIP events on it
    roof, phases, ms_alone = None, {}, None
    pf = phase_flops(ts)
    if not args.no_phase_timing:
        ms_alone, _, phases = timed(prepare(1), True)
        dom = max(("gram", "square", "apply"), key=lambda p: phases[p][0])
        ms_tot, cnt = phases[dom]
        if cnt:
            total_flops = pf[dom] * HYPER["steps"] * args.steps
            avg_ms = ms_tot / cnt
            ach = total_flops / (ms_tot * 1e-3) / 1e12
            roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                    "traffic": measured_traffic(dom, args.workload),
                    "avg_launch_ms": round(avg_ms, 4), "flops_per_launch": round(total_flops / cnt),
                    "launches": cnt,
                    "timing": "HIP events around each launch on its stream, one stream group, "
                              f"{args.steps} timed steps ({ms_alone:.4f} ms per step)"}

    elementwise = None
    if phases and phases.get("ingest", (0.0, 0))[1]:
        ms_i, cnt_i = phases["ingest"]
        elems = sum(int(np.prod(t.shape)) for t in ts)
        alg, moved = ingest_bytes_per_elem(ts[0].grad_dtype, args.precision)
        avg_i = ms_i / cnt_i
        ach = elems * alg / (avg_i * 1e-3) / 1e9
        ceil = copy_ceiling_gbs()
        elementwise = {"kernel": "ingest", "bound": "hbm", "avg_launch_ms": round(avg_i, 4),
                       "elements": elems, "bytes_per_elem": alg, "bytes_per_elem_moved": moved,
                       "achieved": round(ach, 1), "achieved_moved": round(elems * moved / (avg_i * 1e-3) / 1e9, 1),
                       "unit": "GB/s", "peak": PEAK_HBM_GBS, "frac": round(ach / PEAK_HBM_GBS, 4),
                       "copy_ceiling": round(ceil, 1), "frac_of_copy": round(ach / ceil, 4),
                       "target_frac": 0.8,
                       "note": "the decay + update runs inside the last apply launch (no separate kernel)"}

    # the matrix cores alone on the dominant kernel's instruction (the bf16 path
    # runs v_mfma_f32_16x16x32_bf16), under the same power limit: the practical
    # ceiling of a bf16 contraction on random operands
    ceiling = None
    if roof and args.precision == "bf16" and not args.no_mfma_ceiling:
        ceiling = mfma_ceiling(16, 0)
        roof["frac_of_mfma_ceiling"] = round(roof["achieved"] / ceiling["tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, ts)

    props = torch.cuda.get_device_properties(dev)
    shapes = {}
    for t in ts:
        shapes[str(tuple(t.shape))] = shapes.get(str(tuple(t.shape)), 0) + 1
    line = {
        "metric": METRIC,
        "value": round(slices / (ms_step * 1e-3), 3),
        "unit": "matrices/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": args.precision, "data": "synthetic",
        "tflops_effective": round(tflops, 2),
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": args.workload, "matrices": slices, "shapes": shapes,
                   "stream_groups": groups_used, "graph": bool(args.graph),
                   "ns_steps": HYPER["steps"], "grad_dtype": ts[0].grad_dtype,
                   "effective_gflop_per_step": round(flops / 1e9, 1), "publish": bool(args.publish),
                   "lpt": lpt_summary(args.workload)},
        "roofline": roof,
        "counters": measured_mfma_busy(args.workload),
        "cpu_baseline": cpu,
        "elementwise": elementwise,
        "mfma_ceiling": ceiling,
        "phases_ms_per_step": {k: round(v[0] / args.steps, 4) for k, v in phases.items() if v[1]},
        # one-stream pass: Newton–Schulz contractions alone, element-wise kernels alone
        "ns_ms_per_step": round(sum(phases[p][0] for p in ("gram", "square", "apply") if p in phases)
                                / args.steps, 4) if phases else None,
        "elementwise_ms_per_step": round(sum(phases[p][0] for p in ("ingest", "norm", "update")
                                             if p in phases) / args.steps, 4) if phases else None,
        "ms_per_step_one_stream": None if ms_alone is None else round(ms_alone, 4),
        "wall_s_timed": round(wall, 3),
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "peak_clock_mhz": peak_clock_mhz(dev.index)},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
