#!/usr/bin/env python3
"""Throughput of the DP-GRAPE private update step on one MI355X.

A step is one pass of the whole path over one batch, one dpg_private_step
call over every layer of the workload: P generation, projection, per-sample
norms, clip, batch sum, noise, projected Adam and the back-projection into W.
Inputs (A, dY) are synthetic, seeded, and resident in HBM before timing
starts; W, m and v evolve in place and the step counter (which keys P and the
noise) advances every step.

Prints one JSON line: samples/s over the timed steps, the roofline position
of the dominant kernel (per-kernel times from HIP events recorded on the
library's stream over a second pass of the same steps), the CPU oracle's
rate on the host cores, and beside them the rates of the same step as two
calls (dpg_project_clip_noise then dpg_adam_backproject) and in its
streaming form (dpg_project_layer per layer, then dpg_clip_sum_noise and the
update).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dec24]

The default workload is dec24 (24 decoder blocks of q, k, v, o 2048 x 2048
and MLP 2048 <-> 8192, B = 16, T = 512, r = 512, bf16), the largest one; the
others (tiny, mlp4, enc12, long1) are available with --workload.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 matrix cores
FP32_MFMA_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dec24")
    ap.add_argument("--timing-steps", type=int, default=20,
                    help="steps of the per-kernel event pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=2,
                    help="least number of oracle runs")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="oracle runs continue until this much time has passed")
    ap.add_argument("--no-streaming", action="store_true",
                    help="skip timing the two-call and streaming forms of "
                         "the step")
    ap.add_argument("--device-inputs", action="store_true",
                    help="draw A, dY, W on the GPU (workloads.device_layer_inputs); "
                         "the default for enc12, dec24 and long1, whose host "
                         "draws would take minutes. The CPU oracle then runs on "
                         "one block at two batch sizes and is extrapolated.")
    ap.add_argument("--rc-k", type=int, default=32,
                    help="probes per layer of the randomized-clipping norm "
                         "estimate timed beside the step (0: skip it)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="after the steps, copy a buffer of this many MiB "
                         "three times (calibrates HBM byte counters)")
    return ap.parse_args()


def traffic_summary(workload):
    return os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")


def kernel_source_digest():
    """sha256 over the library's kernel and launch sources (the counters in
    the traffic summary hold only for the sources they were taken on)."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dp_grape_projection_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) +
                    glob.glob(os.path.join(csrc, "*.hpp"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy calibration), or None when
    there is none for this workload or the kernels changed since."""
    try:
        with open(traffic_summary(workload)) as fh:
            text = fh.read()
        block = text.split("```json", 1)[1].split("```", 1)[0]
        data = json.loads(block)
    except (OSError, IndexError, ValueError):
        return None
    if data.get("workload") != workload or data.get("source_sha256") != kernel_source_digest():
        return None
    k = data.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def kernel_work(wl):
    """Algorithmic bytes and flops of each kernel kind for one step of `wl`
    (the one-call step: P generated once, the moments updated in the pass
    that forms G_priv).

    Bytes count each input the kernel must read once and each output it must
    write once (es = bytes per A/dY element); flops count the multiply-adds of
    its matrix-core contraction (2 per MAC). xsum only exists to sum split
    partials, so it has no algorithmic work of its own."""
    es = 2 if wl.dtype == "bf16" else 4
    B, T, r = wl.B, wl.T, wl.r
    w = {k: [0.0, 0.0] for k in ("gen_p", "proj", "xsum", "norm", "scale",
                                 "sum", "fin", "prep", "back")}
    for L in wl.layers:
        di, do = L.d_in, L.d_out
        w["gen_p"][0] += r * di * es
        w["proj"][0] += B * T * di * es + r * di * es + B * T * r * es
        w["proj"][1] += 2.0 * B * T * di * r
        w["norm"][0] += B * T * do * es + B * T * r * es
        w["norm"][1] += 2.0 * B * T * r * do
        w["sum"][0] += B * T * do * es + B * T * r * es
        w["sum"][1] += 2.0 * B * T * r * do
        # sum partial in; G_priv, m, v out; m, v in; U out in the operand type
        w["fin"][0] += r * do * (6 * 4 + es)
        w["back"][0] += 8 * di * do + (di + do) * r * es
        w["back"][1] += 2.0 * di * r * do
    w["scale"][0] += B * 4
    return w


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def _time_oracle_step(wl, orc, state, reps, seconds):
    """Wall times of the unchanged float64 oracle on one full step of the
    layers in `orc` (projection, norms, clip, sum, noise, Adam and the
    back-projection): at least `reps` runs, more until `seconds` passed."""
    import oracle
    times = []
    while len(times) < reps or (sum(times) < seconds and len(times) < 200):
        t0 = time.perf_counter()
        res = oracle.project_clip_noise(orc, wl.r, wl.clip_C, wl.sigma,
                                        wl.seed, wl.step, wl.proj_step)
        params = [{"W": st[0], "m": st[1], "v": st[2], "G_priv": g,
                   "layer_id": o["layer_id"]}
                  for st, g, o in zip(state, res["G_priv"], orc)]
        oracle.adam_backproject(params, wl.r, wl.lr, wl.beta1, wl.beta2,
                                wl.eps, wl.seed, wl.step, wl.proj_step)
        times.append(time.perf_counter() - t0)
    return times


def cpu_baseline_blocks(wl, A, dY, Wd, reps, seconds):
    """The float64 oracle on a bounded sample of a block-structured workload
    whose inputs live in device memory: the first block (6 layers) at B = 1
    and at B = 4, with the workload's T, r, shapes and values (host copies of
    the device draws). Every block has the same shapes, and the oracle's
    work splits into a per-step part (P, noise, Adam, back-projection) and a
    per-sample part (the materialised per-sample gradients and their
    projections), so the full step takes n_blocks x (t_fixed + B t_sample),
    with t_sample = (t(4) - t(1)) / 3 and t_fixed = t(1) - t_sample."""
    import numpy as np
    per = 6
    n_blk = len(wl.layers) // per
    sub = list(range(per))

    def host(t, b):
        return t[:b].float().cpu().numpy().astype(np.float64)

    state = [(Wd[l].cpu().numpy().astype(np.float64),
              np.zeros((wl.r, wl.layers[l].d_out)),
              np.zeros((wl.r, wl.layers[l].d_out))) for l in sub]
    med = {}
    runs = {}
    for b in (1, 4):
        orc = [{"A": host(A[l], b), "dY": host(dY[l], b),
                "layer_id": wl.layers[l].layer_id} for l in sub]
        t = _time_oracle_step(wl, orc, state, reps, seconds / 2)
        med[b] = statistics.median(t)
        runs[b] = len(t)
    t_sample = max(med[4] - med[1], 0.0) / 3.0
    t_fixed = med[1] - t_sample
    t_step = n_blk * (t_fixed + wl.B * t_sample)
    return {"value": round(wl.B / t_step, 5), "unit": "samples/s",
            "cores": int(_oracle_threads()), "kind": "oracle",
            "sample": f"float64 numpy oracle, full step of block 0 of {n_blk} "
                      f"({per} layers, T={wl.T}, r={wl.r}) at B=1 (median of "
                      f"{runs[1]} runs: {med[1]:.2f} s) and B=4 (median of "
                      f"{runs[4]} runs: {med[4]:.2f} s); extrapolated to the "
                      f"{len(wl.layers)}-layer step at B={wl.B} as {n_blk} x "
                      f"({t_fixed:.2f} s + {wl.B} x {t_sample:.3f} s) = "
                      f"{t_step:.1f} s"}


def cpu_baseline(wl, host, state, reps, seconds):
    """The float64 oracle on the full step of the same workload: at least
    `reps` runs, and more until `seconds` have passed (at most 200 runs)."""
    import workloads as W
    orc = [{"A": W.as_float64(wl, a), "dY": W.as_float64(wl, d),
            "layer_id": L.layer_id} for (a, d), L in zip(host, wl.layers)]
    times = _time_oracle_step(wl, orc, state, reps, seconds)
    t = statistics.median(times)
    return {"value": round(wl.B / t, 3), "unit": "samples/s",
            "cores": int(_oracle_threads()), "kind": "oracle",
            "sample": f"full step of {wl.name} ({wl.B} samples, "
                      f"{len(wl.layers)} layers), float64 numpy, median of "
                      f"{len(times)} runs ({sum(times):.1f} s in all; "
                      f"{min(times):.2f} to {max(times):.2f} s each)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs the DP-GRAPE step on one GPU; --gpus {args.gpus} "
              "is not supported (the library has no multi-GPU path).",
              file=sys.stderr)
        sys.exit(2)
    for k in ("RANK", "WORLD_SIZE"):
        if os.environ.get(k) not in (None, "0", "1") and k == "WORLD_SIZE":
            print("bench.py is single-GPU only", file=sys.stderr)
            sys.exit(2)

    import numpy as np
    import torch

    import dp_grape_projection_amd as dpg
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dpg.load_library()
    wl = W.workload(args.workload)
    dev = torch.device("cuda:0")

    t_gen = time.perf_counter()
    device_inputs = args.device_inputs or wl.name in ("enc12", "dec24", "long1")
    host = state = None
    if device_inputs:
        A, dY, Wd, md, vd = [], [], [], [], []
        for L in wl.layers:
            a, d = W.device_layer_inputs(wl, L, dev)
            w, m, v = W.device_initial_state(wl, L, dev)
            A.append(a)
            dY.append(d)
            Wd.append(w)
            md.append(m)
            vd.append(v)
    else:
        host = [W.layer_inputs(wl, L) for L in wl.layers]
        state = [W.initial_state(wl, L) for L in wl.layers]

        def to_dev(x):
            if wl.dtype == "bf16":
                return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(x).to(dev)

        A = [to_dev(a) for a, _ in host]
        dY = [to_dev(d) for _, d in host]
        Wd = [torch.from_numpy(s[0].copy()).to(dev) for s in state]
        md = [torch.zeros_like(torch.from_numpy(s[1])).to(dev) for s in state]
        vd = [torch.zeros_like(torch.from_numpy(s[2])).to(dev) for s in state]
    prep = dpg.PreparedStep(A, dY, Wd, md, vd, wl.r, wl.clip_C, wl.sigma,
                            wl.seed, wl.lr, wl.beta1, wl.beta2, wl.eps,
                            layer_ids=[L.layer_id for L in wl.layers])
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: inputs ready in {time.perf_counter() - t_gen:.1f} s",
          file=sys.stderr, flush=True)

    step = 0
    for _ in range(args.warmup):
        step += 1
        prep.run(step)
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step += 1
        prep.run(step)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall * 1e3 / args.steps
    value = wl.B * args.steps / wall
    print(f"[bench] timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step "
          f"(events {ev_ms * 1e3 / args.steps:.1f} us/step)", file=sys.stderr,
          flush=True)

    # Per-kernel times: events around each launch on the library's stream.
    times = {}
    if args.timing_steps > 0:
        dpg.timing_read(reset=True)
        dpg.timing_enable(True)
        for _ in range(args.timing_steps):
            step += 1
            prep.run(step)
        torch.cuda.synchronize()
        times = dpg.timing_read(reset=True)
        dpg.timing_enable(False)
    work = kernel_work(wl)
    peak_flops = BF16_MFMA_PEAK_TFLOPS if wl.dtype == "bf16" else FP32_MFMA_PEAK_TFLOPS
    # the matrix cores bound a kernel whose algorithmic flops per algorithmic
    # byte exceed the machine balance (2500 / 8 = 312.5 flop/byte in bf16)
    ridge = peak_flops * 1e12 / (HBM_PEAK_GBS * 1e9)
    kernels = {}
    for name, (ms, n) in times.items():
        if n == 0:
            continue
        per_step_launches = n / args.timing_steps
        avg_us = ms * 1e3 / n
        byt, flo = work[name]
        # a launch's algorithmic work: one step's work over that step's
        # launches (the average launch)
        byt_l, flo_l = byt / per_step_launches, flo / per_step_launches
        gbs = byt_l / (avg_us * 1e-6) / 1e9
        tfs = flo_l / (avg_us * 1e-6) / 1e12
        mfma = byt > 0 and flo / byt > ridge
        kernels[name] = {
            "avg_us": round(avg_us, 2), "launches_per_step": per_step_launches,
            "us_per_step": round(avg_us * per_step_launches, 2),
            "GB/s": round(gbs, 1), "TFLOP/s": round(tfs, 2),
            "flop_per_byte": round(flo / byt, 1) if byt > 0 else None,
            "bound": "mfma" if mfma else "hbm",
            "frac": round(tfs / peak_flops if mfma else gbs / HBM_PEAK_GBS, 4)}
    roof = None
    if kernels:
        dom = max(kernels, key=lambda k: kernels[k]["us_per_step"])
        dk = kernels[dom]
        byt, flo = work[dom]
        launches = dk["launches_per_step"]
        if dk["bound"] == "mfma":
            roof = {"kernel": dom, "bound": "mfma", "achieved": dk["TFLOP/s"],
                    "peak": peak_flops, "unit": "TFLOP/s", "frac": dk["frac"]}
        else:
            roof = {"kernel": dom, "bound": "hbm", "achieved": dk["GB/s"],
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": dk["frac"]}
        roof.update({
            "traffic": measured_traffic(dom, wl.name),
            "algorithmic_bytes_per_launch": int(byt / launches),
            "algorithmic_flops_per_launch": float(flo / launches),
            "avg_launch_us": dk["avg_us"], "launches_per_step": launches,
            "hbm_GB/s": dk["GB/s"], "ridge_flop_per_byte": round(ridge, 1)})

    # The whole step against its algorithmic HBM bytes at the HBM peak.
    step_bytes = sum(b for b, _ in work.values())
    step_roof = {"algorithmic_bytes": int(step_bytes),
                 "t_lb_us": round(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
                 "frac": round(step_bytes / (HBM_PEAK_GBS * 1e9) / (ms_per_step * 1e-3), 4)}

    # The same step as two calls, and in the streaming form (each layer
    # projected on its own, projections stored, then clip/sum/noise and the
    # update), on the same inputs; reported beside the main figure.
    streaming = two_call = None
    if not args.no_streaming:
        tprep = dpg.PreparedStep(A, dY, Wd, md, vd, wl.r, wl.clip_C, wl.sigma,
                                 wl.seed, wl.lr, wl.beta1, wl.beta2, wl.eps,
                                 layer_ids=[L.layer_id for L in wl.layers],
                                 one_call=False)
        for _ in range(args.warmup):
            step += 1
            tprep.run(step)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step += 1
            tprep.run(step)
        torch.cuda.synchronize()
        twall = time.perf_counter() - t0
        two_call = {"value": round(wl.B * args.steps / twall, 1), "unit": "samples/s",
                    "ms_per_step": round(twall * 1e3 / args.steps, 5)}
        print(f"[bench] two-call form: {twall * 1e6 / args.steps:.1f} us/step",
              file=sys.stderr, flush=True)
        del tprep

        sprep = dpg.PreparedStreamingStep(A, dY, Wd, md, vd, wl.r, wl.clip_C,
                                          wl.sigma, wl.seed, wl.lr, wl.beta1,
                                          wl.beta2, wl.eps,
                                          layer_ids=[L.layer_id for L in wl.layers])
        for _ in range(args.warmup):
            step += 1
            sprep.run(step)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step += 1
            sprep.run(step)
        torch.cuda.synchronize()
        swall = time.perf_counter() - t0
        hat_bytes = sum(wl.B * wl.r * L.d_out * 4 for L in wl.layers)
        streaming = {"value": round(wl.B * args.steps / swall, 1), "unit": "samples/s",
                     "ms_per_step": round(swall * 1e3 / args.steps, 5),
                     "stored_projection_bytes": hat_bytes}
        print(f"[bench] streaming form: {swall * 1e6 / args.steps:.1f} us/step",
              file=sys.stderr, flush=True)
        del sprep

    # Randomized clipping's per-sample norm estimate (dpg_rc_norms) on the
    # same inputs: k probes per layer; its algorithmic bytes are A and dY
    # read once each plus the probes, its flops 2 B T k (d_in + d_out).
    rc = None
    if args.rc_k > 0:
        ids = [L.layer_id for L in wl.layers]
        es = 2 if wl.dtype == "bf16" else 4
        for _ in range(3):
            step += 1
            dpg.dpg_rc_norms(A, dY, k=args.rc_k, clip_C=wl.clip_C, seed=wl.seed, step=step,
                             layer_ids=ids)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            step += 1
            dpg.dpg_rc_norms(A, dY, k=args.rc_k, clip_C=wl.clip_C, seed=wl.seed, step=step,
                             layer_ids=ids)
        e1.record()
        torch.cuda.synchronize()
        rc_ms = e0.elapsed_time(e1) / args.steps
        dpg.timing_read(reset=True)
        dpg.timing_enable(True)
        for _ in range(3):
            step += 1
            dpg.dpg_rc_norms(A, dY, k=args.rc_k, clip_C=wl.clip_C, seed=wl.seed, step=step,
                             layer_ids=ids)
        torch.cuda.synchronize()
        rc_times = dpg.timing_read(reset=True)
        dpg.timing_enable(False)
        rc_bytes = sum(wl.B * wl.T * (L.d_in + L.d_out) * es + args.rc_k * L.d_out * es
                       for L in wl.layers)
        rc_flops = sum(2.0 * wl.B * wl.T * args.rc_k * (L.d_in + L.d_out) for L in wl.layers)
        rc = {"k": args.rc_k, "ms_per_call": round(rc_ms, 5),
              "samples_per_s": round(wl.B / (rc_ms * 1e-3), 1),
              "algorithmic_bytes": int(rc_bytes), "algorithmic_flops": rc_flops,
              "hbm_GB/s": round(rc_bytes / (rc_ms * 1e-3) / 1e9, 1),
              "bound": "hbm", "frac": round(rc_bytes / (rc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
              "kernels_us_per_call": {k: round(ms * 1e3 / 3, 2)
                                      for k, (ms, n) in rc_times.items() if n > 0}}
        print(f"[bench] rc_norms (k={args.rc_k}): {rc_ms * 1e3:.1f} us/call",
              file=sys.stderr, flush=True)

    if args.copy_mb > 0:
        n = args.copy_mb * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Context for the HBM fractions: the rate of the runtime's own
    # device-to-device copy (half reads, half writes, as in the update
    # kernels' read-modify-write streams), bytes read plus written. Not in
    # counter runs (--copy-mb), whose calibration takes the last copies.
    hbm_copy = None
    if args.copy_mb == 0:
        n = 512 * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        copy_gbs = 2 * 4 * n * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
        hbm_copy = {"GB/s": round(copy_gbs, 1), "frac": round(copy_gbs / HBM_PEAK_GBS, 4),
                    "what": "device-to-device copy of 512 MiB, bytes read plus written"}
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        if host is not None:
            cpu = cpu_baseline(wl, host, state, args.cpu_reps, args.cpu_seconds)
        elif len(wl.layers) % 6 == 0:
            cpu = cpu_baseline_blocks(wl, A, dY, Wd, args.cpu_reps, args.cpu_seconds)

    layers = "->".join([str(wl.layers[0].d_in)] + [str(L.d_out) for L in wl.layers]) \
        if all(a.d_out == b.d_in for a, b in zip(wl.layers, wl.layers[1:])) \
        else f"{len(wl.layers)} layers"
    out = {
        "metric": "DP-GRAPE step samples/sec at 1 GPU; MFMA % of bf16 peak, HBM GB/s",
        "value": round(value, 1), "unit": "samples/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic, seeded: A Gaussian, dY %s, W Gaussian%s" % (
            "Student-t(3)" if wl.dy_kind.startswith("t3") else "Gaussian",
            ", drawn on the GPU" if device_inputs else ""),
        "config": {"workload": wl.name, "layers": layers, "B": wl.B,
                   "T": wl.T, "r": wl.r, "clip_C": wl.clip_C,
                   "sigma": wl.sigma, "parallelism": "single GPU"},
        "roofline": roof,
        "step_roofline": step_roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "two_call": two_call,
        "streaming": streaming,
        "rc_norms": rc,
        "hbm_copy": hbm_copy,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
