#!/usr/bin/env python3
"""Benchmark of the LittleBit layer forward on one MI355X.

One step is one forward pass of the token batch through a stack of seeded
synthetic LittleBit linears: by default the Llama2-70B-shaped decoder-layer
linears (q/o 8192x8192, k/v 8192x1024, gate/up 8192x28672, down 28672x8192) at
0.1 bits per weight with the residual path, 80 independent layers, decode T=1,
run as one group (two kernel launches per pass).  The stack holds ~0.8 GB of
packed signs, more than three times the 256 MB Infinity Cache, so every pass
streams from HBM.  Prints ONE JSON line.

The prefill leg times the same shapes at T=2048 (one layer, the GEMM path)
and reports it beside the decode figure.  The CPU baseline times the fp64
oracle on one layer of the same stack and scales to the stack.

    python bench.py [--steps K] [--warmup W] [--workload c5] [--tokens 1]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
METRIC = "LittleBit layer tok/s at T=1 and T=2048; % HBM BW / % MFMA peak"
# a decode group at T <= 8 (bf16 out) runs one launch per pass: k_pass holds
# stage 1, the latents and stage 2 of every linear
PASS_KERNEL = "k_pass"


def _log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def linear_bytes(d_in, d_out, r, P, T, act_bytes=2):
    """Algorithmic bytes of one linear forward, split by stage: tight sign
    bits, fp16 scales, activations in and out (padding excluded)."""
    r_p = r // P
    s1 = r * d_in // 8 + 2 * P * (d_in + r_p) + T * d_in * act_bytes
    s2 = r * d_out // 8 + 2 * P * d_out + T * d_out * act_bytes
    return s1, s2


def build_stack(w, layers, T):
    import torch
    import synth
    from binarized_rank_linear_amd.stack import LayerStack

    def make(L, i, di, do, rp, P):
        return synth.device_layer(synth.layer_seed(L, i), di, do, rp, P)

    t0 = time.time()
    st = LayerStack([(s.name, s.d_in, s.d_out) for s in w.linears], layers, w.b_num, w.b_den,
                    w.residual, make)
    widths = sorted({s.d_in for s in w.linears})
    xs = {d: synth.device_activations(synth.activation_seed(d), T, d, w.dtype) for d in widths}
    st.bind(T, xs, torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    torch.cuda.synchronize()
    _log("stack of %d layers packed in %.1f s (%.1f MB of packed words)"
         % (layers, time.time() - t0, st.packed_bytes() / 1e6))
    return st, xs


def time_decode(st, steps, warmup, settle_s):
    """Runs `warmup` untimed passes, then more untimed passes until `settle_s`
    seconds have gone by (the GPU clocks take some tens of milliseconds to
    leave their idle state; a decode service runs in the steady state), then
    the timed region: `steps` passes (one k_pass launch each) on the launch
    stream between two HIP events, synchronised on both sides (an event after
    every launch would put a marker packet between the passes: about 2.5 us
    more per pass).  Returns (seconds per pass by the host clock, mean
    seconds per launch by the events)."""
    import torch
    s = torch.cuda.current_stream()
    g = st.group
    for _ in range(warmup):
        g.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(20):
            g.run()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        g.run()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = e0.elapsed_time(e1) / steps * 1e-3
    return wall / steps, kern


def time_staged(st, steps):
    """The same pass as three launches per stage pair (stage 1 = k_stage1f +
    k_latent, stage 2 = k_stage2r), HIP events around each stage: a
    diagnostic of where the time goes.  Returns mean (stage-1, stage-2)
    seconds."""
    import torch
    s = torch.cuda.current_stream()
    g = st.group
    for _ in range(5):
        g.run_stage(1)
        g.run_stage(2)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    for k in range(steps):
        ev[k][0].record(s)
        g.run_stage(1)
        ev[k][1].record(s)
        g.run_stage(2)
        ev[k][2].record(s)
    torch.cuda.synchronize()
    s1 = sum(e[0].elapsed_time(e[1]) for e in ev) / steps * 1e-3
    s2 = sum(e[1].elapsed_time(e[2]) for e in ev) / steps * 1e-3
    return s1, s2


def cpu_baseline(w, T, layers, budget_s=10.0):
    """The fp64 oracle on one layer of the stack (all its linears, seeded
    inputs of the same shapes), run repeatedly until about budget_s seconds of
    CPU time, scaled to the L-layer stack (the layers cost the same)."""
    import oracle
    import synth
    inputs = []
    for i, sh in enumerate(w.linears):
        r, rp = oracle.rank_for_budget(sh.d_in, sh.d_out, w.b_num, w.b_den, w.residual)
        inp = synth.layer_inputs(i, sh.d_in, sh.d_out, rp, 2 if w.residual else 1)
        x = synth.activations(synth.activation_seed(T), T, sh.d_in, w.dtype)
        inputs.append((x, inp))
    passes, t_total = 0, 0.0
    while t_total < budget_s and passes < 1000:
        t0 = time.perf_counter()
        for x, inp in inputs:
            oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l)
        t_total += time.perf_counter() - t0
        passes += 1
    t_layer = t_total / passes
    cores = oracle.max_threads()
    return {"value": T / (t_layer * layers), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": "one layer (%d linears, seeded inputs) at T=%d, %d passes in %.1f s, scaled "
                      "to the %d-layer stack" % (len(w.linears), T, passes, t_total, layers)}


def measured_traffic(kernel, workload, T):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is
    none or the kernel source changed since the counters were taken."""
    f = os.path.join(ROOT, "profiles", "traffic_%s_%s_T%d.txt" % (kernel, workload, T))
    if not os.path.exists(f):
        return None
    kv = {}
    for line in open(f):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    src = os.path.join(ROOT, "binarized_rank_linear_amd", "csrc", kv.get("source", ""))
    if not os.path.exists(src):
        return None
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != kv.get("source_sha256"):
        return None
    return float(kv["traffic_bytes_per_launch"])


def calibrate_copy(mib, reps):
    """A plain device-to-device copy of `mib` MiB, `reps` times: the reference
    kernel whose FETCH_SIZE / WRITE_SIZE calibrate the traffic counters."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "reps": reps}), flush=True)


def single_layer_leg(w, T, reps=2000):
    """One layer of the workload's linears (a few MB of packed signs: it stays
    in the 256 MB Infinity Cache across passes) as one decode group at T
    tokens: the cache-resident figure, reported beside the spilled stack's.
    HIP events bracket `reps` back-to-back passes after a settle period."""
    import torch
    P = 2 if w.residual else 1
    st, _ = build_stack(w, 1, T)
    g = st.group
    s = torch.cuda.current_stream()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.2:
        for _ in range(50):
            g.run()
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        g.run()
    e1.record(s)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    nbytes = sum(sum(linear_bytes(lin.d_in, lin.d_out, lin.r, P, T)) for lin in st.linears[0])
    return {"workload": "%s, one layer (%d linears) as one group, decode T=%d, cache-resident"
                        % (w.title, len(st.linears[0]), T),
            "us_per_layer": t * 1e6, "tok_per_s": T / t, "algorithmic_bytes": nbytes,
            "effective_GBs": nbytes / t / 1e9,
            "note": "the layer's %.1f MB stay in the Infinity Cache, so this can exceed the HBM peak"
                    % (nbytes / 1e6)}


def library_gemm_reference(layer, xs, T, steps):
    """A reference point for the prefill roofline fraction, not part of the
    path: torch.nn.functional.linear in bf16 (the vendor GEMM library) on the
    prefill shapes of the layer with dense random weights (no signs, no
    scales): stage 1 = x [T][d_in] times a [r][d_in] weight, stage 2 =
    t [T][r] times a [d_out][r] weight, for every linear.  HIP events bracket
    `steps` repetitions of each stage."""
    import torch
    F = torch.nn.functional
    w1 = [torch.randn((lin.r, lin.d_in), device="cuda", dtype=torch.bfloat16) for lin in layer]
    w2 = [torch.randn((lin.d_out, lin.r), device="cuda", dtype=torch.bfloat16) for lin in layer]
    ts = [torch.randn((T, lin.r), device="cuda", dtype=torch.bfloat16) for lin in layer]
    stages = [lambda: [F.linear(xs[lin.d_in], w1[i]) for i, lin in enumerate(layer)],
              lambda: [F.linear(ts[i], w2[i]) for i in range(len(layer))]]
    s = torch.cuda.current_stream()
    out = []
    for run in stages:
        for _ in range(3):
            run()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(steps):
            run()
        e1.record(s)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps * 1e-3)
    f = sum(2 * T * lin.r * (lin.d_in + lin.d_out) for lin in layer)
    t = out[0] + out[1]
    return {"what": "torch bf16 F.linear (vendor GEMM library) on the same shapes, dense weights",
            "stage1_us": out[0] * 1e6, "stage2_us": out[1] * 1e6, "ms_per_layer": t * 1e3,
            "TFLOPs": f / t / 1e12, "frac": f / t / 1e12 / BF16_PEAK_TFLOPS}


def prefill_per_linear(layer, xs, T, steps, P):
    """Each linear of the prefill layer as a group of its own (both stages,
    HIP events around `steps` runs), against its own roofline: the larger of
    its flops at the bf16 MFMA peak and its bytes at the HBM peak (signs,
    scales, x, y and the bf16 t round trip between the stages)."""
    import torch
    import binarized_rank_linear_amd as lb
    s = torch.cuda.current_stream()
    out = []
    for i, lin in enumerate(layer):
        y = torch.empty((T, lin.d_out), dtype=torch.bfloat16, device="cuda")
        g = lb.Group([(xs[lin.d_in], y, lin)], T, torch.bfloat16, torch.bfloat16)
        for _ in range(2):
            g.run()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(steps):
            g.run()
        e1.record(s)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / steps * 1e-3
        g.release()
        flops = 2 * T * lin.r * (lin.d_in + lin.d_out)
        s1, s2 = linear_bytes(lin.d_in, lin.d_out, lin.r, P, T)
        nbytes = s1 + s2 + 2 * T * lin.r * 2
        t_mfma = flops / (BF16_PEAK_TFLOPS * 1e12)
        t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
        out.append({"linear": "%dx%d r=%d" % (lin.d_in, lin.d_out, lin.r), "us": t * 1e6,
                    "TFLOPs": flops / t / 1e12, "bound": "mfma" if t_mfma >= t_hbm else "hbm",
                    "roofline_us": max(t_mfma, t_hbm) * 1e6, "frac": max(t_mfma, t_hbm) / t})
    return out


def prefill_leg(w, T, steps):
    """One layer of the workload's linears at T tokens as one GEMM-path group:
    stage 1 (and the d_in-piece reduce) for all linears in one launch, then
    stage 2 in one launch; HIP events bracket each on the launch stream."""
    import torch
    import synth
    import binarized_rank_linear_amd as lb
    layer = []
    for i, sh in enumerate(w.linears):
        r, rp = lb.rank_for_budget(sh.d_in, sh.d_out, w.b_num, w.b_den, w.residual)
        U, V, h, g, l = synth.device_layer(synth.layer_seed(0, i), sh.d_in, sh.d_out, rp,
                                           2 if w.residual else 1)
        layer.append(lb.PackedLinear.from_factors(U, V, h, g, l))
        del U, V
    xs = {d: synth.device_activations(synth.activation_seed(d), T, d, "bf16")
          for d in {s.d_in for s in w.linears}}
    ys = [torch.empty((T, lin.d_out), dtype=torch.bfloat16, device="cuda") for lin in layer]
    grp = lb.Group([(xs[lin.d_in], y, lin) for lin, y in zip(layer, ys)], T, torch.bfloat16,
                   torch.bfloat16)
    s = torch.cuda.current_stream()
    for _ in range(2):
        grp.run_stage(1)
        grp.run_stage(2)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record(s)
        grp.run_stage(1)
        ev[k][1].record(s)
        grp.run_stage(2)
        ev[k][2].record(s)
    torch.cuda.synchronize()
    t1 = sum(e[0].elapsed_time(e[1]) for e in ev) / steps * 1e-3
    t2 = sum(e[1].elapsed_time(e[2]) for e in ev) / steps * 1e-3
    t = t1 + t2
    f1 = sum(2 * T * lin.r * lin.d_in for lin in layer)
    f2 = sum(2 * T * lin.r * lin.d_out for lin in layer)
    flops = f1 + f2
    return {"workload": "%s, one layer (%d linears) as one group, T=%d (GEMM path)"
                        % (w.title, len(layer), T), "T": T,
            "tok_per_s": T / t, "ms_per_layer": t * 1e3,
            "stage1_us": t1 * 1e6, "stage2_us": t2 * 1e6,
            "stage1_TFLOPs": f1 / t1 / 1e12, "stage2_TFLOPs": f2 / t2 / 1e12,
            "roofline": {"bound": "mfma", "achieved": flops / t / 1e12, "peak": BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": flops / t / 1e12 / BF16_PEAK_TFLOPS},
            "library_bf16_gemm": library_gemm_reference(layer, xs, T, steps),
            "per_linear": prefill_per_linear(layer, xs, T, steps, 2 if w.residual else 1)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed passes after the warmup (clocks leave idle); 0 under a profiler")
    ap.add_argument("--workload", default="c5", choices=["c3", "c4", "c5"])
    ap.add_argument("--tokens", type=int, default=1)
    ap.add_argument("--layers", type=int, default=0, help="stack depth (default: the workload's)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-prefill", action="store_true", help="skip the T=2048 prefill leg")
    ap.add_argument("--staged", action="store_true",
                    help="also time the pass as three launches (stage 1, stage 2 separately)")
    ap.add_argument("--no-single-layer", action="store_true",
                    help="skip the cache-resident single-layer decode figure (e.g. under a profiler)")
    ap.add_argument("--prefill-tokens", type=int, default=2048)
    ap.add_argument("--prefill-only", action="store_true",
                    help="only run the T=2048 prefill leg and print its JSON")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain MIB-MiB device copy (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the LittleBit stack fits one MI355X, and the "
              "library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(1, args.steps))
        return
    if args.prefill_only:
        w = synth.WORKLOADS[args.workload]
        print(json.dumps(prefill_leg(w, args.prefill_tokens, max(1, args.steps))), flush=True)
        return
    w = synth.WORKLOADS[args.workload]
    layers = args.layers or w.layers
    T = args.tokens

    st, _ = build_stack(w, layers, T)
    P = 2 if w.residual else 1
    b1 = b2 = 0
    for row in st.linears:
        for lin in row:
            s1, s2 = linear_bytes(lin.d_in, lin.d_out, lin.r, P, T)
            b1 += s1
            b2 += s2
    step_s, kern_s = time_decode(st, args.steps, args.warmup, args.settle)
    bw = (b1 + b2) / kern_s / 1e9
    s1_s, s2_s = time_staged(st, max(5, args.steps // 4)) if args.staged else (None, None)
    _log("pass %.1f us by the host clock, %.1f us per launch by events (%.0f GB/s)%s"
         % (step_s * 1e6, kern_s * 1e6, bw,
            "" if s1_s is None else "; three-launch form: stage 1 %.1f us, stage 2 %.1f us"
            % (s1_s * 1e6, s2_s * 1e6)))

    out = {
        "metric": METRIC,
        "value": T / step_s,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1 x e4m3 -> f32 (bf16 in/out)",
        "data": "synthetic",
        "config": {
            "workload": "%s, decode T=%d, %d-layer stack as one group" % (w.title, T, layers),
            "tokens": T, "layers": layers,
            "linears_per_layer": [[s.name, s.d_in, s.d_out] for s in w.linears],
            "algorithmic_bytes_per_pass": b1 + b2,
            "packed_bytes_per_pass": st.packed_bytes() + st.scale_bytes(),
        },
        "roofline": {"bound": "hbm", "achieved": bw, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": bw / HBM_PEAK_GBS,
                     "traffic": measured_traffic(PASS_KERNEL, args.workload, T),
                     "algorithmic_bytes": b1 + b2,
                     "kernel": PASS_KERNEL,
                     "launch_us": kern_s * 1e6,
                     "pass_GBs": (b1 + b2) / step_s / 1e9,
                     "pass_frac": (b1 + b2) / step_s / 1e9 / HBM_PEAK_GBS},
    }
    if s1_s is not None:
        out["three_launch_form"] = {"stage1_us": s1_s * 1e6, "stage1_GBs": b1 / s1_s / 1e9,
                                    "stage2_us": s2_s * 1e6, "stage2_GBs": b2 / s2_s / 1e9}
    del st
    torch.cuda.empty_cache()
    if not args.no_single_layer:
        out["decode_single_layer"] = single_layer_leg(w, T)
    if not args.no_prefill and args.prefill_tokens > 32:
        try:
            out["prefill"] = prefill_leg(w, args.prefill_tokens, max(3, args.steps // 50))
        except Exception as e:  # report, do not hide
            out["prefill"] = {"error": repr(e)}
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, T, layers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
