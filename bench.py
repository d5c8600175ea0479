#!/usr/bin/env python3
"""Benchmark of the LittleBit layer forward on one MI355X.

One step is one forward pass of the token batch through a stack of seeded
synthetic LittleBit linears: by default the Llama2-70B-shaped decoder-layer
linears (q/o 8192x8192, k/v 8192x1024, gate/up 8192x28672, down 28672x8192) at
0.1 bits per weight with the residual path, 80 independent layers, decode T=1,
run as one group (one kernel launch per pass).  The stack holds ~0.8 GB of
packed signs, more than three times the 256 MB Infinity Cache, so every pass
streams from HBM.  Prints ONE JSON line.

Beside it: the prefill leg (the same shapes at T=2048, one layer, the GEMM
path), the Llama2-7B-shaped 32-layer stack at T=4 and T=32, the two small
cache-resident configurations, and the measured ceilings (a streaming read,
back-to-back bf16 matrix instructions).  The CPU baseline times the fp64
oracle on one layer of the same stack and scales to the stack (and on a
token subset of the prefill layer).

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
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector
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


def cpu_info():
    """The host CPU's model name and logical core count (os.cpu_count)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, os.cpu_count()


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
    model, nproc = cpu_info()
    return {"value": T / (t_layer * layers), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "cpu_model": model, "nproc": nproc,
            "sample": "one layer (%d linears, seeded inputs) at T=%d, %d passes in %.1f s, scaled "
                      "to the %d-layer stack" % (len(w.linears), T, passes, t_total, layers)}


def oracle_prefill(w, tokens=16):
    """The fp64 oracle on one layer of the workload at `tokens` tokens (seeded
    inputs of the layer's shapes), scaled linearly to tokens per second (the
    tokens are independent)."""
    import oracle
    import synth
    t_total = 0.0
    for i, sh in enumerate(w.linears):
        r, rp = oracle.rank_for_budget(sh.d_in, sh.d_out, w.b_num, w.b_den, w.residual)
        inp = synth.layer_inputs(i, sh.d_in, sh.d_out, rp, 2 if w.residual else 1)
        x = synth.activations(synth.activation_seed(2048), tokens, sh.d_in, w.dtype)
        t0 = time.perf_counter()
        oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l)
        t_total += time.perf_counter() - t0
    model, nproc = cpu_info()
    return {"value": tokens / t_total, "unit": "tok/s", "cores": oracle.max_threads(), "kind": "oracle",
            "cpu_model": model, "nproc": nproc,
            "sample": "one layer (%d linears) on %d of the 2048 tokens in %.2f s, scaled linearly"
                      % (len(w.linears), tokens, t_total)}


def ceilings():
    """The measured ceilings beside the published peaks: a streaming read of
    2 GiB (eight times the Infinity Cache) and back-to-back bf16 matrix
    instructions on register operands (lb_ceiling_stream_read,
    lb_ceiling_mfma_bf16), each timed with HIP events on the launch stream."""
    import torch
    import binarized_rank_linear_amd as lb
    L = lb.lib()
    s = torch.cuda.current_stream()
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    blocks = 256 * 8
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")

    def timed(fn, reps):
        for _ in range(3):
            fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    def read():
        assert L.lb_ceiling_stream_read(buf.data_ptr(), nbytes, out.data_ptr(), blocks, s.cuda_stream) == 0

    iters, mblocks = 4000, 256 * 4

    def mfma(rnd):
        assert L.lb_ceiling_mfma_bf16(iters, rnd, out.data_ptr(), mblocks, s.cuda_stream) == 0

    t_read = timed(read, 20)
    t_mfma = timed(lambda: mfma(0), 5)
    t_mfma_r = timed(lambda: mfma(1), 5)
    gbs = nbytes / t_read / 1e9
    tfl = mblocks * 4 * iters * 8 * 32768 / t_mfma / 1e12
    tfl_r = mblocks * 4 * iters * 8 * 32768 / t_mfma_r / 1e12
    del buf
    torch.cuda.empty_cache()
    return {"stream_read_GBs": gbs, "stream_read_frac": gbs / HBM_PEAK_GBS,
            "mfma_bf16_TFLOPs": tfl, "mfma_bf16_frac": tfl / BF16_PEAK_TFLOPS,
            "mfma_bf16_random_TFLOPs": tfl_r, "mfma_bf16_random_frac": tfl_r / BF16_PEAK_TFLOPS,
            "how": "2 GiB read by 2048 workgroups (a contiguous share each), 16-byte non-temporal loads, "
                   "8 in flight per thread; "
                   "1024 workgroups x 4 waves x %d x 8 independent v_mfma_f32_32x32x16_bf16 on constant "
                   "operands, and (random) cycling through four pseudo-random operands each" % iters}


def clock_probe(w, secs=3.0):
    """The GPU clock and socket power under each load: the load runs back to
    back for `secs` seconds while a thread samples `rocm-smi --showmetrics`
    (a child process per sample; the metrics refresh about once a second, so
    samples from the load's first second are dropped).  Loads: the decode
    pass of the workload's stack (T = 1), the bf16 matrix-rate ceiling on
    constant and on pseudo-random operands, one prefill layer of the workload
    at T = 2048, and the vendor library's bf16 GEMM of 8192 x 8192 x 8192 on
    random data.  Reports the median clock (MHz), the median power (W) and
    the load's time per call."""
    import re
    import shutil
    import statistics
    import subprocess
    import threading
    import torch
    import synth
    import binarized_rank_linear_amd as lb
    if shutil.which("rocm-smi") is None:
        return {"error": "rocm-smi not found"}
    pat_c = re.compile(r"current_gfxclk \(MHz\):\s*(\d+)")
    pat_p = re.compile(r"current_socket_power \(W\):\s*(\d+)")

    def run(name, fn, calls_per_sync=4):
        samples, stop = [], threading.Event()

        def sample():
            while not stop.is_set():
                t = time.perf_counter()
                r = subprocess.run(["rocm-smi", "--showmetrics"], capture_output=True, text=True, timeout=30)
                c, p = pat_c.search(r.stdout), pat_p.search(r.stdout)
                if c and p:
                    samples.append((t, int(c.group(1)), int(p.group(1))))
                stop.wait(0.1)
        torch.cuda.synchronize()
        th = threading.Thread(target=sample)
        t0 = time.perf_counter()
        th.start()
        n = 0
        while time.perf_counter() - t0 < secs:
            fn()
            n += 1
            if n % calls_per_sync == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        stop.set()
        th.join()
        kept = [x for x in samples if x[0] - t0 >= 1.0]
        _log("clocks: %s %d calls, %d samples kept" % (name, n, len(kept)))
        return {"load": name, "ms_per_call": el / n * 1e3,
                "gfxclk_MHz": statistics.median(x[1] for x in kept) if kept else None,
                "socket_power_W": statistics.median(x[2] for x in kept) if kept else None,
                "samples": len(kept)}

    L = lb.lib()
    s = torch.cuda.current_stream()
    res = []
    st, _ = build_stack(w, w.layers, 1)
    res.append(run("decode pass, %d-layer stack, T=1" % w.layers, st.group.run, 20))
    del st
    torch.cuda.empty_cache()
    out = torch.empty(1024 * 256, dtype=torch.float32, device="cuda")
    for rnd, nm in ((0, "constant"), (1, "pseudo-random")):
        res.append(run("bf16 matrix-rate ceiling, %s operands" % nm,
                       lambda: L.lb_ceiling_mfma_bf16(4000, rnd, out.data_ptr(), 1024, s.cuda_stream)))
    T = 2048
    layer = []
    for i, sh in enumerate(w.linears):
        r, rp = lb.rank_for_budget(sh.d_in, sh.d_out, w.b_num, w.b_den, w.residual)
        U, V, h, g, l = synth.device_layer(synth.layer_seed(0, i), sh.d_in, sh.d_out, rp, 2 if w.residual else 1)
        layer.append(lb.PackedLinear.from_factors(U, V, h, g, l))
        del U, V
    xs = {d: synth.device_activations(synth.activation_seed(d), T, d, "bf16") for d in {q.d_in for q in w.linears}}
    ys = [torch.empty((T, lin.d_out), dtype=torch.bfloat16, device="cuda") for lin in layer]
    grp = lb.Group([(xs[lin.d_in], y, lin) for lin, y in zip(layer, ys)], T, torch.bfloat16, torch.bfloat16)

    def pf():
        grp.run_stage(1)
        grp.run_stage(2)
    res.append(run("prefill, one layer, T=2048", pf))
    del grp, layer, xs, ys
    torch.cuda.empty_cache()
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    res.append(run("vendor bf16 GEMM 8192^3, random data", lambda: torch.mm(a, b)))
    return {"workload": w.title, "clocks": res}


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
    if source_sha256(kv.get("source", "")) != kv.get("source_sha256"):
        return None
    return float(kv["traffic_bytes_per_launch"])


def source_sha256(names):
    """sha256 over the named csrc files (space-separated), in that order; None
    when one is missing."""
    h = hashlib.sha256()
    for name in names.split():
        src = os.path.join(ROOT, "binarized_rank_linear_amd", "csrc", name)
        if not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    return h.hexdigest() if names.split() else None


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


def decode_stack_leg(key, T, steps, layers=0):
    """A second decode figure: the workload's stack at T tokens as one group,
    HIP events around `steps` passes after a settle period.  Below 20 tokens
    HBM bounds the pass (fraction of 8 TB/s over the algorithmic bytes); at
    more tokens the dense-equivalent matrix work 2 T r (d_in + d_out) is
    also reported against the bf16 peak."""
    import torch
    import synth
    w = synth.WORKLOADS[key]
    L = layers or w.layers
    st, _ = build_stack(w, L, T)
    P = 2 if w.residual else 1
    nbytes = sum(sum(linear_bytes(lin.d_in, lin.d_out, lin.r, P, T)) for row in st.linears for lin in row)
    flops = sum(2 * T * lin.r * (lin.d_in + lin.d_out) for row in st.linears for lin in row)
    step_s, kern_s = time_decode(st, steps, 5, 0.2)
    del st
    torch.cuda.empty_cache()
    import binarized_rank_linear_amd as lb
    s0 = w.linears[0]
    r0, _ = lb.rank_for_budget(s0.d_in, s0.d_out, w.b_num, w.b_den, w.residual)
    path = lb.linear_path(s0.d_in, s0.d_out, r0, T, w.residual, torch.bfloat16, torch.bfloat16)
    kernels = {lb.LB_PATH_DECODE: "decode kernels", lb.LB_PATH_PREFILL: "GEMM kernels"}.get(path, "vector-ALU kernels")
    out = {"workload": "%s, T=%d, %d-layer stack as one group (%s)" % (w.title, T, L, kernels),
           "us_per_pass": kern_s * 1e6, "tok_per_s": T / step_s, "algorithmic_bytes": nbytes,
           "GBs": nbytes / kern_s / 1e9, "hbm_frac": nbytes / kern_s / 1e9 / HBM_PEAK_GBS,
           "dense_equivalent_TFLOPs": flops / kern_s / 1e12,
           "mfma_frac": flops / kern_s / 1e12 / BF16_PEAK_TFLOPS}
    out["bound"] = "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (BF16_PEAK_TFLOPS * 1e12) else "mfma"
    return out


def decoder_stack_leg(key, T, steps, layers=0):
    """The workload's layers as a model runs them at decode time: each
    decoder layer (two RMSNorms, q/k/v, a one-token attention, o, the SwiGLU
    block, two residual adds) feeds the next, so the layers run one after
    another.  The whole stack is captured as one HIP graph; HIP events
    around `steps` replays.  Factors are drawn with l scaled for unit gain so
    the activations stay in range through the chain."""
    import torch
    import synth
    from binarized_rank_linear_amd.stack import DecoderStack
    w = synth.WORKLOADS[key]
    L = layers or w.layers
    sh = {s.name: s for s in w.linears}
    P = 2 if w.residual else 1

    def make(layer, i, di, do, rp, paths):
        U, V, h, g, l = synth.device_layer(synth.layer_seed(layer, i), di, do, rp, paths)
        return U, V, h, g, (l.float() * synth.unit_gain_l(di, rp, paths)).half()

    t0 = time.time()
    st = DecoderStack(sh["q"].d_in, sh["gate"].d_out, w.heads[0], w.heads[1], L, w.b_num, w.b_den,
                      w.residual, make)
    x = synth.device_activations(synth.activation_seed(T), T, sh["q"].d_in, "bf16")
    bufs = [torch.empty_like(x), torch.empty_like(x)]
    ws = torch.empty(st.workspace_bytes(T), dtype=torch.uint8, device="cuda")
    _log("decoder stack of %d layers built in %.1f s" % (L, time.time() - t0))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        st.forward(x, bufs, ws, stream=s)              # eager once (the graph needs no warm state)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            st.forward(x, bufs, ws, stream=s)
        for _ in range(5):
            g.replay()
        s.synchronize()
        t1 = time.perf_counter()
        while time.perf_counter() - t1 < 0.2:
            g.replay()
            s.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(steps):
            g.replay()
        e1.record(s)
        s.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / steps
    nbytes = sum(sum(linear_bytes(lin.d_in, lin.d_out, lin.r, P, T)) for lin in st.linears())
    finite = bool(torch.isfinite(bufs[(L - 1) & 1].float()).all())
    del st, g
    torch.cuda.empty_cache()
    return {"workload": "%s, %d decoder layers chained at decode T=%d (one HIP graph)" % (w.title, L, T),
            "us_per_pass": t * 1e6, "us_per_layer": t * 1e6 / L, "tok_per_s": T / t,
            "algorithmic_bytes": nbytes, "GBs": nbytes / t / 1e9,
            "hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBS, "output_finite": finite}


def dual_svid_leg(reps=3):
    """The Dual-SVID initialisation of two linears from seeded dense
    weights with a decaying spectrum: the 1024 x 1024 configuration-1 linear
    (rank 512, one path) and a Qwen3-0.6B-shaped gate projection (1024 ->
    3072, 0.55 bpw, with the residual path).  Seconds per linear by the host
    clock around the synchronous call (after one untimed call), and the fp64
    oracle's time for the same (numpy SVD on the host cores); the same with
    the Joint-ITQ rotation of each path (20 alternations) and the layer's
    relative error with it."""
    import numpy as np
    import torch
    import synth
    import oracle
    from oracle import svid
    import binarized_rank_linear_amd as lb
    out = []
    for (d_out, d_in, bn, bd, res, name) in ((1024, 1024, 1, 1, False, "1024 x 1024 linear, 1.0 bpw"),
                                             (3072, 1024, 55, 100, True, "Qwen3-0.6B-shaped gate 1024 -> 3072, 0.55 bpw + residual")):
        r, rp = lb.rank_for_budget(d_in, d_out, bn, bd, res)
        W = synth.dense_weight(5, d_out, d_in)
        Wd = torch.from_numpy(W).cuda()
        ws = lb.workspace(lb.lib().lb_dual_svid_workspace_bytes(d_out, d_in, r, int(res)))
        lb.dual_svid(Wd, r, res, ws=ws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            lin = lb.dual_svid(Wd, r, res, ws=ws)
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / reps
        t0 = time.perf_counter()
        U, V, h, g, l = svid.dual_svid(W, rp, res)
        t_cpu = time.perf_counter() - t0
        err = oracle.rel_l2(svid.reconstruction(U, V, h, g, l), W)
        # with the Joint-ITQ rotation (LittleBit-2), 20 alternations per path
        wsi = lb.workspace(lb.lib().lb_dual_svid_itq_workspace_bytes(d_out, d_in, r, int(res)))
        lb.dual_svid(Wd, r, res, ws=wsi, itq_iters=20)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        lin_i, Ui, Vi = lb.dual_svid(Wd, r, res, ws=wsi, itq_iters=20, float_factors=True)
        torch.cuda.synchronize()
        t_itq = time.perf_counter() - t0
        err_itq = oracle.rel_l2(svid.reconstruction(
            Ui.cpu().numpy().astype(np.float64), Vi.cpu().numpy().astype(np.float64),
            lin_i.h.cpu().numpy().view(np.uint16), lin_i.g.cpu().numpy().view(np.uint16),
            lin_i.l.cpu().numpy().view(np.uint16)), W)
        out.append({"workload": "Dual-SVID initialisation, %s (r = %d)" % (name, r), "s_per_linear": t,
                    "weights_per_s": d_out * d_in / t, "relative_error_of_the_layer": err,
                    "with_joint_itq": {"alternations": 20, "s_per_linear": t_itq,
                                       "relative_error_of_the_layer": err_itq},
                    "cpu_baseline": {"s_per_linear": t_cpu, "kind": "oracle", "cores": oracle.max_threads(),
                                     "sample": "the same linear, numpy SVD (fp64)"}})
        del lin, ws, Wd, wsi, lin_i, Ui, Vi
    torch.cuda.empty_cache()
    return out


def blas_threads():
    """Threads numpy's BLAS and LAPACK calls may use (the OpenMP setting)."""
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def joint_itq_leg(iters=10):
    """The Joint-ITQ rotation (LittleBit-2 initialisation) of one path's
    factors at two layer shapes: a Llama2-7B-shaped gate projection (4096 ->
    11008, 1.0 bpw with the residual: r_p = 1488) and a Llama2-70B-shaped
    down projection (28672 -> 8192, 0.1 bpw with the residual: r_p = 304).
    The factors are seeded on the GPU: Gaussian columns scaled to unit norm
    times sqrt(s_k), s_k = (1 + k)^-0.6 (the shape of an SVD split of a
    weight with a decaying spectrum).  Seconds per alternation by the host
    clock around one synchronous call of `iters` alternations (after a call
    of one); the rate counts the two GEMMs over the long side (4 D r_p^2
    flops per alternation, D = d_out + d_in), not the polar step's, against
    the fp32 vector peak; the oracle (numpy fp64) runs two alternations on the
    same factors."""
    import numpy as np
    import torch
    from oracle import itq
    import binarized_rank_linear_amd as lb
    out = []
    for (d_out, d_in, r_p, name) in ((11008, 4096, 1488, "Llama2-7B-shaped gate 4096 -> 11008, 1.0 bpw + residual"),
                                     (8192, 28672, 304, "Llama2-70B-shaped down 28672 -> 8192, 0.1 bpw + residual")):
        g = torch.Generator(device="cuda").manual_seed(7)
        sk = (1.0 + torch.arange(r_p, device="cuda", dtype=torch.float32)) ** -0.3
        U = torch.randn((d_out, r_p), device="cuda", generator=g) * (sk / float(np.sqrt(d_out)))
        V = torch.randn((d_in, r_p), device="cuda", generator=g) * (sk / float(np.sqrt(d_in)))
        ws = lb.workspace(lb.lib().lb_joint_itq_workspace_bytes(d_out, d_in, r_p))
        lb.joint_itq(U.clone(), V.clone(), 1, ws=ws)
        torch.cuda.synchronize()
        Ua, Va = U.clone(), V.clone()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        R, obj = lb.joint_itq(Ua, Va, iters, ws=ws)
        torch.cuda.synchronize()
        t = (time.perf_counter() - t0) / iters
        o = obj.cpu().numpy()
        D = d_out + d_in
        rate = 4.0 * D * r_p * r_p / t / 1e12
        Uh, Vh = U.cpu().numpy().astype(np.float64), V.cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        _, qo = itq.joint_itq(Uh, Vh, 2)
        t_cpu = (time.perf_counter() - t0) / 2
        out.append({"workload": "Joint-ITQ rotation, %s: one path's factors (r_p = %d), %d alternations"
                                % (name, r_p, iters),
                    "s_per_alternation": t, "objective_start": float(o[0]), "objective_end": float(o[-1]),
                    "oracle_objective_after_2": float(qo[-1]), "gpu_objective_after_2": float(o[2]),
                    "roofline": {"bound": "alu", "achieved": rate, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": rate / FP32_PEAK_TFLOPS,
                                 "counts": "4 D r_p^2 flops per alternation (the two GEMMs over the long side)"},
                    "cpu_baseline": {"s_per_alternation": t_cpu, "kind": "oracle", "cores": blas_threads(),
                                     "sample": "two alternations on the same factors, numpy fp64"}})
        del U, V, Ua, Va, ws
    torch.cuda.empty_cache()
    return out


def cache_resident_legs(reps=2000):
    """The two small configurations, whose factors stay in the caches: the
    1024 x 1024 linear at 1.0 bit per weight (fp32, T = 1 and 8) and the
    Qwen3-0.6B-shaped SwiGLU block at 0.55 bits per weight with the residual
    (bf16, T = 1 and 16); microseconds per call, HIP events around `reps`
    calls with preallocated outputs and workspace."""
    import torch
    import synth
    import binarized_rank_linear_amd as lb
    s = torch.cuda.current_stream()

    def timed(fn):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.1:
            for _ in range(50):
                fn()
            torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    res = []
    r, rp = lb.rank_for_budget(1024, 1024, 1, 1, False)
    U, V, h, g, l = synth.device_layer(0, 1024, 1024, rp, 1)
    lin = lb.PackedLinear.from_factors(U, V, h, g, l)
    for T in (1, 8):
        x = synth.device_activations(synth.activation_seed(T), T, 1024, "f32")
        y = torch.empty((T, 1024), dtype=torch.float32, device="cuda")
        ws = lb.workspace(lb.linear_workspace_bytes(lin, T))
        t = timed(lambda: lb.linear_forward(x, lin, torch.float32, ws=ws, out=y))
        nb = sum(linear_bytes(1024, 1024, r, 1, T, 4))
        res.append({"workload": "1024 x 1024 linear, 1.0 bpw (r = 512), fp32, T=%d, cache-resident" % T,
                    "us_per_call": t * 1e6, "tok_per_s": T / t, "effective_GBs": nb / t / 1e9})
    w = synth.WORKLOADS["c2"]
    mats = []
    for i, sh in enumerate(w.linears):
        r, rp = lb.rank_for_budget(sh.d_in, sh.d_out, w.b_num, w.b_den, w.residual)
        U, V, h, g, l = synth.device_layer(i, sh.d_in, sh.d_out, rp, 2)
        mats.append(lb.PackedLinear.from_factors(U, V, h, g, l))
    gate, up, down = mats
    for T in (1, 16):
        x = synth.device_activations(synth.activation_seed(T), T, 1024, "bf16")
        y = torch.empty((T, 1024), dtype=torch.bfloat16, device="cuda")
        ws = lb.workspace(lb.mlp_workspace_bytes(gate, down, T))
        t = timed(lambda: lb.mlp_forward(x, gate, up, down, torch.bfloat16, ws=ws, out=y))
        nb = sum(sum(linear_bytes(m.d_in, m.d_out, m.r, 2, T)) for m in mats)
        res.append({"workload": "Qwen3-0.6B-shaped SwiGLU block (1024 -> 3072 -> 1024), 0.55 bpw with the "
                                "residual, bf16, T=%d, cache-resident" % T,
                    "us_per_call": t * 1e6, "tok_per_s": T / t, "effective_GBs": nb / t / 1e9})
    return res


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


def prefill_leg(w, T, steps, settle_s=0.3):
    """One layer of the workload's linears at T tokens as one GEMM-path group:
    stage 1 (and the d_in-piece reduce) for all linears in one launch, then
    stage 2 in one launch.  After untimed passes for settle_s seconds (the
    clocks leave idle and reach their loaded state), HIP events on the launch
    stream bracket `steps` back-to-back passes (the figure and the roofline);
    a second run of `steps` passes with an event between the stages gives
    the split between them."""
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
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(8):
            grp.run_stage(1)
            grp.run_stage(2)
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        grp.run_stage(1)
        grp.run_stage(2)
    e1.record(s)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / steps * 1e-3
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
    f1 = sum(2 * T * lin.r * lin.d_in for lin in layer)
    f2 = sum(2 * T * lin.r * lin.d_out for lin in layer)
    flops = f1 + f2
    return {"workload": "%s, one layer (%d linears) as one group, T=%d (GEMM path)"
                        % (w.title, len(layer), T), "T": T,
            "tok_per_s": T / t, "ms_per_layer": t * 1e3,
            "stage1_us": t1 * 1e6, "stage2_us": t2 * 1e6, "split_note": "stage times from passes with an "
            "event between the stages (their sum exceeds the back-to-back pass)",
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
    ap.add_argument("--svid-only", action="store_true",
                    help="only run the Dual-SVID initialisation leg and print its JSON")
    ap.add_argument("--itq-only", action="store_true",
                    help="only run the Joint-ITQ leg and print its JSON")
    ap.add_argument("--clocks", action="store_true",
                    help="only sample the GPU clock and power (rocm-smi) under each load and print them")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other decode legs (32-layer stack at T=4 and T=32), the "
                         "cache-resident configurations and the measured ceilings")
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
    if args.svid_only:
        print(json.dumps(dual_svid_leg()), flush=True)
        return
    if args.itq_only:
        print(json.dumps(joint_itq_leg()), flush=True)
        return
    if args.clocks:
        print(json.dumps(clock_probe(synth.WORKLOADS[args.workload])), flush=True)
        return
    if args.prefill_only:
        w = synth.WORKLOADS[args.workload]
        print(json.dumps(prefill_leg(w, args.prefill_tokens, max(1, args.steps), args.settle)), flush=True)
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
            out["prefill"] = prefill_leg(w, args.prefill_tokens, max(50, args.steps // 4), args.settle)
        except Exception as e:  # report, do not hide
            out["prefill"] = {"error": repr(e)}
    if not args.no_extra:
        out["decode_more"] = [decode_stack_leg("c3", 4, max(20, args.steps // 2)),
                              decode_stack_leg("c3", 32, max(10, args.steps // 10))]
        out["decoder_chain"] = [decoder_stack_leg(args.workload, T, max(10, args.steps // 10)),
                                decoder_stack_leg("c3", 1, max(10, args.steps // 10))]
        out["cache_resident"] = cache_resident_legs()
        out["dual_svid"] = dual_svid_leg()
        out["joint_itq"] = joint_itq_leg()
        c = ceilings()
        out["ceilings"] = c
        out["roofline"]["frac_of_measured_ceiling"] = bw / c["stream_read_GBs"]
        if isinstance(out.get("prefill"), dict) and "roofline" in out["prefill"]:
            out["prefill"]["roofline"]["frac_of_measured_ceiling"] = \
                out["prefill"]["roofline"]["achieved"] / c["mfma_bf16_TFLOPs"]
            out["prefill"]["roofline"]["frac_of_random_operand_ceiling"] = \
                out["prefill"]["roofline"]["achieved"] / c["mfma_bf16_random_TFLOPs"]
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, T, layers)
        if isinstance(out.get("prefill"), dict) and "roofline" in out["prefill"]:
            out["prefill"]["cpu_baseline"] = oracle_prefill(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
