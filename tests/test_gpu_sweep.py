"""Seeded sweep of the forward against the fp64 oracle over shapes, ranks,
token counts, activation and output dtypes, scale signs and kernel paths.

The fixed cases elsewhere pin each kernel family at chosen sizes; this file
draws many more combinations from one seed, so that an edge the fixed cases
miss (a rank off a tile grid, a d_in off the vector width, a token count
between two tile sizes) meets the oracle too.  Scales g, h and l are drawn
with both signs in a third of the cases: the method's scales are magnitudes,
but the layer's formula (sesamedisk page, "What the method actually
computes", Proposition 1) and the boundary accept any fp16 value.

Tolerances are the parity bounds of the other GPU tests: relative L2 1e-3
(fp32 outputs) or 8e-3 (bf16 outputs), and every element within 8 x bound x
rms(reference).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (TOL, assert_close, dev_layer, dev_layer_ld, host_layer_from_dev, say, torch_or_skip,
                      x_to_dev, y_to_np)

pytestmark = pytest.mark.gpu

PATH_FLAG = {"auto": 0, "decode": 1, "prefill": 2, "valu": 3}
MAX_WORK = 1.2e8          # oracle multiply-adds per case, so the CPU side stays fast


def _dim(rng):
    kind = rng.integers(4)
    if kind == 0:
        return int(rng.integers(1, 64))
    if kind == 1:
        return int(rng.integers(64, 700))
    if kind == 2:
        return int(rng.integers(700, 2600))
    return int(rng.choice([128, 256, 512, 1024, 2048, 4096]) + rng.integers(-3, 4))


def _single_cases(seed=20261204, n=160):
    rng = np.random.default_rng(seed)
    paths = ["auto", "decode", "valu", "prefill"]
    cases = []
    while len(cases) < n:
        path = paths[len(cases) % 4]
        d_in, d_out = max(1, _dim(rng)), max(1, _dim(rng))
        P = int(rng.integers(1, 3))
        r_p = int(rng.choice([rng.integers(1, 40), rng.integers(40, 400)]))
        if path == "decode":
            T = int(rng.integers(1, 33))
        elif path == "valu":
            T = int(rng.integers(1, 41))
        else:
            T = int(rng.choice([rng.integers(1, 40), rng.integers(40, 300)]))
        x_dt = str(rng.choice(["f32", "bf16"]))
        y_dt = "bf16" if path == "prefill" else str(rng.choice(["f32", "bf16"]))
        signed = bool(rng.integers(3) == 0)
        if T * P * r_p * (d_in + d_out) > MAX_WORK:
            continue
        cases.append((len(cases), path, d_in, d_out, r_p, P, T, x_dt, y_dt, signed))
    return cases


SINGLE = _single_cases()


def _inputs(i, d_in, d_out, r_p, P, signed):
    lo = -1.5 if signed else 0.5
    inp = synth.layer_inputs(7000 + i, d_in, d_out, r_p, P, scale_lo=lo, scale_hi=1.5)
    return inp


@pytest.mark.parametrize("case", SINGLE, ids=lambda c: "%d-%s-%dx%d-r%dx%d-T%d-%s-%s%s" % (
    c[0], c[1], c[2], c[3], c[5], c[4], c[6], c[7], c[8], "-signed" if c[9] else ""))
def test_single_linear_sweep(case):
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    i, path, d_in, d_out, r_p, P, T, x_dt, y_dt, signed = case
    inp = _inputs(i, d_in, d_out, r_p, P, signed)
    x = synth.activations(8000 + i, T, d_in, x_dt)
    layer = dev_layer(inp)
    xd = x_to_dev(x)
    od = torch.float32 if y_dt == "f32" else torch.bfloat16
    say("sweep", case)
    y = lb.linear_forward(xd, layer, od, PATH_FLAG[path])
    torch.cuda.synchronize()
    ref = oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l)
    assert_close(y_to_np(y), ref, TOL[y_dt], case)
    assert lb.device_faults() == 0


def _group_cases(seed=20261205, n=24):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        k = len(cases)
        T = int(rng.choice([1, 2, int(rng.integers(3, 9)), int(rng.integers(9, 33)),
                            int(rng.integers(33, 200))]))
        y_dt = "bf16" if k % 2 == 0 else str(rng.choice(["f32", "bf16"]))
        P = int(rng.integers(1, 3))
        d_x = _dim(rng)                              # one shared input width, as in a layer
        lins = []
        for j in range(int(rng.integers(2, 7))):
            d_in = d_x if rng.integers(2) else max(1, _dim(rng))
            d_out = max(1, _dim(rng))
            r_p = int(rng.choice([rng.integers(1, 40), rng.integers(40, 300)]))
            lins.append((d_in, d_out, r_p))
        if sum(T * P * r * (a + b) for a, b, r in lins) > 3 * MAX_WORK:
            continue
        cases.append((k, T, y_dt, P, tuple(lins), bool(rng.integers(3) == 0)))
    return cases


GROUPS = _group_cases()


@pytest.mark.parametrize("case", GROUPS, ids=lambda c: "%d-T%d-%s-P%d-n%d%s" % (
    c[0], c[1], c[2], c[3], len(c[4]), "-signed" if c[5] else ""))
def test_group_sweep(case):
    """The same linears through the stateless grouped call and as a prepared
    group (run twice): each output within the bound of the oracle, and the
    two forms bit for bit equal."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    k, T, y_dt, P, lins, signed = case
    od = torch.float32 if y_dt == "f32" else torch.bfloat16
    say("group sweep", case)
    items, refs = [], []
    xs = {}
    for j, (d_in, d_out, r_p) in enumerate(lins):
        inp = _inputs(100 * k + j, d_in, d_out, r_p, P, signed)
        if d_in not in xs:
            x = synth.activations(9000 + 10 * k + len(xs), T, d_in, "bf16")
            xs[d_in] = (x, x_to_dev(x))
        x, xd = xs[d_in]
        items.append((xd, torch.empty((T, d_out), dtype=od, device="cuda"), dev_layer(inp)))
        refs.append(oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l))
    lb.linear_forward_grouped(items)
    torch.cuda.synchronize()
    for j, it in enumerate(items):
        assert_close(y_to_np(it[1]), refs[j], TOL[y_dt], (case, j))
    grp = lb.Group([(x, torch.empty_like(y), l) for x, y, l in items], T, torch.bfloat16, od)
    for rep in range(2):
        grp.run()
        torch.cuda.synchronize()
        for j, it in enumerate(items):
            a, b = it[1], grp.items[j][1]
            bits = (lambda t: t.view(torch.int16)) if od == torch.bfloat16 else (lambda t: t.view(torch.int32))
            assert torch.equal(bits(a), bits(b)), (case, rep, j)
    grp.release()
    assert lb.device_faults() == 0


def _latent_cases(seed=20261206, n=24):
    rng = np.random.default_rng(seed)
    paths = ["auto", "decode", "valu", "prefill"]
    cases = []
    while len(cases) < n:
        path = paths[len(cases) % 4]
        d_in, d_out = max(1, _dim(rng)), max(1, _dim(rng))
        P = int(rng.integers(1, 3))
        r_p = int(rng.choice([rng.integers(1, 40), rng.integers(40, 300)]))
        T = int(rng.integers(1, 33)) if path in ("decode", "valu") else int(rng.integers(1, 200))
        if T * P * r_p * (d_in + d_out) > MAX_WORK:
            continue
        cases.append((len(cases), path, d_in, d_out, r_p, P, T))
    return cases


LATENT = _latent_cases()


@pytest.mark.parametrize("case", LATENT, ids=lambda c: "%d-%s-%dx%d-r%dx%d-T%d" % (
    c[0], c[1], c[2], c[3], c[5], c[4], c[6]))
def test_latent_sweep(case):
    """lb_linear_stage1 then lb_linear_stage2 equals lb_linear_forward bit for
    bit (bf16 outputs) when t holds the kernels' own latent precision (bf16 on
    the GEMM kernels, fp32 on the decode and vector-ALU kernels: the path the
    library reports for the call), and the latents are within the bf16 bound
    of the oracle's
    t = l * sign(V)^T (g * x)."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    i, path, d_in, d_out, r_p, P, T = case
    inp = _inputs(500 + i, d_in, d_out, r_p, P, i % 3 == 0)
    x = synth.activations(600 + i, T, d_in, "bf16")
    layer = dev_layer(inp)
    xd = x_to_dev(x)
    say("latent sweep", case)
    fl = PATH_FLAG[path]
    gemm = lb.linear_path(d_in, d_out, P * r_p, T, P == 2, torch.bfloat16, torch.bfloat16, fl) == lb.LB_PATH_PREFILL
    tt = torch.bfloat16 if gemm else torch.float32
    y = lb.linear_forward(xd, layer, torch.bfloat16, fl)
    t = lb.linear_stage1(xd, layer, tt, torch.bfloat16, fl)
    y2 = lb.linear_stage2(t, layer, torch.bfloat16, fl)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), case
    tref = oracle.linear_latents(x, inp.V, inp.g, inp.l)
    assert_close(y_to_np(t), tref, TOL["bf16"], case)
    assert lb.device_faults() == 0


def _mlp_cases(seed=20261207, n=12):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d_model, d_ff = max(1, _dim(rng)), max(1, _dim(rng))
        P = int(rng.integers(1, 3))
        r_gu, r_dn = (int(rng.choice([rng.integers(1, 40), rng.integers(40, 300)])) for _ in range(2))
        T = int(rng.choice([1, 2, int(rng.integers(3, 9)), int(rng.integers(9, 33)), int(rng.integers(33, 120))]))
        x_dt = str(rng.choice(["f32", "bf16"]))
        y_dt = "bf16" if len(cases) % 3 else "f32"
        if T * P * (2 * r_gu * (d_model + d_ff) + r_dn * (d_ff + d_model)) > 2 * MAX_WORK:
            continue
        cases.append((len(cases), d_model, d_ff, r_gu, r_dn, P, T, x_dt, y_dt))
    return cases


MLP = _mlp_cases()


@pytest.mark.parametrize("case", MLP, ids=lambda c: "%d-%dx%d-r%d-%d-P%d-T%d-%s-%s" % c)
def test_mlp_sweep(case):
    """The SwiGLU block down(silu(gate(x)) * up(x)) against the oracle's fp64
    composition (no intermediate rounding), within the output dtype's bound."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    i, d_model, d_ff, r_gu, r_dn, P, T, x_dt, y_dt = case
    g = _inputs(300 + 3 * i, d_model, d_ff, r_gu, P, False)
    u = _inputs(301 + 3 * i, d_model, d_ff, r_gu, P, i % 2 == 1)
    d = _inputs(302 + 3 * i, d_ff, d_model, r_dn, P, False)
    x = synth.activations(400 + i, T, d_model, x_dt)
    od = torch.float32 if y_dt == "f32" else torch.bfloat16
    say("mlp sweep", case)
    y = lb.mlp_forward(x_to_dev(x), dev_layer(g), dev_layer(u), dev_layer(d), od)
    torch.cuda.synchronize()
    assert_close(y_to_np(y), oracle.mlp_forward(x, g, u, d), TOL[y_dt], case)
    assert lb.device_faults() == 0


def _strided_cases(seed=20261208, n=32):
    rng = np.random.default_rng(seed)
    paths = ["auto", "decode", "valu", "prefill"]
    cases = []
    while len(cases) < n:
        path = paths[len(cases) % 4]
        d_in, d_out = max(1, _dim(rng)), max(1, _dim(rng))
        P = int(rng.integers(1, 3))
        r_p = int(rng.choice([rng.integers(1, 40), rng.integers(40, 300)]))
        T = int(rng.integers(1, 33)) if path in ("decode", "valu") else int(rng.integers(1, 200))
        pad_v, pad_u = (4 * int(rng.integers(0, 16)) for _ in range(2))
        if T * P * r_p * (d_in + d_out) > MAX_WORK:
            continue
        cases.append((len(cases), path, d_in, d_out, r_p, P, T, pad_v, pad_u))
    return cases


STRIDED = _strided_cases()


@pytest.mark.parametrize("case", STRIDED, ids=lambda c: "%d-%s-%dx%d-r%dx%d-T%d-pad%d-%d" % (
    c[0], c[1], c[2], c[3], c[5], c[4], c[6], c[7], c[8]))
def test_strided_sweep(case):
    """Plane strides the caller picks (the packed length plus any multiple of
    4 words) on every kernel family, bf16 in and out."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    i, path, d_in, d_out, r_p, P, T, pad_v, pad_u = case
    inp = _inputs(1100 + i, d_in, d_out, r_p, P, i % 3 == 1)
    x = synth.activations(1200 + i, T, d_in, "bf16")
    layer = dev_layer_ld(inp, pad_v, pad_u)
    say("strided sweep", case)
    y = lb.linear_forward(x_to_dev(x), layer, torch.bfloat16, PATH_FLAG[path])
    torch.cuda.synchronize()
    assert_close(y_to_np(y), oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l), TOL["bf16"], case)
    assert lb.device_faults() == 0


def _layer_cases(seed=20261209, n=16):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        n_kv = int(rng.choice([1, 2, 4]))
        grp = int(rng.choice([1, 2, 3, 4]))
        n_heads = n_kv * grp
        dh = int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(40, 140))]))
        d_model = n_heads * dh
        d_ff = max(1, _dim(rng))
        P = int(rng.integers(1, 3))
        rps = tuple(int(rng.choice([rng.integers(1, 24), rng.integers(24, 160)])) for _ in range(4))
        T = int(rng.choice([1, 2, int(rng.integers(3, 9)), int(rng.integers(9, 33))]))
        eps = float(rng.choice([0.0, 1e-6, 1e-5]))
        if d_model < 2:
            continue
        work = T * P * (2 * rps[0] * 2 * d_model + 2 * rps[1] * (d_model + n_kv * dh) +
                        2 * rps[2] * (d_model + d_ff) + rps[3] * (d_ff + d_model))
        if work > 2 * MAX_WORK:
            continue
        cases.append((len(cases), d_model, d_ff, n_heads, n_kv, rps, P, T, eps))
    return cases


LAYERS = _layer_cases()
NAMES = ("q", "k", "v", "o", "gate", "up", "down")


@pytest.mark.parametrize("case", LAYERS, ids=lambda c: "%d-d%d-ff%d-h%d:%d-r%s-P%d-T%d-eps%g" % (
    c[0], c[1], c[2], c[3], c[4], "/".join(map(str, c[5])), c[6], c[7], c[8]))
def test_decoder_layer_sweep(case):
    """One decoder layer at decode time (RMSNorm, q/k/v, one-token attention
    with grouped kv heads, o with the residual, RMSNorm, SwiGLU with the
    residual) against the oracle's composition with the same bf16 hand-offs."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    i, d, ff, n_heads, n_kv, rps, P, T, eps = case
    dkv = d // n_heads * n_kv
    shapes = dict(q=(d, d, rps[0]), k=(d, dkv, rps[1]), v=(d, dkv, rps[1]), o=(d, d, rps[0]),
                  gate=(d, ff, rps[2]), up=(d, ff, rps[2]), down=(ff, d, rps[3]))
    dev, host = {}, {}
    for j, name in enumerate(NAMES):
        di, do, rp = shapes[name]
        U, V, h, g, l = synth.device_layer(synth.layer_seed(1300 + i, j), di, do, rp, P)
        l = (l.float() * synth.unit_gain_l(di, rp, P)).half()
        host[name] = host_layer_from_dev(U, V, h, g, l)
        dev[name] = lb.PackedLinear.from_factors(U, V, h, g, l)
    x = synth.activations(1400 + i, T, d, "bf16")
    say("decoder layer sweep", case)
    layer = lb.DecoderLayer(*(dev[n] for n in NAMES), n_heads=n_heads, n_kv_heads=n_kv, eps=eps)
    y = layer.forward(x_to_dev(x))
    torch.cuda.synchronize()
    assert_close(y_to_np(y), oracle.decoder_layer_forward(x, host, n_heads, n_kv, eps), TOL["bf16"], case)
    assert lb.device_faults() == 0


def _mixed_cases(seed=20261210, n=10):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        calls = []
        for j in range(int(rng.integers(2, 8))):
            T = int(rng.choice([0, 1, 2, int(rng.integers(3, 9)), int(rng.integers(9, 33)),
                                int(rng.integers(33, 120))]))
            x_dt = str(rng.choice(["f32", "bf16"]))
            y_dt = str(rng.choice(["f32", "bf16"]))
            d_in, d_out = max(1, _dim(rng)), max(1, _dim(rng))
            r_p = int(rng.choice([rng.integers(1, 40), rng.integers(40, 200)]))
            P = int(rng.integers(1, 3))
            calls.append((T, x_dt, y_dt, d_in, d_out, r_p, P))
        if sum(c[0] * c[6] * c[5] * (c[3] + c[4]) for c in calls) > 3 * MAX_WORK:
            continue
        cases.append((len(cases), tuple(calls)))
    return cases


MIXED = _mixed_cases()


@pytest.mark.parametrize("case", MIXED, ids=lambda c: "%d-n%d" % (c[0], len(c[1])))
def test_mixed_grouped_call_sweep(case):
    """One stateless grouped call holding linears of different token counts
    (empty ones too), activation and output dtypes and shapes: it splits them
    into sub-groups, and every output is within its dtype's bound of the
    oracle; an empty call's output is left as it was."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    k, calls = case
    say("mixed grouped sweep", case)
    items, refs = [], []
    for j, (T, x_dt, y_dt, d_in, d_out, r_p, P) in enumerate(calls):
        inp = _inputs(1500 + 10 * k + j, d_in, d_out, r_p, P, j % 2 == 1)
        x = synth.activations(1600 + 10 * k + j, T, d_in, x_dt)
        od = torch.float32 if y_dt == "f32" else torch.bfloat16
        y = torch.full((T, d_out), 7.0, dtype=od, device="cuda")
        items.append((x_to_dev(x), y, dev_layer(inp)))
        refs.append(oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l) if T else None)
    lb.linear_forward_grouped(items)
    torch.cuda.synchronize()
    for j, (T, x_dt, y_dt, *_ ) in enumerate(calls):
        if T:
            assert_close(y_to_np(items[j][1]), refs[j], TOL[y_dt], (case, j))
    assert lb.device_faults() == 0


def _pack_cases(seed=20261211, n=24):
    rng = np.random.default_rng(seed)
    return [(k, max(1, _dim(rng)), max(1, _dim(rng)), int(rng.integers(2)), 4 * int(rng.integers(0, 12)))
            for k in range(n)]


PACKS = _pack_cases()


@pytest.mark.parametrize("case", PACKS, ids=lambda c: "%d-%dx%d-axis%d-pad%d" % c)
def test_pack_sweep(case):
    """Sign packing bit for bit against the oracle's packer, with zeros of
    both signs, NaN, infinities and a negative subnormal among the values."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    k, rows, cols, axis, pad = case
    rng = np.random.default_rng(1700 + k)
    M = rng.standard_normal((rows, cols)).astype(np.float32)
    flat = M.reshape(-1)
    for step, v in ((13, 0.0), (17, -0.0), (19, np.nan), (23, -np.inf), (29, np.inf), (31, -1e-40)):
        flat[int(rng.integers(step))::step] = v
    ld = lb.packed_ld(cols if axis == 0 else rows) + pad
    say("pack sweep", case)
    got = lb.pack_signs(torch.from_numpy(M).cuda(), axis, ld)
    torch.cuda.synchronize()
    want = oracle.pack_signs(M, axis, ld)
    got = got.cpu().numpy().view(np.uint32)
    assert got.shape == want.shape and np.array_equal(got, want), case


def _noalloc_cases(seed=20261212, n=16):
    rng = np.random.default_rng(seed)
    paths = ["auto", "decode", "valu", "prefill"]
    cases = []
    while len(cases) < n:
        path = paths[len(cases) % 4]
        d_in, d_out = max(1, _dim(rng)), max(1, _dim(rng))
        P = int(rng.integers(1, 3))
        r_p = int(rng.choice([rng.integers(1, 40), rng.integers(40, 400)]))
        T1 = int(rng.integers(2, 33)) if path in ("decode", "valu") else int(rng.integers(2, 300))
        T2 = int(rng.integers(1, T1))
        y_dt = "bf16" if path == "prefill" else str(rng.choice(["f32", "bf16"]))
        cases.append((len(cases), path, d_in, d_out, r_p, P, T1, T2, y_dt))
    return cases


NOALLOC = _noalloc_cases()


@pytest.mark.parametrize("case", NOALLOC, ids=lambda c: "%d-%s-%dx%d-r%dx%d-T%d-then-%d-%s" % c)
def test_noalloc_sweep(case):
    """lb_linear_forward_noalloc bit for bit equal to lb_linear_forward with
    a caller workspace, on two calls in a row (the second with fewer tokens);
    a request may be refused (LB_EWORKSPACE) only when its workspace can
    exceed the fixed one."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    i, path, d_in, d_out, r_p, P, T1, T2, y_dt = case
    inp = _inputs(1800 + i, d_in, d_out, r_p, P, i % 3 == 2)
    layer = dev_layer(inp)
    od = torch.float32 if y_dt == "f32" else torch.bfloat16
    bits = (lambda t: t.view(torch.int16)) if od == torch.bfloat16 else (lambda t: t.view(torch.int32))
    for k, T in enumerate((T1, T2)):
        say("noalloc sweep", case, "call", k)
        x = x_to_dev(synth.activations(1900 + 2 * i + k, T, d_in, "bf16"))
        want = lb.linear_forward(x, layer, od, PATH_FLAG[path])
        got = torch.full((T, d_out), float("nan"), dtype=od, device="cuda")
        try:
            lb.linear_forward_noalloc(x, layer, od, PATH_FLAG[path], out=got)
        except lb.LBError as e:
            # refused only when the request's workspace can exceed the fixed one
            assert e.status == lb.LB_EWORKSPACE, (case, k, e.status)
            assert lb.linear_workspace_bytes(layer, T, PATH_FLAG[path]) > lb.NOALLOC_SCRATCH_BYTES, (case, k)
            continue
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(want)), (case, k)
