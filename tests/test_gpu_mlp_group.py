"""GPU parity of the SwiGLU block and of layer groups (stacks)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, assert_close, dev_layer, host_layer_from_dev, say, torch_or_skip, x_to_dev, y_to_np

pytestmark = pytest.mark.gpu


def _mlp_layers(seed_base=0):
    w = synth.WORKLOADS["c2"]
    out = []
    for i, sh in enumerate(w.linears):
        r, rp = oracle.rank_for_budget(sh.d_in, sh.d_out, w.b_num, w.b_den, w.residual)
        out.append(synth.layer_inputs(seed_base + i, sh.d_in, sh.d_out, rp, 2))
    return w, out


@pytest.mark.parametrize("T", [1, 16, 5])
@pytest.mark.parametrize("path", [0, 3])
def test_config2_mlp_block(T, path):
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    w, (g, u, d) = _mlp_layers()
    x = synth.activations(synth.activation_seed(T), T, 1024, "bf16")
    say("mlp c2 T", T, "path", path)
    y = lb.mlp_forward(x_to_dev(x), dev_layer(g), dev_layer(u), dev_layer(d), torch.bfloat16,
                       flags=path)
    torch.cuda.synchronize()
    ref = oracle.mlp_forward(x, g, u, d)
    assert_close(y_to_np(y), ref, TOL["bf16"], ("mlp", T, path))


@pytest.mark.parametrize("d_model,d_ff,T", [(520, 1100, 1), (520, 1100, 7), (520, 1100, 12), (1024, 2048, 2),
                                             (1024, 2048, 30), (96, 40, 5)])
def test_mlp_fused_swiglu_ragged(d_model, d_ff, T):
    """The fused decode form of the block (bf16 out): gate and up as one
    group writing bf16, down reading silu(gate) * up as it stages its input,
    on widths that are not multiples of 8 (input by input) and on aligned
    ones, through the fused (T <= 8) and the separate (T > 8) stage-1 forms."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    g = synth.layer_inputs(700 + d_ff, d_model, d_ff, 48, 2)
    u = synth.layer_inputs(701 + d_ff, d_model, d_ff, 48, 2)
    d = synth.layer_inputs(702 + d_ff, d_ff, d_model, 32, 2)
    x = synth.activations(703 + T, T, d_model, "bf16")
    say("mlp fused", d_model, d_ff, "T", T)
    y = lb.mlp_forward(x_to_dev(x), dev_layer(g), dev_layer(u), dev_layer(d), torch.bfloat16)
    torch.cuda.synchronize()
    assert_close(y_to_np(y), oracle.mlp_forward(x, g, u, d), TOL["bf16"], ("mlp fused", d_model, d_ff, T))


def test_mlp_prefill_sampled():
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    w, (g, u, d) = _mlp_layers(10)
    T = 96
    x = synth.activations(7, T, 1024, "bf16")
    say("mlp c2 prefill T", T)
    y = lb.mlp_forward(x_to_dev(x), dev_layer(g), dev_layer(u), dev_layer(d), torch.bfloat16)
    torch.cuda.synchronize()
    tok = np.array([0, 31, 32, 63, 95])
    ref = oracle.mlp_forward(x[tok], g, u, d)
    assert_close(y_to_np(y)[tok], ref, TOL["bf16"], "mlp prefill")


def _stack_check(key, layers, T, check_layers, rows_per=512, tokens=None):
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    from binarized_rank_linear_amd.stack import LayerStack
    w = synth.WORKLOADS[key]
    kept = {}

    def make(L, i, di, do, rp, P):
        U, V, h, g, l = synth.device_layer(synth.layer_seed(L, i), di, do, rp, P)
        if L in check_layers:
            kept[(L, i)] = host_layer_from_dev(U, V, h, g, l)
        return U, V, h, g, l

    say("stack", key, layers, "T", T)
    st = LayerStack([(s.name, s.d_in, s.d_out) for s in w.linears], layers, w.b_num, w.b_den,
                    w.residual, make)
    widths = sorted({s.d_in for s in w.linears})
    xs = {d: synth.device_activations(synth.activation_seed(d), T, d, w.dtype) for d in widths}
    st.bind(T, xs, torch.bfloat16)
    st.group.run()
    torch.cuda.synchronize()
    for L in check_layers:
        for i, sh in enumerate(w.linears):
            inp = kept[(L, i)]
            x = xs[sh.d_in].float().cpu().numpy()
            tok = np.arange(T) if tokens is None else np.asarray(tokens)
            rows = np.unique(np.linspace(0, sh.d_out - 1, rows_per).astype(np.int64))
            ref = oracle.linear_forward_rows(x[tok], inp.U, inp.V, inp.h, inp.g, inp.l, rows)
            got = y_to_np(st.outputs[L][i])[tok][:, rows]
            assert_close(got, ref, TOL["bf16"], (key, L, sh.name))


@pytest.mark.parametrize("key,T", [("c3", 4), ("c4", 1), ("c5", 1), ("c3", 32)])
def test_small_stack_all_layers(key, T):
    _stack_check(key, 2, T, {0, 1})


@pytest.mark.parametrize("key,T", [("c5", 100), ("c4", 300), ("c3", 64), ("c5", 2048), ("c4", 1800), ("c3", 2000)])
def test_prefill_layer_group(key, T):
    """One decoder layer's linears as one GEMM-path group (one launch per
    stage for all seven), sampled tokens and rows; also at the prefill
    length (T = 2048) and with a partial last token tile (1800, 2000)."""
    _stack_check(key, 1, T, {0}, rows_per=256, tokens=[0, 1, T // 2, T - 2, T - 1])


@pytest.mark.parametrize("key,layers", [("c3", 32), ("c4", 40)])
def test_full_stack_sampled_layers(key, layers):
    """The 32-layer Llama2-7B-shaped and 40-layer Qwen3-14B-shaped stacks as
    the benchmark runs them (one group, T = 1, one launch per pass); layers 0,
    L/2 and L - 1 are checked against the oracle on sampled rows."""
    _stack_check(key, layers, 1, {0, layers // 2, layers - 1})


def test_full_c5_stack_sampled_layers():
    """The 80-layer Llama2-70B-shaped stack as the benchmark runs it (one
    group, T = 1); layers 0, 40 and 79 are checked on sampled rows."""
    _stack_check("c5", 80, 1, {0, 40, 79})


@pytest.mark.parametrize("key,T,out", [("c3", 3, "bf16"), ("c4", 9, "f32"), ("c3", 1, "f32")])
def test_group_run_matches_staged_run(key, T, out):
    """A whole-group run equals stage 1 then stage 2 bit for bit (the same
    kernels and summation order), also for runs enqueued back to back."""
    torch = torch_or_skip()
    from binarized_rank_linear_amd.stack import LayerStack
    w = synth.WORKLOADS[key]
    say("chunked group", key, "T", T, out)

    def make(L, i, di, do, rp, P):
        return synth.device_layer(synth.layer_seed(L, i) + 1000, di, do, rp, P)

    st = LayerStack([(s.name, s.d_in, s.d_out) for s in w.linears], 3, w.b_num, w.b_den, w.residual, make)
    widths = sorted({s.d_in for s in w.linears})
    xs = {d: synth.device_activations(synth.activation_seed(d) + 7, T, d, w.dtype) for d in widths}
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    st.bind(T, xs, odt)
    st.group.run_stage(1)
    st.group.run_stage(2)
    torch.cuda.synchronize()
    staged = [[y.clone() for y in row] for row in st.outputs]
    for row in st.outputs:
        for y in row:
            y.fill_(float("nan"))
    for _ in range(3):
        st.group.run()
    torch.cuda.synchronize()
    for L, row in enumerate(st.outputs):
        for i, y in enumerate(row):
            assert torch.equal(y.view(torch.int16) if odt == torch.bfloat16 else y.view(torch.int32),
                               staged[L][i].view(torch.int16) if odt == torch.bfloat16
                               else staged[L][i].view(torch.int32)), (L, i)
    st.group.release()


def _runs_match_staged(key, T, out, order):
    """Runs a 2-layer stack of the workload as one group with two sets of
    activations, loaded in `order` before each run, and checks every run
    against the staged run (stage 1 then stage 2) of its own inputs, bit for
    bit."""
    torch = torch_or_skip()
    from binarized_rank_linear_amd.stack import LayerStack
    w = synth.WORKLOADS[key]

    def make(L, i, di, do, rp, P):
        return synth.device_layer(synth.layer_seed(L, i) + 2000, di, do, rp, P)

    st = LayerStack([(s.name, s.d_in, s.d_out) for s in w.linears], 2, w.b_num, w.b_den, w.residual, make)
    widths = sorted({s.d_in for s in w.linears})
    src = [{d: synth.device_activations(synth.activation_seed(d) + 31 * k, T, d, w.dtype) for d in widths}
           for k in range(2)]
    xs = {d: src[0][d].clone() for d in widths}
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    st.bind(T, xs, odt)
    bits = (lambda y: y.view(torch.int16)) if odt == torch.bfloat16 else (lambda y: y.view(torch.int32))

    def load(k):
        for d in widths:
            xs[d].copy_(src[k][d])
        for row in st.outputs:
            for y in row:
                y.fill_(float("nan"))

    refs = []
    for k in range(2):
        load(k)
        st.group.run_stage(1)
        st.group.run_stage(2)
        torch.cuda.synchronize()
        refs.append([[y.clone() for y in row] for row in st.outputs])
    assert not torch.equal(bits(refs[0][0][0]), bits(refs[1][0][0]))
    for k in order:
        load(k)
        st.group.run()
        torch.cuda.synchronize()
        for L, row in enumerate(st.outputs):
            for i, y in enumerate(row):
                assert torch.equal(bits(y), bits(refs[k][L][i])), (k, L, i)
    st.group.release()


@pytest.mark.parametrize("key,T,out", [("c3", 1, "bf16"), ("c4", 1, "bf16"), ("c5", 1, "f32"), ("c3", 2, "bf16"),
                                       ("c5", 6, "bf16"), ("c5", 4, "f32")])
def test_pass_reads_each_runs_inputs(key, T, out):
    """The one-launch pass (bf16 T <= 2, fp32 T = 1) hands each run's latents
    to that run's stage 2: with other activations between runs, every run
    equals the staged run of its own inputs bit for bit (a stale hand-off
    would repeat the previous run's outputs).  Larger T runs three launches
    per run, checked the same way."""
    say("pass inputs", key, "T", T, out)
    _runs_match_staged(key, T, out, (0, 1, 1, 0, 1))


def test_pass_many_runs():
    """200 one-launch passes in a row (2-layer 80-layer-stack slice, T = 1),
    the two input sets in an irregular order: every run equals the staged run
    of its own inputs bit for bit (the hand-off between workgroups uses no
    cache-wide fence, so a stale operand would show as a repeated output)."""
    say("pass, 200 runs")
    _runs_match_staged("c5", 1, "bf16", tuple((k * 7 // 3 + k // 5) % 2 for k in range(200)))


# (d_in, d_out, r_p, P) per linear.  "mixed": ranks from 16 to 2000, some
# under 4 latent tiles of 64 (stage 1 splits K-groups among its waves);
# "wide": every rank at least 4 tiles (4 to 23), none a multiple of 64
# latents (stage 1 splits tiles among its waves).
RAGGED = {
    "mixed": [(1000, 700, 48, 2), (520, 130, 16, 1), (2048, 1536, 160, 2), (96, 1100, 32, 1),
              (1024, 333, 64, 2), (4096, 257, 304, 2), (1024, 512, 1696, 2), (640, 384, 2000, 1)],
    "wide": [(1000, 700, 304, 2), (520, 130, 208, 1), (2048, 1536, 416, 2), (600, 1100, 1456, 1),
             (1024, 333, 1040, 2)],
    # path ranks off the 16-multiple grid (none a multiple of 4): "odd" mixed
    # sizes, "odd_wide" every rank at least 4 latent tiles (the tile split)
    "odd": [(1000, 700, 17, 2), (520, 130, 6, 1), (2048, 1536, 150, 2), (96, 1100, 5, 2), (1024, 333, 1001, 2)],
    "odd_wide": [(1000, 700, 301, 2), (520, 130, 257, 1), (600, 1100, 1457, 1)],
}


@pytest.mark.parametrize("T,out,kind", [(1, "bf16", "mixed"), (2, "bf16", "mixed"), (5, "bf16", "mixed"),
                                        (8, "bf16", "mixed"), (1, "f32", "mixed"), (3, "f32", "mixed"),
                                        (1, "bf16", "wide"), (2, "bf16", "wide"), (6, "bf16", "wide"),
                                        (1, "f32", "wide"), (4, "f32", "wide"),
                                        (1, "bf16", "odd"), (2, "bf16", "odd"), (5, "bf16", "odd"),
                                        (1, "f32", "odd"), (3, "f32", "odd"), (12, "bf16", "odd"),
                                        (40, "bf16", "odd"), (1, "bf16", "odd_wide"), (2, "bf16", "odd_wide"),
                                        (6, "bf16", "odd_wide"), (1, "f32", "odd_wide"), (4, "f32", "odd_wide"),
                                        (24, "bf16", "odd_wide")])
def test_pass_ragged_mixed_group(T, out, kind):
    """A decode group of ragged linears, with and without the residual path
    (d_in, d_out and r_p off every tile size), runs as one launch per pass
    (bf16 T <= 2, fp32 T = 1; three launches beyond): every run equals the
    staged run bit for bit, and the oracle within the tolerance.  In the mixed
    set the last two ranks span two stage-1 latent groups per path at T = 1
    (more than 24 tiles of 64 latents), the second one ragged.  The odd sets
    take ranks that are not multiples of 4, also at 12 to 40 tokens (GEMM
    kernels)."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    say("pass ragged group T", T, out, kind)
    shapes = RAGGED[kind]
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    items, inps, xs = [], [], []
    for i, (d_in, d_out, r_p, P) in enumerate(shapes):
        inp = synth.layer_inputs(500 + i, d_in, d_out, r_p, P)
        x = synth.activations(600 + i, T, d_in, "bf16")
        y = torch.empty((T, d_out), dtype=odt, device="cuda")
        items.append((x_to_dev(x), y, dev_layer(inp)))
        inps.append(inp)
        xs.append(x)
    g = lb.Group(items, T, torch.bfloat16, odt)
    bits = (lambda y: y.view(torch.int16)) if odt == torch.bfloat16 else (lambda y: y.view(torch.int32))
    g.run_stage(1)
    g.run_stage(2)
    torch.cuda.synchronize()
    staged = [it[1].clone() for it in items]
    for _ in range(3):
        for it in items:
            it[1].fill_(float("nan"))
        g.run()
        torch.cuda.synchronize()
        for i, it in enumerate(items):
            assert torch.equal(bits(it[1]), bits(staged[i])), i
    for i, inp in enumerate(inps):
        xf = synth.bf16_bits_to_f32(xs[i]) if xs[i].dtype == np.uint16 else xs[i]
        ref = oracle.linear_forward(xf, inp.U, inp.V, inp.h, inp.g, inp.l)
        assert_close(y_to_np(items[i][1]), ref, TOL[out], ("ragged group", kind, T, i))
    g.release()


@pytest.mark.parametrize("T,kind", [(1, "mixed"), (2, "mixed"), (4, "mixed"), (1, "wide"), (2, "wide"),
                                    (6, "wide")])
def test_group_two_limb_exact_regime(T, kind):
    """Decode groups with bf16 outputs (two fp8 limbs) in the regime where two
    limbs are exact (integer g x with |g x| <= 4, integer |t| <= 128): every
    output of the one-launch pass (T <= 2) and of the three-launch form (T >= 4)
    equals the oracle rounded to bf16, bit for bit."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    from test_gpu_linear import _integer_layer, _sparse_x
    say("group exact two-limb T", T, kind)
    items, refs = [], []
    for i, (d_in, d_out, r_p, P) in enumerate(RAGGED[kind]):
        inp = _integer_layer(800 + i, d_in, d_out, r_p, P)
        x = _sparse_x(900 + i + T, T, d_in)
        refs.append(synth.f32_to_bf16_bits(oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l)
                                           .astype(np.float32)))
        y = torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda")
        items.append((x_to_dev(synth.f32_to_bf16_bits(x)), y, dev_layer(inp)))
    g = lb.Group(items, T, torch.bfloat16, torch.bfloat16)
    for _ in range(2):
        for it in items:
            it[1].fill_(float("nan"))
        g.run()
        torch.cuda.synchronize()
        for i, it in enumerate(items):
            y = it[1].cpu().view(torch.int16).numpy().view(np.uint16)
            bad = np.argwhere(y != refs[i])
            assert bad.size == 0, (i, bad[:4])
    assert lb.device_faults() == 0
    g.release()
