"""GPU tests of the group entry points: the stateless grouped call
(lb_linear_forward_grouped), the fault report (lb_device_faults), the
workspace stamp of prepared groups, and graph capture and replay."""
import numpy as np
import pytest

import synth
from gpu_util import say, torch_or_skip

pytestmark = pytest.mark.gpu


def _stack(key, layers, seed_off):
    from binarized_rank_linear_amd.stack import LayerStack
    w = synth.WORKLOADS[key]

    def make(L, i, di, do, rp, P):
        return synth.device_layer(synth.layer_seed(L, i) + seed_off, di, do, rp, P)

    return w, LayerStack([(s.name, s.d_in, s.d_out) for s in w.linears], layers, w.b_num, w.b_den,
                         w.residual, make)


def _inputs(w, T, salt):
    widths = sorted({s.d_in for s in w.linears})
    return {d: synth.device_activations(synth.activation_seed(d) + salt, T, d, w.dtype) for d in widths}


def _bits(torch, y):
    return y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)


def _items(st, xs, torch, odt, T):
    return [(xs[lin.d_in], torch.empty((T, lin.d_out), dtype=odt, device="cuda"), lin)
            for row in st.linears for lin in row]


@pytest.mark.parametrize("key,T,out", [("c5", 1, "bf16"), ("c3", 1, "f32"), ("c3", 4, "bf16"),
                                       ("c5", 2, "bf16"), ("c4", 64, "bf16")])
def test_stateless_grouped_equals_prepared(key, T, out):
    """lb_linear_forward_grouped with no prior set-up gives every output bit
    for bit as the prepared group of the same linears (the same kernels and
    summation order): the one-launch pass (T = 1, 2), three launches (T = 4)
    and the GEMM kernels (T = 64).  The second and third calls reuse the
    cached plan, the third with other activations."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    lb.device_faults()
    say("stateless grouped", key, "T", T, out)
    w, st = _stack(key, 2, 3000)
    odt = torch.bfloat16 if out == "bf16" else torch.float32
    xs = _inputs(w, T, 11)
    st.bind(T, xs, odt)
    items = _items(st, xs, torch, odt, T)
    for rep in range(3):
        if rep == 2:
            for d, x in _inputs(w, T, 77).items():
                xs[d].copy_(x)
        st.group.run()
        torch.cuda.synchronize()
        ref = [y.clone() for row in st.outputs for y in row]
        for it in items:
            it[1].fill_(float("nan"))
        lb.linear_forward_grouped(items)
        torch.cuda.synchronize()
        for i, it in enumerate(items):
            assert torch.equal(_bits(torch, it[1]), _bits(torch, ref[i])), (rep, i)
    assert lb.device_faults() == 0
    st.group.release()


def test_stateless_mixed_subgroups():
    """One grouped call holding linears at T = 1 (bf16 out) and T = 3 (fp32
    out), interleaved: it runs as two groups, each equal bit for bit to the
    prepared group of its own linears."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    say("stateless mixed sub-groups")
    w, st = _stack("c5", 1, 3100)
    xa, xb = _inputs(w, 1, 5), _inputs(w, 3, 6)
    lins = st.linears[0]
    ia = [(xa[l.d_in], torch.empty((1, l.d_out), dtype=torch.bfloat16, device="cuda"), l) for l in lins]
    ib = [(xb[l.d_in], torch.empty((3, l.d_out), dtype=torch.float32, device="cuda"), l) for l in lins]
    ga = lb.Group([(x, torch.empty_like(y), l) for x, y, l in ia], 1, torch.bfloat16, torch.bfloat16)
    gb = lb.Group([(x, torch.empty_like(y), l) for x, y, l in ib], 3, torch.bfloat16, torch.float32)
    ga.run()
    gb.run()
    mixed = [it for pair in zip(ia, ib) for it in pair]
    lb.linear_forward_grouped(mixed)
    torch.cuda.synchronize()
    for i in range(len(lins)):
        assert torch.equal(_bits(torch, ia[i][1]), _bits(torch, ga.items[i][1])), ("T=1", i)
        assert torch.equal(_bits(torch, ib[i][1]), _bits(torch, gb.items[i][1])), ("T=3", i)
    ga.release()
    gb.release()


def test_handoff_timeout_is_reported():
    """LB_GROUP_FAULT_TEST makes every stage-2 wait of the one-launch pass ask
    for one latent group more than exists and give up after a few polls: each
    run reports LB_FAULT_HANDOFF_TIMEOUT (a bounded wait, so every kernel ends).
    Normal runs of the same linears afterwards report nothing and equal their
    staged runs bit for bit."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    lb.device_faults()
    say("hand-off timeout report")
    w, st = _stack("c5", 2, 3200)
    xs = _inputs(w, 1, 21)
    items = _items(st, xs, torch, torch.bfloat16, 1)
    bad = lb.Group(items, 1, torch.bfloat16, torch.bfloat16, lb.LB_GROUP_FAULT_TEST)
    for _ in range(3):
        bad.run()
        assert lb.device_faults() & lb.LB_FAULT_HANDOFF_TIMEOUT
    bad.release()
    for _ in range(2):      # the stateless form of the same test
        lb.linear_forward_grouped(items, lb.LB_GROUP_FAULT_TEST)
        assert lb.device_faults() & lb.LB_FAULT_HANDOFF_TIMEOUT
    good = lb.Group(items, 1, torch.bfloat16, torch.bfloat16)
    good.run_stage(1)
    good.run_stage(2)
    torch.cuda.synchronize()
    ref = [it[1].clone() for it in items]
    for _ in range(3):
        for it in items:
            it[1].fill_(float("nan"))
        good.run()
        assert lb.device_faults() == 0
        for i, it in enumerate(items):
            assert torch.equal(_bits(torch, it[1]), _bits(torch, ref[i])), i
    good.release()


@pytest.mark.parametrize("key,T", [("c5", 1), ("c3", 4), ("c4", 64)])
def test_stale_workspace_is_reported(key, T):
    """A prepared group whose workspace stamp was overwritten (as when its
    memory is reused without a new prepare) does nothing and reports
    LB_FAULT_STALE_WORKSPACE; preparing it again restores normal runs."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    lb.device_faults()
    say("stale workspace", key, "T", T)
    w, st = _stack(key, 1, 3300)
    xs = _inputs(w, T, 31)
    st.bind(T, xs, torch.bfloat16)
    g = st.group
    g.run()
    torch.cuda.synchronize()
    ref = [y.clone() for y in st.outputs[0]]
    assert lb.device_faults() == 0
    for y in st.outputs[0]:
        y.fill_(float("nan"))
    g.ws[:8].zero_()
    g.run()
    assert lb.device_faults() & lb.LB_FAULT_STALE_WORKSPACE
    for y in st.outputs[0]:
        assert torch.isnan(y.float()).all()
    g.release()
    st.bind(T, xs, torch.bfloat16)
    st.group.run()
    assert lb.device_faults() == 0
    for i, y in enumerate(st.outputs[0]):
        assert torch.equal(_bits(torch, y), _bits(torch, ref[i])), i
    st.group.release()


@pytest.mark.parametrize("form", ["prepared", "stateless"])
def test_graph_replay_reads_each_replays_inputs(form):
    """A one-launch pass captured in a graph and replayed with other
    activations between replays (and eager work in between): every replay
    equals the staged run of its own inputs bit for bit (the hand-off counters
    return to zero at the end of each run, so a replay starts like a fresh
    run).  The stateless form replays its table copy and counter clear too."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    lb.device_faults()
    say("graph replay", form)
    w, st = _stack("c5", 2, 3400)
    srcs = [_inputs(w, 1, 41 + k) for k in range(2)]
    xs = {d: srcs[0][d].clone() for d in srcs[0]}
    st.bind(1, xs, torch.bfloat16)
    outs = [y for row in st.outputs for y in row]

    def load(k):
        for d in xs:
            xs[d].copy_(srcs[k][d])
        for y in outs:
            y.fill_(float("nan"))

    refs = []
    for k in range(2):
        load(k)
        st.group.run_stage(1)
        st.group.run_stage(2)
        torch.cuda.synchronize()
        refs.append([y.clone() for y in outs])
    items = [(xs[lin.d_in], y, lin) for (row, yr) in zip(st.linears, st.outputs) for lin, y in zip(row, yr)]
    ws = lb.workspace(lb.grouped_workspace_bytes(items))
    run = (lambda: st.group.run()) if form == "prepared" else (lambda: lb.linear_forward_grouped(items, ws=ws))
    run()                      # eager first (one-time attributes), then capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for k in (0, 1, 1, 0, 1, 0):
        load(k)
        graph.replay()
        torch.cuda.synchronize()
        for i, y in enumerate(outs):
            assert torch.equal(_bits(torch, y), _bits(torch, refs[k][i])), (k, i)
        assert lb.device_faults() == 0
    st.group.release()
