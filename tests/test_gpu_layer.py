"""GPU parity of one decoder layer at decode time (lb_decoder_layer_forward):
two RMSNorms, q/k/v as one group, attention over a one-token context with
grouped kv heads, o with the residual, the SwiGLU MLP with the residual,
against the oracle's fp64 composition of its linears."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, assert_close, host_layer_from_dev, say, torch_or_skip, x_to_dev, y_to_np

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "o", "gate", "up", "down")


def _layer(seed, d, ff, dkv, rps, P=2):
    """Device-drawn factors (l scaled for unit gain, so layers chain) and
    their host copies for the oracle.  rps: r_p of (q/o, k/v, gate/up, down)."""
    import binarized_rank_linear_amd as lb
    shapes = dict(q=(d, d, rps[0]), k=(d, dkv, rps[1]), v=(d, dkv, rps[1]), o=(d, d, rps[0]),
                  gate=(d, ff, rps[2]), up=(d, ff, rps[2]), down=(ff, d, rps[3]))
    dev, host = {}, {}
    for i, name in enumerate(NAMES):
        di, do, rp = shapes[name]
        U, V, h, g, l = synth.device_layer(synth.layer_seed(seed, i), di, do, rp, P)
        l = (l.float() * synth.unit_gain_l(di, rp, P)).half()
        host[name] = host_layer_from_dev(U, V, h, g, l)
        dev[name] = lb.PackedLinear.from_factors(U, V, h, g, l)
    return dev, host


def _decoder(dev, n_heads, n_kv, eps):
    import binarized_rank_linear_amd as lb
    return lb.DecoderLayer(*(dev[n] for n in NAMES), n_heads=n_heads, n_kv_heads=n_kv, eps=eps)


def _budget_rps(key):
    w = synth.WORKLOADS[key]
    sh = {s.name: s for s in w.linears}
    rp = lambda n: oracle.rank_for_budget(sh[n].d_in, sh[n].d_out, w.b_num, w.b_den, w.residual)[1]
    return (rp("q"), rp("k"), rp("gate"), rp("down")), sh


@pytest.mark.parametrize("T", [1, 3, 8, 17, 32])
def test_decoder_layer_ragged_gqa(T):
    """Widths that are not multiples of 8 (d_model 520 with 8 heads of 65,
    2 kv heads; d_ff 1100), every T the decode kernels take, including the
    fused (T <= 8) and separate stage-1 forms."""
    torch = torch_or_skip()
    dev, host = _layer(3, 520, 1100, 130, (48, 32, 64, 48))
    x = synth.activations(40 + T, T, 520, "bf16")
    say("decoder layer 520/1100 gqa 8:2 T", T)
    y = _decoder(dev, 8, 2, 1e-6).forward(x_to_dev(x))
    torch.cuda.synchronize()
    ref = oracle.decoder_layer_forward(x, host, 8, 2, 1e-6)
    assert_close(y_to_np(y), ref, TOL["bf16"], ("layer ragged", T))


@pytest.mark.parametrize("T", [1, 2, 5, 12, 32])
def test_decoder_layer_odd_ranks(T):
    """Path ranks that are not multiples of 4 (17, 6, 30 and 21 for q/o, k/v,
    gate/up and down) through every step of the layer, with the fused (T <= 8)
    and separate stage-1 forms."""
    torch = torch_or_skip()
    dev, host = _layer(5, 520, 1100, 130, (17, 6, 30, 21))
    x = synth.activations(60 + T, T, 520, "bf16")
    say("decoder layer odd ranks T", T)
    y = _decoder(dev, 8, 2, 1e-6).forward(x_to_dev(x))
    torch.cuda.synchronize()
    ref = oracle.decoder_layer_forward(x, host, 8, 2, 1e-6)
    assert_close(y_to_np(y), ref, TOL["bf16"], ("layer odd ranks", T))


@pytest.mark.parametrize("T", [1, 4])
def test_decoder_layer_llama2_7b_shape(T):
    """A Llama2-7B-shaped layer (4096, 11008, 32 heads, no kv grouping) at
    1.0 bpw with the residual path."""
    torch = torch_or_skip()
    rps, sh = _budget_rps("c3")
    dev, host = _layer(5, 4096, 11008, 4096, rps)
    x = synth.activations(50 + T, T, 4096, "bf16")
    say("decoder layer c3 shape T", T, "r_p", rps)
    y = _decoder(dev, 32, 32, 1e-5).forward(x_to_dev(x))
    torch.cuda.synchronize()
    ref = oracle.decoder_layer_forward(x, host, 32, 32, 1e-5)
    assert_close(y_to_np(y), ref, TOL["bf16"], ("layer c3", T))


@pytest.mark.parametrize("T", [1, 2])
def test_decoder_layer_llama2_70b_shape(T):
    """A Llama2-70B-shaped layer (8192, 28672, 64 heads over 8 kv heads of
    128) at 0.1 bpw with the residual path."""
    torch = torch_or_skip()
    rps, sh = _budget_rps("c5")
    dev, host = _layer(6, 8192, 28672, 1024, rps)
    x = synth.activations(60 + T, T, 8192, "bf16")
    say("decoder layer c5 shape T", T, "r_p", rps)
    y = _decoder(dev, 64, 8, 1e-5).forward(x_to_dev(x))
    torch.cuda.synchronize()
    ref = oracle.decoder_layer_forward(x, host, 64, 8, 1e-5)
    assert_close(y_to_np(y), ref, TOL["bf16"], ("layer c5", T))


def test_decoder_layers_chained_and_graph_replayed():
    """Three layers chained (each one's y the next one's x) in eager order and
    as one captured HIP graph replayed three times with eager work between
    the replays; every replay equals the eager result bit for bit, and the
    chain matches the oracle's chain with its hand-offs kept in bf16."""
    torch = torch_or_skip()
    layers = [_layer(10 + i, 256, 704, 64, (32, 32, 64, 32)) for i in range(3)]
    decs = [_decoder(d, 4, 1, 1e-6) for d, _ in layers]
    T = 2
    x = synth.activations(77, T, 256, "bf16")
    xd = x_to_dev(x)
    say("decoder chain of 3, T", T)
    ws = torch.empty(max(d.workspace_bytes(T) for d in decs), dtype=torch.uint8, device="cuda")
    bufs = [torch.empty_like(xd) for _ in range(3)]

    def chain():
        cur = xd
        for d, b in zip(decs, bufs):
            d.forward(cur, out=b, ws=ws, stream=torch.cuda.current_stream())
            cur = b
        return cur

    eager = chain().clone()
    torch.cuda.synchronize()
    ref = x
    for _, host in layers:
        ref = oracle.decoder_layer_forward(ref, host, 4, 1, 1e-6, store=oracle.round_bf16)
    assert_close(y_to_np(eager), ref, TOL["bf16"], "chain")

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            chain()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        bufs[2].fill_(0)
        _ = (xd.float() * 2).sum()                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bufs[2], eager), ("replay", rep)


def test_decoder_layer_empty_and_errors():
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    dev, _ = _layer(12, 128, 256, 64, (32, 32, 32, 32))
    dec = _decoder(dev, 4, 2, 1e-6)
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    say("decoder layer T=0 and argument errors")
    assert dec.forward(x).shape == (0, 128)
    assert dec.workspace_bytes(0) == 0 and dec.workspace_bytes(33) == 0
    with pytest.raises(lb.LBError) as e:
        dec.forward(torch.zeros((33, 128), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == lb.LB_EUNSUPPORTED
    bad = lb.DecoderLayer(*(dev[n] for n in NAMES), n_heads=3, n_kv_heads=1)     # 128 % 3 != 0
    with pytest.raises(lb.LBError) as e:
        bad.forward(torch.zeros((1, 128), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == lb.LB_EINVAL
    xs = torch.zeros((2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lb.LBError) as e:
        dec.forward(xs, out=xs)
    assert e.value.status == lb.LB_EINVAL
