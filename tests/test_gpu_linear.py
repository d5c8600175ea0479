"""GPU parity of lb_linear_forward against the fp64 oracle.

Tolerances (relative L2 over the whole output, or over the sampled outputs):
1e-3 for fp32 outputs and 8e-3 for bf16 outputs.  In the exact-integer
regimes every partial sum is exactly representable, so the GPU must match the
oracle bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, assert_close, dev_layer, dev_layer_ld, say, torch_or_skip, x_to_dev, y_to_np

pytestmark = pytest.mark.gpu

DECODE_PATHS = ["valu", "decode"]
PATH_FLAG = {"auto": 0, "decode": 1, "prefill": 2, "valu": 3}


def _run(inp, x, out_dtype, path, T):
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    layer = dev_layer(inp)
    xd = x_to_dev(x)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    say("linear", inp.d_in, inp.d_out, inp.r_path, inp.paths, "T", T, out_dtype, path)
    y = lb.linear_forward(xd, layer, od, PATH_FLAG[path])
    torch.cuda.synchronize()
    return y


def _check(inp, x, out_dtype, path, rows=None, tokens=None):
    T = x.shape[0]
    y = y_to_np(_run(inp, x, out_dtype, path, T))
    xs = x if tokens is None else x[tokens]
    if rows is None:
        ref = oracle.linear_forward(xs, inp.U, inp.V, inp.h, inp.g, inp.l)
        got = y if tokens is None else y[tokens]
    else:
        ref = oracle.linear_forward_rows(xs, inp.U, inp.V, inp.h, inp.g, inp.l, rows)
        got = (y if tokens is None else y[tokens])[:, rows]
    return assert_close(got, ref, TOL[out_dtype], (inp.d_in, inp.d_out, inp.r_path, T, out_dtype, path))


# ---- configuration 1: 1024 x 1024, 1.0 bpw -> r = 512, no residual, fp32 ----

@pytest.mark.parametrize("T", [1, 8])
@pytest.mark.parametrize("path", ["auto", "valu", "decode"])
def test_config1_single_linear(T, path):
    r, rp = oracle.rank_for_budget(1024, 1024, 1, 1, False)
    inp = synth.layer_inputs(0, 1024, 1024, rp, 1)
    x = synth.activations(synth.activation_seed(0), T, 1024, "f32")
    _check(inp, x, "f32", path)


# ---- ragged shapes spanning several tiles ----

@pytest.mark.parametrize("d_in,d_out,r_p,P", [(1000, 1100, 48, 2), (100, 70, 16, 2),
                                              (96, 1, 32, 1), (2080, 515, 200, 2),
                                              (32, 4096, 8, 1)])
@pytest.mark.parametrize("T", [1, 3, 17, 32])
@pytest.mark.parametrize("path", DECODE_PATHS)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ragged_shapes(d_in, d_out, r_p, P, T, path, dt):
    inp = synth.layer_inputs(d_in + d_out, d_in, d_out, r_p, P)
    x = synth.activations(T + d_in, T, d_in, dt)
    _check(inp, x, dt, path)


@pytest.mark.parametrize("T", [33, 100])
def test_more_tokens_than_decode_width_fp32(T):
    """fp32 outputs above 32 tokens run the plain decode kernels in chunks."""
    inp = synth.layer_inputs(5, 512, 384, 64, 2)
    x = synth.activations(6, T, 512, "f32")
    _check(inp, x, "f32", "auto")


@pytest.mark.parametrize("d_in,d_out,r_p,P", [(1000, 700, 48, 2), (520, 130, 16, 1),
                                              (9000, 300, 96, 2), (100, 70, 16, 2),
                                              (2048, 1100, 304, 2)])
@pytest.mark.parametrize("T", [5, 20, 32, 33, 100, 257])
@pytest.mark.parametrize("xdt", ["bf16", "f32"])
def test_prefill_ragged(d_in, d_out, r_p, P, T, xdt):
    """GEMM path over ragged tiles: token and column tails, a K tail (d_in % 64),
    two d_in pieces (9000 > 8192), a path boundary inside a packed word
    (r_p = 304), fp32 inputs rounded to bf16 on staging; every token-tile size
    (32, 64, 128 and 256/128 tokens); d_in = 100 is not a multiple of 8 and
    runs on the vector-ALU kernels."""
    inp = synth.layer_inputs(d_in + 3 * d_out, d_in, d_out, r_p, P)
    x = synth.activations(T + 7 * d_in, T, d_in, xdt)
    _check(inp, x, "bf16", "prefill")


# ---- the configurations' linears at full size ----

def _cfg_linear(key, name):
    w = synth.WORKLOADS[key]
    sh = [s for s in w.linears if s.name == name][0]
    r, rp = oracle.rank_for_budget(sh.d_in, sh.d_out, w.b_num, w.b_den, w.residual)
    inp = synth.layer_inputs(w.linears.index(sh), sh.d_in, sh.d_out, rp, 2 if w.residual else 1)
    return w, sh, inp


@pytest.mark.parametrize("key,name,T", [
    ("c3", "q", 1), ("c3", "q", 4), ("c3", "q", 32), ("c3", "gate", 1), ("c3", "gate", 4),
    ("c3", "down", 1), ("c3", "down", 32),
    ("c4", "q", 1), ("c4", "k", 1), ("c4", "gate", 1), ("c4", "down", 1),
    ("c5", "q", 1), ("c5", "k", 1), ("c5", "gate", 1), ("c5", "down", 1), ("c5", "down", 4)])
@pytest.mark.parametrize("path", ["auto", "valu"])
def test_config_linears_decode(key, name, T, path):
    w, sh, inp = _cfg_linear(key, name)
    x = synth.activations(synth.activation_seed(T), T, sh.d_in, w.dtype)
    rows = None if sh.d_out * T <= 8192 * 4 else np.linspace(0, sh.d_out - 1, 2048).astype(np.int64)
    _check(inp, x, w.dtype, path, rows=rows)


@pytest.mark.parametrize("key,name,T", [("c3", "q", 20), ("c3", "q", 32), ("c3", "down", 32), ("c5", "gate", 24)])
def test_config_linears_decode_kernels_above_16(key, name, T):
    """The decode kernels keep serving 17 to 32 tokens when asked for (AUTO
    takes the GEMM kernels there for bf16 outputs)."""
    w, sh, inp = _cfg_linear(key, name)
    x = synth.activations(synth.activation_seed(T), T, sh.d_in, w.dtype)
    rows = None if sh.d_out * T <= 8192 * 4 else np.linspace(0, sh.d_out - 1, 2048).astype(np.int64)
    _check(inp, x, w.dtype, "decode", rows=rows)


@pytest.mark.parametrize("key,name", [("c4", "q"), ("c4", "k"), ("c4", "gate"), ("c4", "down"),
                                      ("c5", "q"), ("c5", "k"), ("c5", "gate"), ("c5", "down")])
def test_config_linears_prefill_sampled(key, name):
    """T = 2048 through the GEMM path; checked on 24 sampled tokens x 1024 sampled rows."""
    w, sh, inp = _cfg_linear(key, name)
    T = 2048
    x = synth.activations(synth.activation_seed(T), T, sh.d_in, w.dtype)
    tokens = np.array([0, 1, 2, 63, 64, 127, 128, 255, 256, 511, 777, 1023, 1024, 1200, 1500,
                       1791, 1792, 1919, 2000, 2040, 2044, 2045, 2046, 2047])
    rows = np.unique(np.linspace(0, sh.d_out - 1, 1024).astype(np.int64))
    _check(inp, x, w.dtype, "auto", rows=rows, tokens=tokens)


# ---- exact regimes ----

def _pow2(rng, shape, lo=-1, hi=1):
    return synth.f16_bits(2.0 ** rng.integers(lo, hi + 1, shape))


@pytest.mark.parametrize("path", DECODE_PATHS + ["prefill"])
def test_exact_integer_regime_bit_exact(path):
    """x in {-1, 0, 1}, power-of-two scales: every partial sum is an exact
    small dyadic number, so fp32 output equals the oracle bit for bit (bf16
    output for the GEMM path equals the oracle rounded to bf16)."""
    rng = np.random.default_rng(1)
    P, d_in, d_out, r_p, T = 2, 1024, 700, 96, (64 if path == "prefill" else 5)
    base = synth.layer_inputs(9, d_in, d_out, r_p, P)
    inp = synth.LayerInputs(d_in, d_out, r_p, P, base.U, base.V, _pow2(rng, (P, d_out)),
                            _pow2(rng, (P, d_in), 0, 0), _pow2(rng, (P, r_p)))
    x = rng.integers(-1, 2, (T, d_in)).astype(np.float32)
    ref = oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l)
    if path == "prefill":
        xb = synth.f32_to_bf16_bits(x)
        y = _run(inp, xb, "bf16", path, T).cpu().view(__import__("torch").int16).numpy().view(np.uint16)
        assert np.array_equal(y, synth.f32_to_bf16_bits(ref.astype(np.float32)))
    else:
        y = _run(inp, x, "f32", path, T).cpu().numpy()
        assert np.array_equal(y.astype(np.float64), ref)


def _hadamard(n):
    i = np.arange(n)
    par = np.array([[bin(a & b).count("1") & 1 for b in i] for a in i])
    return np.where(par == 1, -1.0, 1.0).astype(np.float32)


@pytest.mark.parametrize("path,n,xmax", [("valu", 1024, 15), ("valu", 256, 15),
                                         ("decode", 256, 1), ("decode", 64, 3)])
def test_hadamard_closed_form_bit_exact(path, n, xmax):
    """S_U = S_V = H_n, l = 1/n: W = diag(h*g), so y = h*g*x exactly,
    independently of the oracle."""
    rng = np.random.default_rng(n)
    H = _hadamard(n)[None]
    h = _pow2(rng, (1, n), -1, 1)
    g = _pow2(rng, (1, n), 0, 0) if xmax == 1 else _pow2(rng, (1, n), -1, 1)
    l = synth.f16_bits(np.full((1, n), 1.0 / n))
    inp = synth.LayerInputs(n, n, n, 1, H, H, h, g, l)
    x = rng.integers(-xmax, xmax + 1, (4, n)).astype(np.float32)
    y = _run(inp, x, "f32", path, 4).cpu().numpy()
    want = x * (oracle.widen_f16(h[0]) * oracle.widen_f16(g[0]))[None, :]
    assert np.array_equal(y.astype(np.float64), want)


@pytest.mark.parametrize("path", DECODE_PATHS)
def test_invariants_bit_exact(path):
    torch = torch_or_skip()
    inp = synth.layer_inputs(21, 640, 900, 80, 2)
    x = synth.activations(22, 6, 640, "f32")
    y = _run(inp, x, "f32", path, 6).cpu().numpy()
    # odd in x
    yn = _run(inp, -x, "f32", path, 6).cpu().numpy()
    assert np.array_equal(yn, -y)
    # (2h, l/2) leaves y unchanged
    h2 = synth.f16_bits(oracle.widen_f16(inp.h) * 2)
    l2 = synth.f16_bits(oracle.widen_f16(inp.l) / 2)
    inp2 = synth.LayerInputs(inp.d_in, inp.d_out, inp.r_path, 2, inp.U, inp.V, h2, inp.g, l2)
    assert np.array_equal(_run(inp2, x, "f32", path, 6).cpu().numpy(), y)
    # flipping latent column 5 of both factors leaves y unchanged
    U, V = inp.U.copy(), inp.V.copy()
    U[:, :, 5] *= -1
    V[:, :, 5] *= -1
    inp3 = synth.LayerInputs(inp.d_in, inp.d_out, inp.r_path, 2, U, V, inp.h, inp.g, inp.l)
    assert np.array_equal(_run(inp3, x, "f32", path, 6).cpu().numpy(), y)
    # residual path equal to the first doubles the single-path output
    one = synth.LayerInputs(inp.d_in, inp.d_out, inp.r_path, 1, inp.U[:1], inp.V[:1], inp.h[:1],
                            inp.g[:1], inp.l[:1])
    dup = synth.LayerInputs(inp.d_in, inp.d_out, inp.r_path, 2, inp.U[[0, 0]], inp.V[[0, 0]],
                            inp.h[[0, 0]], inp.g[[0, 0]], inp.l[[0, 0]])
    y1 = _run(one, x, "f32", path, 6).cpu().numpy()
    assert np.array_equal(_run(dup, x, "f32", path, 6).cpu().numpy(), 2 * y1)


def test_zero_tokens_is_a_noop():
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    inp = synth.layer_inputs(3, 256, 128, 32, 2)
    layer = dev_layer(inp)
    x = torch.empty((0, 256), device="cuda")
    y = lb.linear_forward(x, layer, torch.float32)
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


@pytest.mark.parametrize("path", ["decode", "prefill"])
def test_decode_and_prefill_agree(path):
    """The same bf16 request through both kernel families, both near the oracle."""
    inp = synth.layer_inputs(40, 2048, 1536, 160, 2)
    x = synth.activations(41, 32, 2048, "bf16")
    _check(inp, x, "bf16", path)


def _integer_layer(seed, d_in, d_out, r_p, P):
    """Random signs with integer-friendly scales: g, l in {1, 2}, h in {1/2, 1, 2}."""
    rng = np.random.default_rng(seed)
    base = synth.layer_inputs(seed, d_in, d_out, r_p, P)
    return synth.LayerInputs(d_in, d_out, r_p, P, base.U, base.V, _pow2(rng, (P, d_out), -1, 1),
                             _pow2(rng, (P, d_in), 0, 1), _pow2(rng, (P, r_p), 0, 1))


def _sparse_x(seed, T, d_in, nnz=16):
    """x in {-2..2}, at most nnz non-zeros per token: |g x| <= 4, |t| <= 2 * 4 * nnz = 128."""
    rng = np.random.default_rng(seed)
    x = np.zeros((T, d_in), np.float32)
    for n in range(T):
        idx = rng.choice(d_in, size=min(nnz, d_in), replace=False)
        x[n, idx] = rng.integers(-2, 3, idx.size)
    return x


@pytest.mark.parametrize("d_in,d_out,r_p,P", [(1024, 700, 96, 2), (2080, 515, 200, 2), (96, 1100, 32, 1),
                                              (4096, 4096, 1024, 2)])
@pytest.mark.parametrize("T", [1, 2, 5])
def test_two_limb_decode_exact_regime_bit_exact(d_in, d_out, r_p, P, T):
    """The bf16-output decode path (two fp8 limbs per activation) in a regime
    where two limbs are exact: g x integers with |g x| <= 4 (one limb), t an
    integer with |t| <= 128 (an integer below 256 is the sum of its nearest
    e4m3 value and an e4m3 remainder, with the block's power-of-two scale), so
    every partial sum is exact and the bf16 output equals the oracle rounded
    to bf16 (nearest even) bit for bit."""
    inp = _integer_layer(50 + T + d_in, d_in, d_out, r_p, P)
    x = _sparse_x(60 + T, T, d_in)
    ref = oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l)
    xb = synth.f32_to_bf16_bits(x)
    y = _run(inp, xb, "bf16", "decode", T).cpu().view(__import__("torch").int16).numpy().view(np.uint16)
    want = synth.f32_to_bf16_bits(ref.astype(np.float32))
    bad = np.argwhere(y != want)
    assert bad.size == 0, (bad[:4], y[tuple(bad[0])], want[tuple(bad[0])])


@pytest.mark.parametrize("path,T,dt", [("decode", 1, "bf16"), ("decode", 4, "bf16"), ("decode", 1, "f32"),
                                       ("decode", 3, "f32"), ("valu", 2, "bf16"), ("prefill", 64, "bf16")])
def test_outlier_activations(path, T, dt):
    """A few input channels 100x larger than the rest (the activation outliers
    of real models): each 32-input block shares one power-of-two limb scale
    on the decode path, and the limbs are floating point, so the small inputs
    beside an outlier keep their own precision.  Within tolerance, and every
    element within the per-element bound."""
    d_in, d_out, r_p, P = 4096, 1536, 160, 2
    inp = synth.layer_inputs(71, d_in, d_out, r_p, P)
    x = synth.activations(72, T, d_in, "f32")
    rng = np.random.default_rng(73)
    ch = rng.choice(d_in, size=12, replace=False)
    x[:, ch] *= 100.0
    if dt == "bf16":
        x = synth.f32_to_bf16_bits(x)
    _check(inp, x, dt, path)


# ---- stage-1 pieces of a prepared group ----

@pytest.mark.parametrize("d_in,d_out,r_p,P,T", [(16384, 1024, 128, 2, 500), (28672, 1536, 304, 2, 2048),
                                                (9000, 300, 96, 1, 100)])
def test_prefill_pieces_group_equals_single(d_in, d_out, r_p, P, T):
    """A group of one long-d_in linear on the GEMM kernels: stage 1 splits
    d_in into pieces (up to 32 here) that a reduce launch adds in piece order;
    the single-linear call plans the same split.  Every run of the prepared
    group, with other inputs in between, equals the single call on its own
    inputs bit for bit, and the oracle on sampled tokens and rows."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    inp = synth.layer_inputs(d_in + 5 * d_out + r_p, d_in, d_out, r_p, P)
    layer = dev_layer(inp)
    xh = [synth.activations(T + 11 * k + d_in, T, d_in, "bf16") for k in range(2)]
    xs = [x_to_dev(x) for x in xh]
    say("pieces", d_in, d_out, r_p, P, "T", T)
    refs = [lb.linear_forward(x, layer, torch.bfloat16, PATH_FLAG["prefill"]) for x in xs]
    x = xs[0].clone()
    y = torch.empty(T, d_out, dtype=torch.bfloat16, device="cuda")
    grp = lb.Group([(x, y, layer)], T, torch.bfloat16, torch.bfloat16, PATH_FLAG["prefill"])
    torch.cuda.synchronize()
    assert not torch.equal(refs[0].view(torch.int16), refs[1].view(torch.int16))
    for k in (0, 1, 1, 0):
        x.copy_(xs[k])
        y.fill_(float("nan"))
        grp.run()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), refs[k].view(torch.int16)), k
    grp.release()
    tokens = np.unique(np.array([0, 1, T // 2, T - 2, T - 1]))
    rows = np.unique(np.linspace(0, d_out - 1, 256).astype(np.int64))
    ref = oracle.linear_forward_rows(xh[0][tokens], inp.U, inp.V, inp.h, inp.g, inp.l, rows)
    assert_close(y_to_np(refs[0])[tokens][:, rows], ref, TOL["bf16"], ("pieces", d_in, T))


@pytest.mark.parametrize("d_in,d_out,r_p,P,T", [(1000, 700, 17, 2, 40), (520, 130, 6, 1, 100), (9000, 300, 30, 2, 64),
                                                (256, 96, 2, 2, 300), (2048, 1100, 21, 1, 257), (16384, 200, 5, 2, 20)])
def test_prefill_ranks_off_the_rank_grid(d_in, d_out, r_p, P, T):
    """GEMM path with path ranks that the bit-budget rule never gives (not
    multiples of 16, most not of 4): the run of 4 latent columns that crosses
    r_p takes l = 0 past it, so the padding latents of t stay zero and add
    nothing in stage 2; unsplit and split d_in (9000, 16384), every token-tile
    size."""
    inp = synth.layer_inputs(d_in + 7 * d_out + r_p, d_in, d_out, r_p, P)
    x = synth.activations(T + 13 * d_in, T, d_in, "bf16")
    _check(inp, x, "bf16", "prefill")


# ---- the largest d_in the kernels take ----

_BIG_D_IN = (1 << 21) - 64          # the GEMM kernels take d_in below 2^21


@pytest.fixture(scope="module")
def big_d_in_layer():
    return synth.layer_inputs(2 ** 21, _BIG_D_IN, 80, 16, 2)


@pytest.mark.parametrize("path,T", [("decode", 1), ("decode", 3), ("valu", 1), ("prefill", 40)])
def test_largest_d_in(big_d_in_layer, path, T):
    """d_in just under the GEMM kernels' limit (2^21 - 64, 4 MB of V planes
    per path at r_p = 16): the decode kernels sum about 512 stage-1 chunk
    partials per latent, the GEMM kernels split d_in into their largest number
    of pieces, and the 32-bit buffer offsets over x (168 MB at T = 40) and over
    the planes stay in range; sampled tokens against the oracle."""
    inp = big_d_in_layer
    x = synth.activations(T + 5, T, _BIG_D_IN, "bf16")
    tokens = None if T <= 3 else np.array([0, 17, T - 1])
    _check(inp, x, "bf16", path, tokens=tokens)


# ---- caller-chosen strides of the packed factors ----

@pytest.mark.parametrize("path,T", [("decode", 1), ("decode", 4), ("decode", 24), ("valu", 2), ("valu", 24),
                                    ("prefill", 40)])
@pytest.mark.parametrize("d_in,d_out,r_p,P,pad_v,pad_u", [(1000, 700, 48, 2, 4, 12), (520, 130, 17, 2, 0, 4),
                                                          (2048, 1100, 304, 2, 8, 0)])
def test_packed_strides_not_aligned(d_in, d_out, r_p, P, pad_v, pad_u, path, T):
    """Plane strides the caller picks (any multiple of 4 words at least the
    packed length; the binding's default is a multiple of 32): every kernel
    family addresses the planes through ld_v / ld_u."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    inp = synth.layer_inputs(d_in + 3 * d_out + pad_v, d_in, d_out, r_p, P)
    x = synth.activations(T + d_in, T, d_in, "bf16")
    layer = dev_layer_ld(inp, pad_v, pad_u)
    say("strides", d_in, d_out, r_p, P, layer.ld_v, layer.ld_u, path, "T", T)
    y = lb.linear_forward(x_to_dev(x), layer, torch.bfloat16, PATH_FLAG[path])
    torch.cuda.synchronize()
    ref = oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l)
    assert_close(y_to_np(y), ref, TOL["bf16"], ("strides", d_in, r_p, path, T))


@pytest.mark.parametrize("d_in,d_out,r_p,P", [(33, 65, 17, 2), (520, 130, 17, 2), (1000, 300, 30, 1), (96, 40, 6, 2)])
@pytest.mark.parametrize("T", [9, 17, 32])
@pytest.mark.parametrize("path", DECODE_PATHS)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_decode_kernels_odd_ranks_many_tokens(d_in, d_out, r_p, P, T, path, dt):
    """Path ranks that are not multiples of 4 above 8 tokens, where the decode
    kernels run stage 1 unfused: each latent's partial sum is stored on its
    own, so the 4-latent group crossing r_p does not spill into the next
    path's latents (as it did while the stores took whole groups of 4)."""
    inp = synth.layer_inputs(d_in + 2 * d_out + r_p, d_in, d_out, r_p, P)
    x = synth.activations(T + d_in + 1, T, d_in, dt)
    _check(inp, x, dt, path)
