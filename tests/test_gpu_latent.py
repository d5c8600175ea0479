"""GPU tests of the latent API (lb_linear_stage1 / lb_linear_stage2): the two
halves of the layer around the rank-r intermediate t, against the whole
layer and the oracle's latents, and a k-projection latent cache."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, assert_close, dev_layer, say, torch_or_skip, x_to_dev, y_to_np

pytestmark = pytest.mark.gpu

FLAG = {"auto": 0, "decode": 1, "prefill": 2, "valu": 3}


def _bits(torch, y):
    return y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)


@pytest.mark.parametrize("shape,T,xdt,ydt,tdt,path", [
    ((1024, 700, 96, 2), 1, "bf16", "bf16", "f32", "auto"),      # decode kernels, two limbs
    ((4096, 4096, 1024, 2), 4, "bf16", "bf16", "f32", "auto"),
    ((2080, 515, 200, 2), 3, "f32", "f32", "f32", "auto"),       # decode kernels, three limbs
    ((8192, 1024, 32, 2), 20, "bf16", "bf16", "f32", "decode"),  # unfused stage 1 (prep + stage 1)
    ((8192, 1024, 32, 2), 20, "bf16", "bf16", "f32", "auto"),    # GEMM kernels, 64-token tiles
    ((2048, 1536, 160, 2), 300, "bf16", "bf16", "bf16", "auto"),  # GEMM kernels: bf16 latents
    ((2048, 1100, 304, 2), 64, "bf16", "bf16", "f32", "auto"),
    ((1000, 700, 48, 2), 40, "f32", "f32", "f32", "auto"),       # vector-ALU kernels (fp32 out, T > 32)
    ((520, 130, 16, 1), 5, "bf16", "bf16", "f32", "valu"),
    # path ranks off the 16-multiple grid (not multiples of 4) on each kernel family
    ((1000, 700, 17, 2), 1, "bf16", "bf16", "f32", "auto"),
    ((1000, 700, 17, 2), 20, "bf16", "bf16", "f32", "decode"),
    ((1000, 700, 17, 2), 40, "bf16", "bf16", "bf16", "auto"),
    ((9000, 300, 30, 2), 64, "bf16", "bf16", "bf16", "auto"),
    ((520, 130, 6, 1), 5, "f32", "f32", "f32", "valu"),
])
def test_stages_compose_to_the_layer(shape, T, xdt, ydt, tdt, path):
    """stage 2 of stage 1's latents gives lb_linear_forward's bits when t
    holds the kernels' own latent precision, and stage 1's t is the oracle's
    latents within the output tolerance."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    d_in, d_out, r_p, P = shape
    say("latent API", shape, "T", T, xdt, ydt, tdt, path)
    inp = synth.layer_inputs(d_in + d_out + T, d_in, d_out, r_p, P)
    layer = dev_layer(inp)
    x = synth.activations(T + 3 * d_in, T, d_in, xdt)
    xd = x_to_dev(x)
    tt = torch.float32 if tdt == "f32" else torch.bfloat16
    yt = torch.float32 if ydt == "f32" else torch.bfloat16
    want = lb.linear_forward(xd, layer, yt, FLAG[path])
    t = lb.linear_stage1(xd, layer, tt, yt, FLAG[path])
    y = lb.linear_stage2(t, layer, yt, FLAG[path])
    torch.cuda.synchronize()
    assert torch.equal(_bits(torch, y), _bits(torch, want))
    t_ref = oracle.linear_latents(x, inp.V, inp.g, inp.l)
    assert_close(y_to_np(t), t_ref, TOL[ydt], "latents")


def test_bf16_latents_on_the_decode_kernels():
    """A bf16 t on the decode kernels rounds the latents once more: still
    within the bf16 tolerance of the oracle, output and latents."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    inp = synth.layer_inputs(33, 4096, 1100, 304, 2)
    x = synth.activations(34, 2, 4096, "bf16")
    layer = dev_layer(inp)
    t = lb.linear_stage1(x_to_dev(x), layer, torch.bfloat16, torch.bfloat16)
    y = lb.linear_stage2(t, layer, torch.bfloat16)
    torch.cuda.synchronize()
    assert_close(y_to_np(t), oracle.linear_latents(x, inp.V, inp.g, inp.l), TOL["bf16"], "latents")
    assert_close(y_to_np(y), oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l), TOL["bf16"], "y")


def test_k_projection_latent_cache():
    """A Llama2-7B-shaped k projection (4096 -> 4096, 0.1 bits per weight with
    the residual: rank 192) decodes 40 tokens one at a time, caching each
    token's bf16 latents (192 values) instead of its 4096 outputs: the cache is
    21.3x smaller (sesamedisk, "The real result").  Expanding the whole cache
    at once (stage 2 at T = 40, the GEMM kernels) gives the oracle's k within
    the bf16 tolerance."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    r, rp = lb.rank_for_budget(4096, 4096, 1, 10, True)
    assert (r, rp) == (192, 96)
    inp = synth.layer_inputs(44, 4096, 4096, rp, 2)
    layer = dev_layer(inp)
    steps = 40
    x = synth.activations(45, steps, 4096, "bf16")
    xd = x_to_dev(x)
    cache = torch.empty((steps, r), dtype=torch.bfloat16, device="cuda")
    for n in range(steps):
        lb.linear_stage1(xd[n:n + 1], layer, torch.bfloat16, torch.bfloat16, out=cache[n:n + 1])
    k = lb.linear_stage2(cache, layer, torch.bfloat16)
    torch.cuda.synchronize()
    full_bytes = steps * 4096 * 2
    assert round(full_bytes / (cache.numel() * cache.element_size()), 1) == 21.3
    ref = oracle.linear_forward(x, inp.U, inp.V, inp.h, inp.g, inp.l)
    assert_close(y_to_np(k), ref, TOL["bf16"], "k from the latent cache")
    # each cached row is that token's own latents, as the oracle computes them
    assert_close(y_to_np(cache), oracle.linear_latents(x, inp.V, inp.g, inp.l), TOL["bf16"], "cache")
