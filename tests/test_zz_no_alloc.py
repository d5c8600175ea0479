"""lb_linear_forward_noalloc (the library's own fixed workspace) against
lb_linear_forward with a caller workspace: the same kernels, so the same bits.
Two calls in a row, the second with a smaller input; also requests past the
fixed workspace, which must be refused."""
import numpy as np
import pytest

import synth
from gpu_util import dev_layer, say, torch_or_skip, x_to_dev

pytestmark = pytest.mark.gpu


def _bits(torch, y):
    return y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32)


@pytest.mark.parametrize("shape,calls", [
    ((8192, 28672, 304, 2), [(32, "bf16", 1), (1, "bf16", 1)]),        # c5 gate: decode, T 32 then 1
    ((17408, 5120, 1088, 2), [(8, "bf16", 1), (2, "bf16", 1)]),        # c4 down
    ((1024, 1024, 512, 1), [(8, "f32", 0), (3, "f32", 0)]),            # c1, fp32 out
    ((2048, 1536, 160, 2), [(300, "bf16", 2), (64, "bf16", 2)]),       # GEMM path, 300 then 64 tokens
    ((1000, 700, 48, 2), [(17, "f32", 3), (5, "f32", 3)]),             # vector-ALU path, ragged
])
def test_noalloc_equals_caller_workspace(shape, calls):
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    d_in, d_out, r_p, P = shape
    inp = synth.layer_inputs(d_in + 5 * d_out, d_in, d_out, r_p, P)
    layer = dev_layer(inp)
    for k, (T, dt, flags) in enumerate(calls):
        say("noalloc", shape, "call", k, "T", T, dt, "flags", flags)
        x = x_to_dev(synth.activations(400 + 7 * k + T, T, d_in, dt))
        odt = torch.float32 if dt == "f32" else torch.bfloat16
        want = lb.linear_forward(x, layer, odt, flags)
        got = torch.full((T, d_out), float("nan"), dtype=odt, device="cuda")
        lb.linear_forward_noalloc(x, layer, odt, flags, out=got)
        torch.cuda.synchronize()
        assert torch.equal(_bits(torch, got), _bits(torch, want)), (shape, k)


def test_noalloc_refuses_requests_past_its_workspace():
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    d_in, d_out, r_p, P = 17408, 5120, 1088, 2               # c4 down at T = 2048
    need = lb.lib().lb_linear_workspace_bytes(d_in, d_out, 2 * r_p, 2048, 1, lb.LB_PATH_PREFILL)
    assert need > lb.NOALLOC_SCRATCH_BYTES
    inp = synth.layer_inputs(9, d_in, d_out, r_p, P)
    layer = dev_layer(inp)
    x = torch.zeros((2048, d_in), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lb.LBError) as e:
        lb.linear_forward_noalloc(x, layer, torch.bfloat16, lb.LB_PATH_PREFILL)
    assert e.value.status == lb.LB_EWORKSPACE
