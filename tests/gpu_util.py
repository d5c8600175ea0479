"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import pytest

import synth

TOL = {"f32": 1e-3, "bf16": 8e-3}    # relative L2 bound against the fp64 oracle


def torch_or_skip():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(*a):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def x_to_dev(x):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def y_to_np(y):
    import torch
    return y.float().cpu().numpy().astype(np.float64)


def dev_layer(inp):
    import torch
    import binarized_rank_linear_amd as lb
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    h16 = lambda a: t(a.view(np.int16)) if a.dtype == np.uint16 else t(a.astype(np.float16))
    return lb.PackedLinear.from_factors(t(inp.U), t(inp.V), h16(inp.h), h16(inp.g), h16(inp.l))


def host_layer_from_dev(U, V, h, g, l):
    """Copy GPU-generated float factors back for the oracle."""
    d = lambda a: a.detach().cpu().numpy()
    P, d_out, r_p = U.shape
    return synth.LayerInputs(V.shape[1], d_out, r_p, P, d(U), d(V),
                             d(h).view(np.uint16), d(g).view(np.uint16), d(l).view(np.uint16))
