"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import pytest

import oracle
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


def dev_layer_ld(inp, pad_v, pad_u):
    """The layer packed with plane strides ld_v = packed_ld(r_p) + pad_v and
    ld_u = packed_ld(d_out) + pad_u (multiples of 4 words, not of 32)."""
    import torch
    import binarized_rank_linear_amd as lb
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    U, V = t(inp.U), t(inp.V)
    P, d_out, r_p = U.shape
    d_in = V.shape[1]
    ld_v, ld_u = lb.packed_ld(r_p) + pad_v, lb.packed_ld(d_out) + pad_u
    v_bits = torch.empty((P, (d_in + 31) // 32, ld_v), dtype=torch.int32, device="cuda")
    u_bits = torch.empty((P, (r_p + 31) // 32, ld_u), dtype=torch.int32, device="cuda")
    for p in range(P):
        lb.pack_signs(V[p], 0, ld_v, out=v_bits[p])
        lb.pack_signs(U[p], 1, ld_u, out=u_bits[p])
    h16 = lambda a: t(a.view(np.int16))
    return lb.PackedLinear(d_in, d_out, P * r_p, P == 2, v_bits, u_bits, h16(inp.g), h16(inp.l), h16(inp.h),
                           ld_v, ld_u)


def host_layer_from_dev(U, V, h, g, l):
    """Copy GPU-generated float factors back for the oracle."""
    d = lambda a: a.detach().cpu().numpy()
    P, d_out, r_p = U.shape
    return synth.LayerInputs(V.shape[1], d_out, r_p, P, d(U), d(V),
                             d(h).view(np.uint16), d(g).view(np.uint16), d(l).view(np.uint16))


def assert_close(got, ref, tol, what=""):
    """Relative L2 over the whole tensor within tol, and every element within
    8 * tol * rms(ref): a single wrong element (a lane, a tail row) can hide
    inside the L2 of a wide output but not under the per-element bound.  The
    worst element is named on failure."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = oracle.rel_l2(got, ref)
    assert err <= tol, (what, "rel-L2", err, tol)
    d = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    if d.size:
        i = int(np.argmax(d))
        bound = 8.0 * tol * rms
        assert d.flat[i] <= bound, (what, "worst element", np.unravel_index(i, d.shape), float(d.flat[i]),
                                    "bound", bound, "got", float(got.flat[i]), "want", float(ref.flat[i]))
    return err
