"""GPU parity of the Dual-SVID initialisation (lb_dual_svid) against the
oracle's (oracle/svid.py, fp64 numpy).

The first path is unique up to each singular pair's sign, so it is compared
directly: the fp16 scales within two fp16 steps (the GPU rounds from fp32),
and U' and V' column by column after matching the column's sign, within a
bound derived from the fp32 arithmetic and the gap between neighbouring
singular values (signs may differ only inside that bound).  The residual path is fitted to what the first
path leaves, which depends on those roundings, so it is checked as valid
rather than equal: it is the oracle's fit of the GPU's own remainder.  The
packed output is checked through the forward: lb_linear_forward with the
initialised layer against the oracle's forward on the GPU's float factors."""
import numpy as np
import pytest

import oracle
import synth
from oracle import svid
from gpu_util import TOL, assert_close, say, torch_or_skip, x_to_dev, y_to_np

pytestmark = pytest.mark.gpu


def _sin_bounds(M, r_p):
    """Per latent k, a bound on the angle between a computed singular vector
    and the exact one: 64 fp32 roundings of the largest singular value over
    the gap to the neighbouring singular values (the perturbation bound
    sin(theta) <= |E| / gap), capped at 1."""
    s = np.linalg.svd(np.asarray(M, np.float64), compute_uv=False)
    out = np.empty(r_p)
    for k in range(r_p):
        lo = s[k - 1] - s[k] if k > 0 else np.inf
        hi = s[k] - s[k + 1] if k + 1 < len(s) else np.inf
        gap = min(lo, hi)
        out[k] = 1.0 if gap <= 0 else min(1.0, 64 * 2.0 ** -24 * s[0] / gap)
    return out


def _signs_match(got, want, sin_k, what):
    """Columns of got equal columns of want up to one sign per column; an
    entry's sign may differ only where the entry is within the column's error
    bound of zero (8 sin(theta) of the column RMS); values agree within that
    bound (at least 2e-3 of the RMS)."""
    for k in range(want.shape[1]):
        flip = -1.0 if np.dot(got[:, k], want[:, k]) < 0 else 1.0
        g, w = flip * got[:, k], want[:, k]
        scale = np.sqrt(np.mean(w * w))
        tol = max(2e-3, 8 * sin_k[k]) * scale
        bad = (np.sign(g) != np.sign(w)) & (np.abs(w) > tol)
        assert not bad.any(), (what, "column", k, np.nonzero(bad)[0][:5], tol / scale)
        assert np.allclose(g, w, rtol=0, atol=tol), (what, "column", k, np.max(np.abs(g - w)) / scale, tol / scale)


def _close_f16(got_bits, want_bits, what):
    g, w = oracle.widen_f16(got_bits), oracle.widen_f16(want_bits)
    assert np.allclose(g, w, rtol=2 * 2.0 ** -10, atol=0), (what, np.max(np.abs(g - w) / np.abs(w)))


@pytest.mark.parametrize("d_out,d_in,r,residual", [(96, 64, 32, True), (64, 96, 48, True), (256, 256, 128, False),
                                                   (1024, 1024, 512, False), (384, 1024, 208, True),
                                                   (96, 64, 34, True), (130, 70, 13, False)])
def test_dual_svid_against_oracle(d_out, d_in, r, residual):
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    W = synth.dense_weight(900 + d_out + d_in, d_out, d_in)
    say("dual svid", d_out, d_in, r, residual)
    lin, U, V = lb.dual_svid(torch.from_numpy(W).cuda(), r, residual, float_factors=True)
    torch.cuda.synchronize()
    Ug, Vg = U.cpu().numpy().astype(np.float64), V.cpu().numpy().astype(np.float64)
    hg = lin.h.cpu().numpy().view(np.uint16)
    gg = lin.g.cpu().numpy().view(np.uint16)
    lg = lin.l.cpu().numpy().view(np.uint16)
    r_p = r // (2 if residual else 1)
    # path 0 against the oracle
    Uo, Vo, ho, go, lo = svid.svid_path(W.astype(np.float64), r_p)
    sin0 = _sin_bounds(W, r_p)
    _signs_match(Ug[0], Uo, sin0, "U'")
    _signs_match(Vg[0], Vo, sin0, "V'")
    _close_f16(hg[0], ho, "h")
    _close_f16(gg[0], go, "g")
    _close_f16(lg[0], lo, "l")
    if residual:
        # path 1: the oracle's fit of the GPU's remainder
        W1 = oracle.dense_weight(Ug[:1], Vg[:1], hg[:1], gg[:1], lg[:1])
        R = W.astype(np.float64) - W1
        U1, V1, h1, g1, l1 = svid.svid_path(R, r_p)
        sin1 = _sin_bounds(R, r_p)
        _signs_match(Ug[1], U1, sin1, "U' residual")
        _signs_match(Vg[1], V1, sin1, "V' residual")
        _close_f16(hg[1], h1, "h residual")
        _close_f16(gg[1], g1, "g residual")
        _close_f16(lg[1], l1, "l residual")
    # the approximation error the layer reaches, against the oracle's
    err = oracle.rel_l2(svid.reconstruction(Ug, Vg, hg, gg, lg), W)
    err_o = oracle.rel_l2(svid.reconstruction(*svid.dual_svid(W, r_p, residual)), W)
    assert abs(err - err_o) < 1e-3, (err, err_o)
    # the packed layer through the forward, against the oracle on the float factors
    T = 3
    x = synth.activations(77, T, d_in, "f32")
    y = lb.linear_forward(x_to_dev(x), lin, torch.float32)
    torch.cuda.synchronize()
    ref = oracle.linear_forward(x, Ug.astype(np.float32), Vg.astype(np.float32), hg, gg, lg)
    assert_close(y_to_np(y), ref, TOL["f32"], ("svid forward", d_out, d_in))


def test_dual_svid_reproduces_a_hadamard_layer():
    """The oracle pin's exact case on the GPU: a layer with orthogonal
    Hadamard sign columns and constant row/column scales comes back within the
    fp16 rounding of its three scales."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    def syl(n):
        H = np.ones((1, 1))
        while H.shape[0] < n:
            H = np.block([[H, H], [H, -H]])
        return H
    d_out, d_in, r = 64, 128, 16
    W = (0.125 * syl(d_out)[:, :r] @ np.diag(2.0 ** -np.arange(r)) @ syl(d_in)[:, :r].T).astype(np.float32)
    say("dual svid hadamard")
    lin, U, V = lb.dual_svid(torch.from_numpy(W).cuda(), r, False, float_factors=True)
    torch.cuda.synchronize()
    got = svid.reconstruction(U.cpu().numpy().astype(np.float64), V.cpu().numpy().astype(np.float64),
                              lin.h.cpu().numpy().view(np.uint16), lin.g.cpu().numpy().view(np.uint16),
                              lin.l.cpu().numpy().view(np.uint16))
    assert np.max(np.abs(got - W) / np.abs(W)) <= 4 * 2.0 ** -11


def test_dual_svid_argument_errors():
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    W = torch.zeros((32, 16), dtype=torch.float32, device="cuda")
    say("dual svid errors")
    with pytest.raises(lb.LBError) as e:
        lb.dual_svid(W, 33, True)                       # odd total rank with the residual
    assert e.value.status == lb.LB_EINVAL
    with pytest.raises(lb.LBError) as e:
        lb.dual_svid(W, 64, True)                       # r_p above min(d_out, d_in)
    assert e.value.status == lb.LB_EINVAL
