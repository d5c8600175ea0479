"""GPU parity of the Joint-ITQ rotation (lb_joint_itq, lb_dual_svid_itq)
against the oracle (oracle/itq.py, fp64 numpy).

One alternation is compared step by step: from the same starting rotation
the GPU's next rotation must lie within a perturbation bound of the oracle's.
The bound follows from the fp32 arithmetic: the rotated factors A = F R carry
at most (r + 1) 2^-24 sum_l |F_il||R_lj| per entry, so a code may differ only
where |A_ij| is below that; each such code moves Z = F^T sign(A) by
2 sum |F_ik| in its column, and the accumulation over D rows adds
(D + 1) 2^-24 sum_i |F_ik| per entry.  The polar factor moves by at most
2 ||dZ||_F / (sigma_r + sigma_{r-1}) (the perturbation bound of the
orthogonal polar factor of a real square matrix), plus the fp32 Newton-Schulz
iteration's own rounding, r^1.5 2^-24 in the Frobenius norm.  Whole runs are
checked for what the method guarantees: an orthogonal R, a non-increasing
objective, an unchanged factor product, and the same result as the same
number of single steps."""
import numpy as np
import pytest

import oracle
import synth
from oracle import itq, svid
from gpu_util import TOL, assert_close, say, torch_or_skip, x_to_dev, y_to_np

pytestmark = pytest.mark.gpu

EPS = 2.0 ** -24


def _factors(seed, d_out, d_in, r_p):
    """fp32 U' [d_out][r_p], V' [d_in][r_p]: the SVD split of a seeded dense
    weight with a decaying spectrum (as Dual-SVID hands them to the rotation)."""
    W = synth.dense_weight(seed, d_out, d_in)
    Up, Vp = svid.truncated_factors(W, r_p)
    return Up.astype(np.float32), Vp.astype(np.float32)


def _step_bound(F, R):
    """Frobenius bound on |R_gpu - R_oracle| after one step from R (both fp64
    copies of the fp32 values the GPU used), and the oracle's next R."""
    D, r = F.shape
    A = F @ R
    dA = (r + 1) * EPS * (np.abs(F) @ np.abs(R))
    amb = (np.abs(A) <= dA).astype(np.float64)
    Z = F.T @ itq.sign_pm(A)
    colsum = np.abs(F).sum(axis=0)
    dZ = (D + 1) * EPS * colsum[:, None] * np.ones((1, r)) + 2.0 * (np.abs(F).T @ amb)
    s = np.linalg.svd(Z, compute_uv=False)
    den = s[-1] + (s[-2] if r > 1 else s[-1])
    return 2.0 * np.linalg.norm(dZ) / den + r ** 1.5 * EPS, itq.procrustes(Z), int(amb.sum())


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def _run(lb, U, V, iters, rot0=None):
    """One lb_joint_itq call on copies; returns (U R, V R, R, objective) as fp64 numpy."""
    import torch
    Ud, Vd = _dev(U), _dev(V)
    R, obj = lb.joint_itq(Ud, Vd, iters, rot0=None if rot0 is None else _dev(rot0))
    torch.cuda.synchronize()
    f = lambda t: t.cpu().numpy().astype(np.float64)
    return f(Ud), f(Vd), f(R), obj.cpu().numpy()


@pytest.mark.parametrize("d_out,d_in,r_p", [(96, 64, 16), (320, 192, 48), (1100, 700, 200), (300, 2100, 130)])
def test_itq_steps_against_oracle(d_out, d_in, r_p):
    """Eight single steps, each from the GPU's previous rotation, against the
    oracle's step from that same rotation; the objective the GPU reports for
    its start against the oracle's within the fp32 product error."""
    torch_or_skip()
    import binarized_rank_linear_amd as lb
    U, V = _factors(950 + r_p, d_out, d_in, r_p)
    F = np.vstack([U, V]).astype(np.float64)
    R = np.eye(r_p)
    say("itq steps", d_out, d_in, r_p)
    for step in range(8):
        Ur, Vr, Rg, obj = _run(lb, U, V, 1, rot0=R if step else None)
        bound, Ro, amb = _step_bound(F, R)
        dev = np.linalg.norm(Rg - Ro)
        assert dev <= bound, ("step", step, dev, bound, amb)
        # the objective at the start of the step
        A = F @ R
        dA = (r_p + 1) * EPS * (np.abs(F) @ np.abs(R))
        q = itq.objective(U, V, R)
        dq = np.sum(2.0 * np.abs(1.0 - np.abs(A)) * dA + dA * dA) + 1e-12 * q
        assert abs(obj[0] - q) <= dq, ("objective", step, obj[0], q, dq)
        if step == 0:
            # R = I: the product is exact and the first codes are the factors' own signs
            assert abs(obj[0] - q) <= 1e-9 * q
            assert amb == 0
        # the rotated factors are F times the returned rotation
        Rf = Rg.astype(np.float32).astype(np.float64)
        dAr = (r_p + 1) * EPS * (np.abs(F) @ np.abs(Rf)) + 1e-30
        assert np.all(np.abs(np.vstack([Ur, Vr]) - F @ Rf) <= dAr), ("rotated factors", step)
        R = Rf


def _eval_err(F, R):
    """Bound on |GPU objective - exact objective| at R: the GPU squares
    (1 - |a|) in fp64 from fp32 products a carrying the product error dA."""
    A = F @ R
    dA = (R.shape[0] + 1) * EPS * (np.abs(F) @ np.abs(R))
    return float(np.sum(2.0 * np.abs(1.0 - np.abs(A)) * dA + dA * dA)) + 1e-12 * float(np.sum((1 - np.abs(A)) ** 2))


@pytest.mark.parametrize("d_out,d_in,r_p,iters", [(320, 192, 48, 20), (1100, 700, 200, 12)])
def test_itq_run_properties(d_out, d_in, r_p, iters):
    """A whole run: R orthogonal, the factor product unchanged, the run equal
    bit for bit to the same number of single steps (the same kernels in the
    same order), and the objective never rising by more than the step's
    rounding allows: with the exact codes and rotation an alternation cannot
    raise it; the GPU's codes may differ where |a| <= dA (at most 4 dA each),
    its rotation sits within the step bound of the exact Procrustes solution
    (at most 2 |Z|_F times that), and each reported value carries its own
    evaluation error."""
    torch_or_skip()
    import binarized_rank_linear_amd as lb
    U, V = _factors(960 + r_p, d_out, d_in, r_p)
    F = np.vstack([U, V]).astype(np.float64)
    say("itq run", d_out, d_in, r_p, iters)
    Ur, Vr, Rg, obj = _run(lb, U, V, iters)
    orth = np.max(np.abs(Rg.T @ Rg - np.eye(r_p)))
    assert orth <= 32 * r_p * EPS, orth
    assert obj[-1] < obj[0]
    P0 = F[:d_out] @ F[d_out:].T
    P1 = Ur @ Vr.T
    assert np.linalg.norm(P1 - P0) <= (2 * r_p * EPS + 2 * orth) * np.linalg.norm(F[:d_out]) * np.linalg.norm(F[d_out:])
    # the same run as single steps, and the objective's slack per step
    R, Rprev = None, np.eye(r_p)
    for k in range(iters):
        _, _, Rs, _ = _run(lb, U, V, 1, rot0=R)
        bound, _, _ = _step_bound(F, Rprev)
        A = F @ Rprev
        dA = (r_p + 1) * EPS * (np.abs(F) @ np.abs(Rprev))
        Z = F.T @ itq.sign_pm(A)
        R = Rs.astype(np.float32)
        slack = (4.0 * float(np.sum(dA[np.abs(A) <= dA])) + 2.0 * np.linalg.norm(Z) * bound +
                 _eval_err(F, Rprev) + _eval_err(F, R.astype(np.float64)))
        assert obj[k + 1] <= obj[k] + slack, ("step", k, obj[k + 1] - obj[k], slack)
        Rprev = R.astype(np.float64)
    assert np.array_equal(R.astype(np.float64), Rg)
    _, qo = itq.joint_itq(F[:d_out], F[d_out:], iters)
    print("itq objective gpu %.9e oracle %.9e start %.9e" % (obj[-1], qo[-1], qo[0]))


def test_itq_recovers_a_planted_rotation():
    """The oracle pin's exact case on the GPU: orthogonal +-1 columns turned by
    a rotation Q near I come back as the columns, with R = Q."""
    torch_or_skip()
    import binarized_rank_linear_amd as lb
    from scipy.linalg import expm

    def syl(n):
        H = np.ones((1, 1))
        while H.shape[0] < n:
            H = np.block([[H, H], [H, -H]])
        return H
    r = 32
    a = np.random.default_rng(44).standard_normal((r, r))
    Q = expm(0.02 * (a - a.T))
    Bu, Bv = syl(256)[:, :r], syl(128)[:, 3:r + 3]
    U, V = (Bu @ Q.T).astype(np.float32), (Bv @ Q.T).astype(np.float32)
    say("itq planted")
    Ur, Vr, Rg, obj = _run(lb, U, V, 3)
    assert np.max(np.abs(Rg - Q)) <= 64 * r * EPS
    assert np.max(np.abs(Ur - Bu)) <= 64 * r * EPS
    assert np.max(np.abs(Vr - Bv)) <= 64 * r * EPS
    assert obj[1] <= (256 + 128) * r * (64 * r * EPS) ** 2


def test_itq_zero_factors_keep_the_start():
    """Zero factors: Z = 0, every rotation is optimal and the start is kept;
    the objective counts 1 per entry (sign(0) = +1)."""
    torch_or_skip()
    import binarized_rank_linear_amd as lb
    U, V = np.zeros((40, 8), np.float32), np.zeros((24, 8), np.float32)
    say("itq zero")
    Ur, Vr, Rg, obj = _run(lb, U, V, 2)
    assert np.array_equal(Rg, np.eye(8))
    assert np.all(obj == 64 * 8)
    assert not Ur.any() and not Vr.any()


def _sin_bounds(M, r_p):
    s = np.linalg.svd(np.asarray(M, np.float64), compute_uv=False)
    out = np.empty(r_p)
    for k in range(r_p):
        lo = s[k - 1] - s[k] if k > 0 else np.inf
        hi = s[k] - s[k + 1] if k + 1 < len(s) else np.inf
        gap = min(lo, hi)
        out[k] = 1.0 if gap <= 0 else min(1.0, 64 * EPS * s[0] / gap)
    return s, out


@pytest.mark.parametrize("d_out,d_in,r,residual", [(96, 64, 32, True), (256, 256, 128, False),
                                                   (384, 1024, 208, True)])
def test_dual_svid_itq(d_out, d_in, r, residual):
    """lb_dual_svid_itq: path 0's rotated factors are lb_joint_itq's rotation of
    lb_dual_svid's factors (bit for bit: the same kernels); every path's
    rotated product matches the oracle's truncated SVD of what the path fits
    (W, or the GPU's remainder) within the singular-gap bound; the signs are the
    rotated factors' own (packed bit for bit), the scales the oracle's rank-1
    fits of their magnitudes (two fp16 steps); the rotation lowers the sign-fit
    objective; the packed layer through the forward matches the oracle."""
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    iters = 10
    W = synth.dense_weight(970 + d_out + d_in, d_out, d_in)
    P = 2 if residual else 1
    r_p = r // P
    Wd = torch.from_numpy(W).cuda()
    say("dual svid itq", d_out, d_in, r, residual)
    _, U0, V0 = lb.dual_svid(Wd, r, residual, float_factors=True)
    lin, U1, V1 = lb.dual_svid(Wd, r, residual, float_factors=True, itq_iters=iters)
    torch.cuda.synchronize()
    Ua, Va = U0[0].clone(), V0[0].clone()
    lb.joint_itq(Ua, Va, iters)
    torch.cuda.synchronize()
    assert torch.equal(Ua, U1[0]) and torch.equal(Va, V1[0])
    Ug, Vg = U1.cpu().numpy().astype(np.float64), V1.cpu().numpy().astype(np.float64)
    hg = lin.h.cpu().numpy().view(np.uint16)
    gg = lin.g.cpu().numpy().view(np.uint16)
    lg = lin.l.cpu().numpy().view(np.uint16)
    vb = lin.v_bits.cpu().numpy().view(np.uint32)
    ub = lin.u_bits.cpu().numpy().view(np.uint32)
    target = W.astype(np.float64)
    for p in range(P):
        if p == 1:
            target = W.astype(np.float64) - oracle.dense_weight(Ug[:1], Vg[:1], hg[:1], gg[:1], lg[:1])
        Uo, Vo = svid.truncated_factors(target, r_p)
        s, sin = _sin_bounds(target, r_p)
        # each latent's term s_k u_k v_k^T moves by at most 2 s_k times its
        # vectors' error (8 sin(theta_k), at least 8 r_p fp32 roundings), plus
        # the rotation's rounding
        tol = np.sum(2 * s[:r_p] * np.maximum(8 * sin, 8 * r_p * EPS)) + 1e-5 * np.linalg.norm(target)
        dev = np.linalg.norm(Ug[p] @ Vg[p].T - Uo @ Vo.T)
        assert dev <= tol, ("path", p, dev, tol)
        # signs packed bit for bit; scales the oracle's fits of the rotated magnitudes
        assert np.array_equal(vb[p], oracle.pack_signs(Vg[p].astype(np.float32), 0, vb.shape[2]))
        assert np.array_equal(ub[p], oracle.pack_signs(Ug[p].astype(np.float32), 1, ub.shape[2]))
        h, lu = svid.rank1_nonneg(np.abs(Ug[p]))
        g, lv = svid.rank1_nonneg(np.abs(Vg[p]))
        for got, want, what in ((hg[p], h, "h"), (gg[p], g, "g"), (lg[p], lu * lv, "l")):
            gw = oracle.widen_f16(got)
            assert np.allclose(gw, want, rtol=2 * 2.0 ** -10, atol=0), (what, p)
        # the rotation lowers the objective it minimises (the start: the SVD split)
        q1 = itq.objective(Ug[p], Vg[p], np.eye(r_p))
        q0 = itq.objective(Uo, Vo, np.eye(r_p))
        assert q1 < q0, (p, q1, q0)
    T = 3
    x = synth.activations(78, T, d_in, "f32")
    y = lb.linear_forward(x_to_dev(x), lin, torch.float32)
    torch.cuda.synchronize()
    ref = oracle.linear_forward(x, Ug.astype(np.float32), Vg.astype(np.float32), hg, gg, lg)
    assert_close(y_to_np(y), ref, TOL["f32"], ("svid itq forward", d_out, d_in))


def test_joint_itq_argument_errors():
    torch = torch_or_skip()
    import binarized_rank_linear_amd as lb
    U = torch.zeros((32, 8), dtype=torch.float32, device="cuda")
    V = torch.zeros((16, 8), dtype=torch.float32, device="cuda")
    say("itq errors")
    with pytest.raises(lb.LBError) as e:
        lb.joint_itq(U, V, -1)
    assert e.value.status == lb.LB_EINVAL
    with pytest.raises(lb.LBError) as e:
        lb.joint_itq(U[:, :4].contiguous(), torch.zeros((2, 4), dtype=torch.float32, device="cuda"), 1)
    assert e.value.status == lb.LB_EINVAL                  # r_p above min(d_out, d_in)
