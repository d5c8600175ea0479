"""Joint-ITQ rotation of a layer's latent factors, in numpy fp64 (TEST
INFRASTRUCTURE ONLY, like the rest of this package: the product path never
imports it).

Written from the pages' description of the LittleBit-2 initialisation
(littlebitllm, hero and "The method"; trove, "How it works", step 2; deniz.in,
"LittleBit-2 fixes the initialization"): an internal rotation of the latent
space lines the SVD-derived factors up with the corners of the binary
hypercube before the sign step, and it folds into the factors, so the deployed
layer keeps its form.

For any orthogonal R (r_p x r_p), (U' R)(V' R)^T = U' V'^T: the rotation leaves
the truncated product unchanged and only moves where the signs are taken.  The
rotation is found by iterative quantisation (ITQ) done jointly on both factors
with one shared R:

    minimise  Q(R) = ||sign(U'R) - U'R||_F^2 + ||sign(V'R) - V'R||_F^2,

alternating two exact steps:
1. with R fixed, the best codes are B_u = sign(U'R), B_v = sign(V'R);
2. with the codes fixed, Q is ||B||^2 + ||F||^2 - 2 <U'^T B_u + V'^T B_v, R>,
   so the best orthogonal R is the orthogonal Procrustes solution: the polar
   factor P Q^T of Z = U'^T B_u + V'^T B_v = P S Q^T (its SVD).
Neither step can raise Q, so the sequence of objectives never increases.

Readings where the pages leave a step open (each is a plain choice):
- the objective is the classic ITQ loss of each factor as it comes out of the
  SVD split (each column carrying sqrt of its singular value), summed over the
  two factors, with no extra weighting;
- sign(0) = +1, as for the layer's own signs;
- the iteration starts from R = I (the unrotated Dual-SVID factors), so the
  result is never worse than no rotation by this objective; the iteration
  count is a parameter;
- the rotation is applied to each path's factors before their signs and
  scales are taken, the residual path included (on its own remainder).
"""
from __future__ import annotations

import numpy as np


def sign_pm(a: np.ndarray) -> np.ndarray:
    """+1 / -1 with sign(0) = sign(-0) = +1 (bit = value < 0)."""
    return np.where(np.asarray(a) < 0, -1.0, 1.0)


def procrustes(Z: np.ndarray) -> np.ndarray:
    """The orthogonal R that maximises <Z, R>_F = trace(Z^T R): the polar
    factor P Q^T of Z = P S Q^T (numpy's SVD)."""
    P, _, Qt = np.linalg.svd(np.asarray(Z, dtype=np.float64))
    return P @ Qt


def objective(Up: np.ndarray, Vp: np.ndarray, R: np.ndarray) -> float:
    """Q(R): the squared distance of both rotated factors to their signs."""
    A = np.asarray(Up, dtype=np.float64) @ R
    C = np.asarray(Vp, dtype=np.float64) @ R
    return float(np.sum((sign_pm(A) - A) ** 2) + np.sum((sign_pm(C) - C) ** 2))


def itq_step(Up: np.ndarray, Vp: np.ndarray, R: np.ndarray) -> np.ndarray:
    """One alternation from R: the codes of the rotated factors, then the
    rotation that best fits both factors to them."""
    Up = np.asarray(Up, dtype=np.float64)
    Vp = np.asarray(Vp, dtype=np.float64)
    Bu = sign_pm(Up @ R)
    Bv = sign_pm(Vp @ R)
    return procrustes(Up.T @ Bu + Vp.T @ Bv)


def joint_itq(Up: np.ndarray, Vp: np.ndarray, iters: int, R0: np.ndarray = None):
    """(R, objectives): the rotation after `iters` alternations from R0
    (identity when None) and Q after 0, 1, ..., iters of them."""
    r_p = np.asarray(Up).shape[1]
    R = np.eye(r_p) if R0 is None else np.asarray(R0, dtype=np.float64)
    q = [objective(Up, Vp, R)]
    for _ in range(iters):
        R = itq_step(Up, Vp, R)
        q.append(objective(Up, Vp, R))
    return R, q
