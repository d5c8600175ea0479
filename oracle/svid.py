"""Dual-SVID initialisation of a LittleBit linear from a dense weight, in
numpy fp64 (TEST INFRASTRUCTURE ONLY, like the rest of this package: the
product path never imports it).

Written from the pages' description of the initialisation (sesamedisk, "How
low-rank binarization works", the Dual-SVID paragraph; mlsanity, abstract:
Dual Sign-Value-Independent Decomposition and residual compensation):

1. a truncated SVD of W (d_out x d_in) to r_p singular triplets, the square
   root of each singular value put into both factors: U' = U_r sqrt(S_r),
   V' = V_r sqrt(S_r), so W_r = U' V'^T;
2. the binary factors start as sign(U'), sign(V');
3. the magnitudes |U'| and |V'| are each replaced by their best rank-1
   approximation: |U'| ~ h l_u^T, |V'| ~ g l_v^T (h: rows, g: input columns,
   l_u, l_v: latents), and the latent scale is l = l_u (.) l_v;
4. with the residual path, the same is done to the remainder W - W_1, where
   W_1 is the first path's layer as stored (fp16 scales).
With Joint-ITQ (LittleBit-2; oracle/itq.py) the two factors of each path are
rotated by the shared latent rotation between steps 1 and 2.

Readings where the pages leave a step open (each is a plain choice):
- the singular values are split evenly (sqrt into each factor);
- a rank-1 fit is the top singular pair of the nonnegative matrix, taken
  nonnegative (its Perron vectors; rounding-level negative entries are set to
  zero), with sqrt(sigma_1) in each of the two vectors;
- scales are stored as fp16 (round to nearest even), as the layer holds them,
  and the remainder for the residual path is taken against that stored layer.
"""
from __future__ import annotations

import numpy as np

from . import dense_weight
from . import itq as _itq


def rank1_nonneg(M: np.ndarray):
    """(a, b) with a b^T the best rank-1 approximation of the nonnegative M
    (Eckart-Young: the top singular pair), a and b nonnegative, the singular
    value split evenly between them."""
    M = np.asarray(M, dtype=np.float64)
    u, s, vt = np.linalg.svd(M, full_matrices=False)
    a, b = u[:, 0], vt[0]
    if a.sum() + b.sum() < 0:
        a, b = -a, -b
    a, b = np.maximum(a, 0.0), np.maximum(b, 0.0)
    r = np.sqrt(s[0])
    return r * a, r * b


def truncated_factors(W: np.ndarray, r_p: int):
    """U' [d_out][r_p], V' [d_in][r_p] with U' V'^T the best rank-r_p
    approximation of W and each factor holding sqrt of the singular values."""
    W = np.asarray(W, dtype=np.float64)
    u, s, vt = np.linalg.svd(W, full_matrices=False)
    root = np.sqrt(s[:r_p])
    return u[:, :r_p] * root[None, :], vt[:r_p].T * root[None, :]


def _f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float16)).view(np.uint16)


def svid_path(W: np.ndarray, r_p: int, f16: bool = True, itq_iters: int = 0):
    """One path: (U', V', h, g, l), the float factors (only their signs are
    kept by the layer) and the scales: fp16 bits, or fp64 values with f16
    False (to check the arithmetic apart from the storage rounding).  With
    itq_iters > 0 the factors are U' R and V' R, R from Joint-ITQ."""
    Up, Vp = truncated_factors(W, r_p)
    if itq_iters > 0:
        R, _ = _itq.joint_itq(Up, Vp, itq_iters)
        Up, Vp = Up @ R, Vp @ R
    h, l_u = rank1_nonneg(np.abs(Up))
    g, l_v = rank1_nonneg(np.abs(Vp))
    store = _f16_bits if f16 else (lambda a: np.asarray(a, dtype=np.float64))
    return Up, Vp, store(h), store(g), store(l_u * l_v)


def dual_svid(W: np.ndarray, r_p: int, residual: bool, f16: bool = True, itq_iters: int = 0):
    """The layer's factors, stacked path-major as the layer takes them:
    U [P][d_out][r_p], V [P][d_in][r_p] (fp64), h [P][d_out], g [P][d_in],
    l [P][r_p] (fp16 bits, or fp64 with f16 False).  itq_iters > 0: each
    path's factors are rotated by Joint-ITQ first (LittleBit-2)."""
    W = np.asarray(W, dtype=np.float64)
    paths = [svid_path(W, r_p, f16, itq_iters)]
    if residual:
        U1, V1, h1, g1, l1 = paths[0]
        W1 = dense_weight(U1[None], V1[None], h1[None], g1[None], l1[None])
        paths.append(svid_path(W - W1, r_p, f16, itq_iters))
    U = np.stack([p[0] for p in paths])
    V = np.stack([p[1] for p in paths])
    h, g, l = (np.stack([p[k] for p in paths]) for k in (2, 3, 4))
    return U, V, h, g, l


def reconstruction(U, V, h, g, l) -> np.ndarray:
    """The dense weight the initialised layer computes (all paths)."""
    return dense_weight(np.asarray(U), np.asarray(V), h, g, l)
