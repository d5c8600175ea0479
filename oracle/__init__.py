"""CPU oracle of the LittleBit linear layer forward (fp64).

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path (the HIP library
and its Python binding) never imports it, and it never imports them.

Two independent formulations live here:

* the factorised forward, in plain C (lb_oracle.c, built with gcc), in the
  order of Proposition 1 on the sesamedisk page ("What the method actually
  computes"): scale by g, contract with sign(V), scale by l, contract with
  sign(U), scale by h, sum the residual path;
* the dense reconstruction W = sum_p diag(h_p) sign(U_p) diag(l_p)
  sign(V_p)^T diag(g_p) (the same proposition read as one matrix), in numpy,
  used to pin the factorised C code on small shapes.

Inputs are widened to fp64 exactly (fp16 scales, bf16 or fp32 activations).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lb_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblb_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def build(force: bool = False) -> str:
    """Compile lb_oracle.c with gcc (OpenMP) into liblb_oracle.so."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_rank_for_budget.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, _i64p, _i64p]
        L.oracle_rank_for_budget.restype = ctypes.c_int
        L.oracle_pack_signs.argtypes = [_fp, _i64, _i64, ctypes.c_int, _u32p, _i64]
        L.oracle_pack_signs.restype = None
        L.oracle_unpack_signs.argtypes = [_u32p, _i64, _i64, ctypes.c_int, _i64, _dp]
        L.oracle_unpack_signs.restype = None
        L.oracle_linear_forward.argtypes = [_dp, _i64, _i64, _i64, _i64, ctypes.c_int,
                                            _fp, _fp, _dp, _dp, _dp, _dp, ctypes.c_int]
        L.oracle_linear_forward.restype = None
        L.oracle_linear_forward_rows.argtypes = [_dp, _i64, _i64, _i64, _i64, ctypes.c_int,
                                                 _fp, _fp, _dp, _dp, _dp, _i64p, _i64, _dp,
                                                 ctypes.c_int]
        L.oracle_linear_forward_rows.restype = None
        L.oracle_linear_latents.argtypes = [_dp, _i64, _i64, _i64, ctypes.c_int, _fp, _dp, _dp, _dp,
                                            ctypes.c_int]
        L.oracle_linear_latents.restype = None
        L.oracle_linear_from_latents.argtypes = [_dp, _i64, _i64, _i64, ctypes.c_int, _fp, _dp, _dp,
                                                 ctypes.c_int]
        L.oracle_linear_from_latents.restype = None
        L.oracle_mlp_forward.argtypes = ([_dp, _i64, _i64, _i64, ctypes.c_int, _i64, _i64]
                                         + [_fp, _fp, _dp, _dp, _dp] * 3 + [_dp, ctypes.c_int])
        L.oracle_mlp_forward.restype = None
        L.oracle_silu.argtypes = [ctypes.c_double]
        L.oracle_silu.restype = ctypes.c_double
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray, typ):
    return a.ctypes.data_as(typ)


# ----------------------------------------------------------------------------
# exact widening of the storage types to fp64
# ----------------------------------------------------------------------------

def widen_f16(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns (uint16) -> fp64, exactly."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64, exactly (bf16 is the top half of fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def widen_x(x: np.ndarray) -> np.ndarray:
    if x.dtype == np.uint16:
        return widen_bf16(x)
    return np.ascontiguousarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# rank rule and packing
# ----------------------------------------------------------------------------

def rank_for_budget(d_in: int, d_out: int, b_num: int, b_den: int, residual: bool):
    """(r_total, r_path) from the bit budget b = b_num / b_den, exact integers."""
    r = ctypes.c_int64()
    rp = ctypes.c_int64()
    rc = lib().oracle_rank_for_budget(d_in, d_out, b_num, b_den, int(residual),
                                      ctypes.byref(r), ctypes.byref(rp))
    if rc != 0:
        raise ValueError("rank rounds to zero for this budget")
    return r.value, rp.value


def pack_signs(src: np.ndarray, axis: int, ld: Optional[int] = None) -> np.ndarray:
    """Packed sign words of src (float32 [rows][cols]); see lb_oracle.c."""
    src = np.ascontiguousarray(src, dtype=np.float32)
    rows, cols = src.shape
    n_pack, n_other = (rows, cols) if axis == 0 else (cols, rows)
    ld = n_other if ld is None else ld
    assert ld >= n_other
    out = np.empty(((n_pack + 31) // 32, ld), np.uint32)
    lib().oracle_pack_signs(_ptr(src, _fp), rows, cols, axis, _ptr(out, _u32p), ld)
    return out


def unpack_signs(words: np.ndarray, rows: int, cols: int, axis: int) -> np.ndarray:
    words = np.ascontiguousarray(words, dtype=np.uint32)
    out = np.empty((rows, cols), np.float64)
    lib().oracle_unpack_signs(_ptr(words, _u32p), rows, cols, axis, words.shape[1],
                              _ptr(out, _dp))
    return out


# ----------------------------------------------------------------------------
# forward
# ----------------------------------------------------------------------------

def linear_forward(x: np.ndarray, U: np.ndarray, V: np.ndarray, h: np.ndarray,
                   g: np.ndarray, l: np.ndarray, nthreads: int = 0) -> np.ndarray:
    """Factorised forward (C).  x: fp32 [T][d_in] or bf16 bits; U [P][d_out][r_p],
    V [P][d_in][r_p] float32; h, g, l fp16 bits [P][*] (or float64 arrays)."""
    xd = widen_x(x)
    T, d_in = xd.shape
    P, d_out, r_p = U.shape
    assert V.shape == (P, d_in, r_p)
    U = np.ascontiguousarray(U, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    hd, gd, ldd = (_scale64(s) for s in (h, g, l))
    y = np.empty((T, d_out), np.float64)
    lib().oracle_linear_forward(_ptr(xd, _dp), T, d_in, d_out, r_p, P,
                                _ptr(U, _fp), _ptr(V, _fp), _ptr(hd, _dp), _ptr(gd, _dp),
                                _ptr(ldd, _dp), _ptr(y, _dp), nthreads)
    return y


def linear_forward_rows(x: np.ndarray, U, V, h, g, l, rows: Sequence[int],
                        nthreads: int = 0) -> np.ndarray:
    """Output rows `rows` (indices into d_out) of the factorised forward: [T][len(rows)]."""
    xd = widen_x(x)
    T, d_in = xd.shape
    P, d_out, r_p = U.shape
    U = np.ascontiguousarray(U, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    hd, gd, ldd = (_scale64(s) for s in (h, g, l))
    idx = np.ascontiguousarray(rows, dtype=np.int64)
    y = np.empty((T, len(idx)), np.float64)
    lib().oracle_linear_forward_rows(_ptr(xd, _dp), T, d_in, d_out, r_p, P,
                                     _ptr(U, _fp), _ptr(V, _fp), _ptr(hd, _dp), _ptr(gd, _dp),
                                     _ptr(ldd, _dp), _ptr(idx, _i64p), len(idx), _ptr(y, _dp),
                                     nthreads)
    return y


def linear_latents(x: np.ndarray, V: np.ndarray, g, l, nthreads: int = 0) -> np.ndarray:
    """The rank-r intermediate t [T][P*r_p] (path p in columns p*r_p..):
    t = l_p * (sign(V_p)^T (g_p * x)) per path (C)."""
    xd = widen_x(x)
    T, d_in = xd.shape
    P, _, r_p = V.shape
    V = np.ascontiguousarray(V, dtype=np.float32)
    gd, ldd = _scale64(g), _scale64(l)
    t = np.empty((T, P * r_p), np.float64)
    lib().oracle_linear_latents(_ptr(xd, _dp), T, d_in, r_p, P, _ptr(V, _fp), _ptr(gd, _dp),
                                _ptr(ldd, _dp), _ptr(t, _dp), nthreads)
    return t


def linear_from_latents(t: np.ndarray, U: np.ndarray, h, nthreads: int = 0) -> np.ndarray:
    """y [T][d_out] = sum_p h_p * (sign(U_p) t_p) from latents t [T][P*r_p] (C)."""
    td = np.ascontiguousarray(t, dtype=np.float64)
    P, d_out, r_p = U.shape
    T = td.shape[0]
    assert td.shape == (T, P * r_p)
    U = np.ascontiguousarray(U, dtype=np.float32)
    hd = _scale64(h)
    y = np.empty((T, d_out), np.float64)
    lib().oracle_linear_from_latents(_ptr(td, _dp), T, d_out, r_p, P, _ptr(U, _fp), _ptr(hd, _dp),
                                     _ptr(y, _dp), nthreads)
    return y


def mlp_forward(x: np.ndarray, gate, up, down, nthreads: int = 0) -> np.ndarray:
    """SwiGLU block y = down(silu(gate(x)) * up(x)).  gate/up/down are objects
    with U, V, h, g, l attributes (see synth.LayerInputs)."""
    xd = widen_x(x)
    T, d_model = xd.shape
    P, d_ff, r_gu = gate.U.shape
    r_dn = down.U.shape[2]
    arrays = []
    for f in (gate, up, down):
        arrays += [np.ascontiguousarray(f.U, np.float32), np.ascontiguousarray(f.V, np.float32)]
        arrays += [_scale64(s) for s in (f.h, f.g, f.l)]
    ptrs = [_ptr(a, _fp if a.dtype == np.float32 else _dp) for a in arrays]
    y = np.empty((T, d_model), np.float64)
    lib().oracle_mlp_forward(_ptr(xd, _dp), T, d_model, d_ff, P, r_gu, r_dn, *ptrs,
                             _ptr(y, _dp), nthreads)
    return y


# ----------------------------------------------------------------------------
# one decoder layer at decode time (numpy composition of the C linears)
# ----------------------------------------------------------------------------
# The pages keep the model architecture as it is and replace its dense linears
# by LittleBit linears (trove.briskstack page, overview; deniz.in, "Factorize
# first, then binarize"; the mlsanity page lists Llama 2 and GQA as the models
# it builds on).  The layer here is the Llama form: pre-RMSNorm, attention
# with grouped kv heads, SwiGLU MLP, residual adds.  Attention is over a
# context of one token, whose softmax weight is 1.

def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp64 values rounded to the nearest bf16 (8 significant bits, ties to
    even), kept in fp64.  With a = m * 2^e, 0.5 <= |m| < 1, the bf16 step is
    2^(e-8); below the smallest normal the step stays 2^-133."""
    a = np.asarray(a, dtype=np.float64)
    out = a.copy()
    nz = np.isfinite(a) & (a != 0)
    _, e = np.frexp(a[nz])
    step = np.ldexp(1.0, np.maximum(e, -125) - 8)
    out[nz] = np.round(a[nz] / step) * step        # numpy rounds halves to even
    return out


def rms_inverse(x: np.ndarray, eps: float) -> np.ndarray:
    """1 / sqrt(mean over channels of x^2 + eps), one value per token."""
    xd = widen_x(x)
    return 1.0 / np.sqrt(np.mean(xd * xd, axis=1) + eps)


def attend_one_token(v: np.ndarray, n_heads: int, n_kv_heads: int) -> np.ndarray:
    """Attention output [T][n_heads * d_head] over a context of one token:
    query head h reads value head h // (n_heads / n_kv_heads)."""
    T, d_kv = v.shape
    dh = d_kv // n_kv_heads
    grp = n_heads // n_kv_heads
    out = np.empty((T, n_heads * dh), np.float64)
    for h in range(n_heads):
        kv = h // grp
        out[:, h * dh:(h + 1) * dh] = v[:, kv * dh:(kv + 1) * dh]
    return out


def decoder_layer_forward(x: np.ndarray, lin: dict, n_heads: int, n_kv_heads: int, eps: float,
                          store=None, nthreads: int = 0) -> np.ndarray:
    """One decoder layer: a = x / rms(x); v = V(a);
    x1 = x + O(attend(v)); b = x1 / rms(x1); y = x1 + Down(silu(Gate(b)) * Up(b)).
    lin maps q, k, v, o, gate, up, down to objects with U, V, h, g, l.  The
    RMSNorm weights are taken as folded into the linears' g.  `store` (None or
    round_bf16) is applied to every tensor handed from one step to the next,
    to model an implementation that keeps them in a narrower type."""
    keep = store or (lambda a: a)
    f = lambda name, a: linear_forward(a, lin[name].U, lin[name].V, lin[name].h, lin[name].g,
                                       lin[name].l, nthreads)
    xd = widen_x(x)
    a = xd * rms_inverse(xd, eps)[:, None]
    v = keep(f("v", a))                  # q and k do not change a one-token attention
    x1 = keep(xd + f("o", attend_one_token(v, n_heads, n_kv_heads)))
    b = x1 * rms_inverse(x1, eps)[:, None]
    zg, zu = keep(f("gate", b)), keep(f("up", b))
    m = zg / (1.0 + np.exp(-zg)) * zu
    return x1 + f("down", m)


def _scale64(s: np.ndarray) -> np.ndarray:
    if s.dtype == np.uint16:
        return widen_f16(s)
    return np.ascontiguousarray(s, dtype=np.float64)


def silu(z: float) -> float:
    return lib().oracle_silu(z)


def max_threads() -> int:
    return lib().oracle_max_threads()


# ----------------------------------------------------------------------------
# dense reconstruction (numpy, fp64) -- the second formulation
# ----------------------------------------------------------------------------

def dense_weight(U: np.ndarray, V: np.ndarray, h, g, l) -> np.ndarray:
    """W [d_out][d_in] = sum_p diag(h_p) S_Up diag(l_p) S_Vp^T diag(g_p)."""
    P, d_out, r_p = U.shape
    d_in = V.shape[1]
    hd, gd, ldd = (_scale64(s).reshape(P, -1) for s in (h, g, l))
    W = np.zeros((d_out, d_in), np.float64)
    for p in range(P):
        SU = np.where(U[p] < 0, -1.0, 1.0)
        SV = np.where(V[p] < 0, -1.0, 1.0)
        W += (hd[p][:, None] * SU) @ (ldd[p][:, None] * SV.T) * gd[p][None, :]
    return W


def dense_forward(x: np.ndarray, U, V, h, g, l) -> np.ndarray:
    return widen_x(x) @ dense_weight(U, V, h, g, l).T


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    return float(num / den) if den > 0 else float(num)
