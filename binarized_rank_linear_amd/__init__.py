"""Python binding of liblittlebit.so (the LittleBit layer forward on MI355X).

Argument marshalling only: every step of the layer runs in the HIP library.
PyTorch provides device memory and the current HIP stream.  Importing this
package does not need a GPU; calling the library's compute entry points does.
If the shared library is missing, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblittlebit.so")

LB_OK = 0
LB_EINVAL = -1
LB_EUNSUPPORTED = -2
LB_EALIGN = -3
LB_EWORKSPACE = -4
LB_EHIP = -5
LB_EDEVICE = -6

LB_F32 = 0
LB_BF16 = 1

LB_PATH_AUTO = 0
LB_PATH_DECODE = 1
LB_PATH_PREFILL = 2
LB_PATH_DECODE_VALU = 3
LB_GROUP_FAULT_TEST = 1 << 8

LB_FAULT_HANDOFF_TIMEOUT = 1
LB_FAULT_STALE_WORKSPACE = 2

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


class lb_factors(ctypes.Structure):
    _fields_ = [("v_bits", _vp), ("u_bits", _vp), ("g", _vp), ("l", _vp), ("h", _vp),
                ("ld_v", _i64), ("ld_u", _i64)]


class lb_linear_desc(ctypes.Structure):
    _fields_ = [("x", _vp), ("y", _vp), ("w", lb_factors), ("d_in", _i64), ("d_out", _i64),
                ("r", _i64), ("residual", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class lb_linear_call(ctypes.Structure):
    _fields_ = [("x", _vp), ("y", _vp), ("w", lb_factors), ("d_in", _i64), ("d_out", _i64),
                ("r", _i64), ("T", _i64), ("residual", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("y_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class lb_decoder_layer(ctypes.Structure):
    _fields_ = [("q", lb_factors), ("k", lb_factors), ("v", lb_factors), ("o", lb_factors),
                ("gate", lb_factors), ("up", lb_factors), ("down", lb_factors),
                ("d_model", _i64), ("d_ff", _i64), ("n_heads", _i64), ("n_kv_heads", _i64),
                ("r_qo", _i64), ("r_kv", _i64), ("r_gu", _i64), ("r_down", _i64),
                ("residual", ctypes.c_int32), ("eps", ctypes.c_float)]


class LBError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (%d)" % (what, status_string(status), status))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("liblittlebit.so is not built (python -m binarized_rank_linear_amd.build)")
        # torch ships its own HIP runtime under the same soname; load it first so
        # the library binds to that runtime instead of pulling in a second copy
        # whose streams and allocations torch's would not recognise.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.lb_version.restype = ctypes.c_int
        L.lb_status_string.argtypes = [ctypes.c_int]
        L.lb_status_string.restype = ctypes.c_char_p
        L.lb_last_hip_error.argtypes = []
        L.lb_last_hip_error.restype = ctypes.c_char_p
        L.lb_rank_for_budget.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int,
                                         ctypes.POINTER(_i64), ctypes.POINTER(_i64)]
        L.lb_rank_for_budget.restype = ctypes.c_int
        L.lb_packed_ld.argtypes = [_i64]
        L.lb_packed_ld.restype = _i64
        L.lb_packed_ld_aligned.argtypes = [_i64]
        L.lb_packed_ld_aligned.restype = _i64
        L.lb_packed_words.argtypes = [_i64, _i64, ctypes.c_int, _i64]
        L.lb_packed_words.restype = _i64
        L.lb_pack_signs.argtypes = [_vp, _i64, _i64, ctypes.c_int, _vp, _i64, _vp]
        L.lb_pack_signs.restype = ctypes.c_int
        L.lb_linear_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_uint]
        L.lb_linear_workspace_bytes.restype = _sz
        L.lb_linear_forward.argtypes = [_vp, ctypes.c_int, _vp, ctypes.c_int,
                                        ctypes.POINTER(lb_factors), _i64, _i64, _i64, _i64,
                                        ctypes.c_int, _vp, _sz, ctypes.c_uint, _vp]
        L.lb_linear_forward.restype = ctypes.c_int
        L.lb_mlp_workspace_bytes.argtypes = [_i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                             ctypes.c_uint]
        L.lb_mlp_workspace_bytes.restype = _sz
        L.lb_mlp_forward.argtypes = [_vp, ctypes.c_int, _vp, ctypes.c_int,
                                     ctypes.POINTER(lb_factors), ctypes.POINTER(lb_factors),
                                     ctypes.POINTER(lb_factors), _i64, _i64, _i64, _i64, _i64,
                                     ctypes.c_int, _vp, _sz, ctypes.c_uint, _vp]
        L.lb_mlp_forward.restype = ctypes.c_int
        L.lb_grouped_workspace_bytes.argtypes = [ctypes.POINTER(lb_linear_desc), ctypes.c_int,
                                                 _i64, ctypes.c_uint]
        L.lb_grouped_workspace_bytes.restype = _sz
        L.lb_grouped_prepare.argtypes = [ctypes.POINTER(lb_linear_desc), ctypes.c_int, _i64,
                                         ctypes.c_int, ctypes.c_int, _vp, _sz, ctypes.c_uint, _vp]
        L.lb_grouped_prepare.restype = ctypes.c_int
        L.lb_grouped_run.argtypes = [_vp, _vp]
        L.lb_grouped_run.restype = ctypes.c_int
        L.lb_grouped_run_stage.argtypes = [_vp, ctypes.c_int, _vp]
        L.lb_grouped_run_stage.restype = ctypes.c_int
        L.lb_grouped_release.argtypes = [_vp]
        L.lb_grouped_release.restype = ctypes.c_int
        L.lb_linear_grouped_workspace_bytes.argtypes = [ctypes.POINTER(lb_linear_call), ctypes.c_int]
        L.lb_linear_grouped_workspace_bytes.restype = _sz
        L.lb_linear_forward_grouped.argtypes = [ctypes.POINTER(lb_linear_call), ctypes.c_int, _vp, _sz, _vp]
        L.lb_linear_forward_grouped.restype = ctypes.c_int
        L.lb_device_faults.argtypes = [_vp, ctypes.POINTER(ctypes.c_uint32)]
        L.lb_device_faults.restype = ctypes.c_int
        L.lb_linear_path.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_uint]
        L.lb_linear_path.restype = ctypes.c_int
        L.lb_linear_forward_noalloc.argtypes = [_vp, ctypes.c_int, _vp, ctypes.c_int,
                                                ctypes.POINTER(lb_factors), _i64, _i64, _i64, _i64,
                                                ctypes.c_int, ctypes.c_uint, _vp]
        L.lb_linear_forward_noalloc.restype = ctypes.c_int
        L.lb_linear_stage1.argtypes = [_vp, ctypes.c_int, _vp, ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(lb_factors), _i64, _i64, _i64, _i64, ctypes.c_int,
                                       _vp, _sz, ctypes.c_uint, _vp]
        L.lb_linear_stage1.restype = ctypes.c_int
        L.lb_linear_stage2.argtypes = [_vp, ctypes.c_int, _vp, ctypes.c_int, ctypes.POINTER(lb_factors),
                                       _i64, _i64, _i64, _i64, ctypes.c_int, _vp, _sz, ctypes.c_uint, _vp]
        L.lb_linear_stage2.restype = ctypes.c_int
        L.lb_decoder_layer_workspace_bytes.argtypes = [ctypes.POINTER(lb_decoder_layer), _i64]
        L.lb_decoder_layer_workspace_bytes.restype = _sz
        L.lb_decoder_layer_forward.argtypes = [ctypes.POINTER(lb_decoder_layer), _vp, _vp, _i64, _vp, _sz, _vp]
        L.lb_decoder_layer_forward.restype = ctypes.c_int
        L.lb_dual_svid_workspace_bytes.argtypes = [_i64, _i64, _i64, ctypes.c_int]
        L.lb_dual_svid_workspace_bytes.restype = _sz
        L.lb_dual_svid.argtypes = [_vp, _i64, _i64, _i64, ctypes.c_int, ctypes.POINTER(lb_factors), _vp, _vp,
                                   _vp, _sz, _vp]
        L.lb_dual_svid.restype = ctypes.c_int
        L.lb_dual_svid_itq_workspace_bytes.argtypes = [_i64, _i64, _i64, ctypes.c_int]
        L.lb_dual_svid_itq_workspace_bytes.restype = _sz
        L.lb_dual_svid_itq.argtypes = [_vp, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                       ctypes.POINTER(lb_factors), _vp, _vp, _vp, _sz, _vp]
        L.lb_dual_svid_itq.restype = ctypes.c_int
        L.lb_joint_itq_workspace_bytes.argtypes = [_i64, _i64, _i64]
        L.lb_joint_itq_workspace_bytes.restype = _sz
        L.lb_joint_itq.argtypes = [_vp, _vp, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _sz, _vp]
        L.lb_joint_itq.restype = ctypes.c_int
        L.lb_ceiling_stream_read.argtypes = [_vp, _sz, _vp, ctypes.c_int, _vp]
        L.lb_ceiling_stream_read.restype = ctypes.c_int
        L.lb_ceiling_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, _vp, ctypes.c_int, _vp]
        L.lb_ceiling_mfma_bf16.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lb_status_string(status).decode()


def _check(rc: int, what: str):
    if rc != LB_OK:
        if rc == LB_EHIP:
            what += " [%s]" % lib().lb_last_hip_error().decode()
        raise LBError(rc, what)


# ----------------------------------------------------------------------------
# host-side helpers
# ----------------------------------------------------------------------------

def rank_for_budget(d_in: int, d_out: int, b_num: int, b_den: int, residual: bool):
    r = _i64()
    rp = _i64()
    _check(lib().lb_rank_for_budget(d_in, d_out, b_num, b_den, int(residual),
                                    ctypes.byref(r), ctypes.byref(rp)), "lb_rank_for_budget")
    return r.value, rp.value


def packed_ld(n_other: int) -> int:
    return lib().lb_packed_ld(n_other)


def packed_ld_aligned(n_other: int) -> int:
    return lib().lb_packed_ld_aligned(n_other)


def packed_words(rows: int, cols: int, axis: int, ld: int) -> int:
    return lib().lb_packed_words(rows, cols, axis, ld)


def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return LB_F32
    if dt == torch.bfloat16:
        return LB_BF16
    raise ValueError("activation dtype must be float32 or bfloat16, got %s" % dt)


def _stream_ptr(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _dev_check(*tensors):
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("tensor must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensor must be contiguous")


def workspace(nbytes: int, device=None):
    """A device byte buffer of at least nbytes (torch allocations are 256-aligned)."""
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device or "cuda")


# ----------------------------------------------------------------------------
# sign packing
# ----------------------------------------------------------------------------

def pack_signs(src, axis: int, ld: Optional[int] = None, out=None, stream=None):
    """Packed sign words (int32 tensor viewed as uint32 words) of a 2-D fp32 GPU tensor."""
    torch = _torch()
    _dev_check(src)
    if src.dtype != torch.float32 or src.dim() != 2:
        raise ValueError("src must be a 2-D float32 tensor")
    rows, cols = src.shape
    n_pack, n_other = (rows, cols) if axis == 0 else (cols, rows)
    ld = packed_ld(n_other) if ld is None else ld
    planes = (n_pack + 31) // 32
    if out is None:
        out = torch.empty((planes, ld), dtype=torch.int32, device=src.device)
    elif out.numel() < planes * ld or out.dtype != torch.int32:
        raise ValueError("out too small or not int32")
    _check(lib().lb_pack_signs(src.data_ptr(), rows, cols, axis, out.data_ptr(), ld,
                               _stream_ptr(stream)), "lb_pack_signs")
    return out


class PackedLinear:
    """Packed factors and fp16 scales of one LittleBit linear on the GPU.

    Layout (littlebit.h): v_bits [P][ceil(d_in/32)][ld_v], u_bits
    [P][ceil(r_p/32)][ld_u], g [P][d_in], l [P][r_p], h [P][d_out] (fp16 bits).
    """

    def __init__(self, d_in, d_out, r, residual, v_bits, u_bits, g, l, h, ld_v, ld_u):
        self.d_in, self.d_out, self.r, self.residual = d_in, d_out, r, bool(residual)
        self.P = 2 if residual else 1
        self.r_p = r // self.P
        self.v_bits, self.u_bits, self.g, self.l, self.h = v_bits, u_bits, g, l, h
        self.ld_v, self.ld_u = ld_v, ld_u

    @classmethod
    def from_factors(cls, U, V, h, g, l, stream=None):
        """Pack float factors on the GPU.  U [P][d_out][r_p], V [P][d_in][r_p]
        float32 cuda tensors; h, g, l [P][*] float16 (or int16 bit) tensors."""
        torch = _torch()
        _dev_check(U, V, h, g, l)
        P, d_out, r_p = U.shape
        d_in = V.shape[1]
        if V.shape != (P, d_in, r_p):
            raise ValueError("U and V shapes disagree")
        ld_v, ld_u = packed_ld_aligned(r_p), packed_ld_aligned(d_out)
        kw_v, kw_u = (d_in + 31) // 32, (r_p + 31) // 32
        v_bits = torch.empty((P, kw_v, ld_v), dtype=torch.int32, device=U.device)
        u_bits = torch.empty((P, kw_u, ld_u), dtype=torch.int32, device=U.device)
        for p in range(P):
            pack_signs(V[p], 0, ld_v, out=v_bits[p], stream=stream)
            pack_signs(U[p], 1, ld_u, out=u_bits[p], stream=stream)
        as16 = lambda t: t.contiguous().view(torch.int16) if t.dtype in (torch.float16, torch.int16) \
            else t.to(torch.float16).contiguous().view(torch.int16)
        return cls(d_in, d_out, P * r_p, P == 2, v_bits, u_bits, as16(g), as16(l), as16(h),
                   ld_v, ld_u)

    def struct(self) -> lb_factors:
        return lb_factors(self.v_bits.data_ptr(), self.u_bits.data_ptr(), self.g.data_ptr(),
                          self.l.data_ptr(), self.h.data_ptr(), self.ld_v, self.ld_u)

    def packed_bytes(self) -> int:
        return (self.v_bits.numel() + self.u_bits.numel()) * 4

    def tight_sign_bytes(self) -> int:
        return self.r * (self.d_in + self.d_out) // 8

    def scale_bytes(self) -> int:
        return 2 * self.P * (self.d_in + self.d_out + self.r_p)


def linear_workspace_bytes(layer: PackedLinear, T: int, flags: int = 0) -> int:
    return lib().lb_linear_workspace_bytes(layer.d_in, layer.d_out, layer.r, T,
                                           int(layer.residual), flags)


def linear_forward(x, layer: PackedLinear, out_dtype=None, flags: int = LB_PATH_AUTO,
                   ws=None, out=None, stream=None):
    """y [T][d_out] = LittleBit layer(x [T][d_in]) on the GPU."""
    torch = _torch()
    _dev_check(x)
    T, d_in = x.shape
    if d_in != layer.d_in:
        raise ValueError("x has %d features, layer expects %d" % (d_in, layer.d_in))
    out_dtype = out_dtype or x.dtype
    if out is None:
        out = torch.empty((T, layer.d_out), dtype=out_dtype, device=x.device)
    _dev_check(out)
    need = linear_workspace_bytes(layer, T, flags)
    if ws is None or ws.numel() < need:
        ws = workspace(need, x.device)
    f = layer.struct()
    _check(lib().lb_linear_forward(x.data_ptr(), _dtype_code(x.dtype), out.data_ptr(),
                                   _dtype_code(out.dtype), ctypes.byref(f), layer.d_in,
                                   layer.d_out, layer.r, T, int(layer.residual), ws.data_ptr(),
                                   ws.numel(), flags, _stream_ptr(stream)), "lb_linear_forward")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20


def linear_forward_noalloc(x, layer: PackedLinear, out_dtype=None, flags: int = LB_PATH_AUTO,
                           out=None, stream=None):
    """lb_linear_forward_noalloc: the library's own fixed workspace (no
    allocation by the library; `out` may be passed to avoid torch's)."""
    torch = _torch()
    _dev_check(x)
    T, d_in = x.shape
    if d_in != layer.d_in:
        raise ValueError("x has %d features, layer expects %d" % (d_in, layer.d_in))
    out_dtype = out_dtype or x.dtype
    if out is None:
        out = torch.empty((T, layer.d_out), dtype=out_dtype, device=x.device)
    _dev_check(out)
    f = layer.struct()
    _check(lib().lb_linear_forward_noalloc(x.data_ptr(), _dtype_code(x.dtype), out.data_ptr(),
                                           _dtype_code(out.dtype), ctypes.byref(f), layer.d_in,
                                           layer.d_out, layer.r, T, int(layer.residual), flags,
                                           _stream_ptr(stream)), "lb_linear_forward_noalloc")
    return out


def linear_stage1(x, layer: PackedLinear, t_dtype=None, out_dtype=None, flags: int = LB_PATH_AUTO,
                  ws=None, out=None, stream=None):
    """The latents t [T][r] = l (.) sign(V)^T (g (.) x) per path (lb_linear_stage1).
    out_dtype: the dtype of the layer's output, which selects the kernels."""
    torch = _torch()
    _dev_check(x)
    T, d_in = x.shape
    if d_in != layer.d_in:
        raise ValueError("x has %d features, layer expects %d" % (d_in, layer.d_in))
    t_dtype = t_dtype or torch.float32
    out_dtype = out_dtype or x.dtype
    if out is None:
        out = torch.empty((T, layer.r), dtype=t_dtype, device=x.device)
    _dev_check(out)
    need = linear_workspace_bytes(layer, T, flags)
    if ws is None or ws.numel() < need:
        ws = workspace(need, x.device)
    f = layer.struct()
    _check(lib().lb_linear_stage1(x.data_ptr(), _dtype_code(x.dtype), out.data_ptr(), _dtype_code(out.dtype),
                                  _dtype_code(out_dtype), ctypes.byref(f), layer.d_in, layer.d_out, layer.r, T,
                                  int(layer.residual), ws.data_ptr(), ws.numel(), flags, _stream_ptr(stream)),
           "lb_linear_stage1")
    return out


def linear_stage2(t, layer: PackedLinear, out_dtype, flags: int = LB_PATH_AUTO, ws=None, out=None,
                  stream=None):
    """y [T][d_out] from the latents t [T][r] (lb_linear_stage2)."""
    torch = _torch()
    _dev_check(t)
    T, r = t.shape
    if r != layer.r:
        raise ValueError("t has %d latents, layer has %d" % (r, layer.r))
    if out is None:
        out = torch.empty((T, layer.d_out), dtype=out_dtype, device=t.device)
    _dev_check(out)
    need = linear_workspace_bytes(layer, T, flags)
    if ws is None or ws.numel() < need:
        ws = workspace(need, t.device)
    f = layer.struct()
    _check(lib().lb_linear_stage2(t.data_ptr(), _dtype_code(t.dtype), out.data_ptr(), _dtype_code(out.dtype),
                                  ctypes.byref(f), layer.d_in, layer.d_out, layer.r, T, int(layer.residual),
                                  ws.data_ptr(), ws.numel(), flags, _stream_ptr(stream)), "lb_linear_stage2")
    return out


def mlp_workspace_bytes(gate: PackedLinear, down: PackedLinear, T: int, flags: int = 0) -> int:
    return lib().lb_mlp_workspace_bytes(gate.d_in, gate.d_out, gate.r, down.r, T,
                                        int(gate.residual), flags)


def mlp_forward(x, gate: PackedLinear, up: PackedLinear, down: PackedLinear, out_dtype=None,
                flags: int = LB_PATH_AUTO, ws=None, out=None, stream=None):
    """y = down(silu(gate(x)) * up(x)) on the GPU."""
    torch = _torch()
    _dev_check(x)
    T, d_model = x.shape
    out_dtype = out_dtype or x.dtype
    if out is None:
        out = torch.empty((T, d_model), dtype=out_dtype, device=x.device)
    need = mlp_workspace_bytes(gate, down, T, flags)
    if ws is None or ws.numel() < need:
        ws = workspace(need, x.device)
    fg, fu, fd = gate.struct(), up.struct(), down.struct()
    _check(lib().lb_mlp_forward(x.data_ptr(), _dtype_code(x.dtype), out.data_ptr(),
                                _dtype_code(out.dtype), ctypes.byref(fg), ctypes.byref(fu),
                                ctypes.byref(fd), d_model, gate.d_out, gate.r, down.r, T,
                                int(gate.residual), ws.data_ptr(), ws.numel(), flags,
                                _stream_ptr(stream)), "lb_mlp_forward")
    return out


class DecoderLayer:
    """One decoder layer at decode time (lb_decoder_layer_forward): pre-norm
    attention over a one-token context with q, k, v, o LittleBit linears, then
    a LittleBit SwiGLU MLP, both with residuals.  bf16 in and out."""

    def __init__(self, q, k, v, o, gate, up, down, n_heads: int, n_kv_heads: int, eps: float = 1e-6):
        self.lin = dict(q=q, k=k, v=v, o=o, gate=gate, up=up, down=down)
        self.d_model, self.d_ff = q.d_in, gate.d_out
        self.n_heads, self.n_kv_heads, self.eps = n_heads, n_kv_heads, eps
        self.desc = lb_decoder_layer(q.struct(), k.struct(), v.struct(), o.struct(), gate.struct(),
                                     up.struct(), down.struct(), q.d_in, gate.d_out, n_heads, n_kv_heads,
                                     q.r, k.r, gate.r, down.r, int(q.residual), eps)

    def workspace_bytes(self, T: int) -> int:
        return lib().lb_decoder_layer_workspace_bytes(ctypes.byref(self.desc), T)

    def forward(self, x, out=None, ws=None, stream=None):
        torch = _torch()
        _dev_check(x)
        T = x.shape[0]
        if x.dtype != torch.bfloat16 or x.shape != (T, self.d_model):
            raise ValueError("x must be bf16 [T][d_model]")
        if out is None:
            out = torch.empty_like(x)
        need = self.workspace_bytes(T)
        if ws is None or ws.numel() < need:
            ws = workspace(max(need, 1), x.device)
        _check(lib().lb_decoder_layer_forward(ctypes.byref(self.desc), x.data_ptr(), out.data_ptr(), T,
                                              ws.data_ptr(), ws.numel(), _stream_ptr(stream)),
               "lb_decoder_layer_forward")
        return out


def dual_svid(W, r: int, residual: bool, float_factors: bool = False, ws=None, stream=None,
              itq_iters: int = 0):
    """Dual-SVID initialisation (lb_dual_svid, or lb_dual_svid_itq with
    itq_iters > 0: the LittleBit-2 Joint-ITQ rotation of each path's factors
    first) of a LittleBit linear from a dense fp32 weight W [d_out][d_in] on
    the GPU.  Returns the PackedLinear, and with float_factors also the fp32
    U' [P][d_out][r_p] and V' [P][d_in][r_p]."""
    torch = _torch()
    _dev_check(W)
    if W.dtype != torch.float32 or W.dim() != 2:
        raise ValueError("W must be a 2-D float32 tensor")
    W = W.contiguous()
    d_out, d_in = W.shape
    P = 2 if residual else 1
    r_p = r // P
    ld_v, ld_u = packed_ld_aligned(r_p), packed_ld_aligned(d_out)
    dev = W.device
    v_bits = torch.empty((P, (d_in + 31) // 32, ld_v), dtype=torch.int32, device=dev)
    u_bits = torch.empty((P, (r_p + 31) // 32, ld_u), dtype=torch.int32, device=dev)
    g = torch.empty((P, d_in), dtype=torch.int16, device=dev)
    l = torch.empty((P, r_p), dtype=torch.int16, device=dev)
    h = torch.empty((P, d_out), dtype=torch.int16, device=dev)
    lin = PackedLinear(d_in, d_out, r, residual, v_bits, u_bits, g, l, h, ld_v, ld_u)
    U = torch.empty((P, d_out, r_p), dtype=torch.float32, device=dev) if float_factors else None
    V = torch.empty((P, d_in, r_p), dtype=torch.float32, device=dev) if float_factors else None
    if itq_iters > 0:
        need = lib().lb_dual_svid_itq_workspace_bytes(d_out, d_in, r, int(residual))
    else:
        need = lib().lb_dual_svid_workspace_bytes(d_out, d_in, r, int(residual))
    if ws is None or ws.numel() < need:
        ws = workspace(max(need, 1), dev)
    f = lin.struct()
    up = U.data_ptr() if U is not None else None
    vp = V.data_ptr() if V is not None else None
    if itq_iters > 0:
        _check(lib().lb_dual_svid_itq(W.data_ptr(), d_out, d_in, r, int(residual), int(itq_iters),
                                      ctypes.byref(f), up, vp, ws.data_ptr(), ws.numel(), _stream_ptr(stream)),
               "lb_dual_svid_itq")
    else:
        _check(lib().lb_dual_svid(W.data_ptr(), d_out, d_in, r, int(residual), ctypes.byref(f), up, vp,
                                  ws.data_ptr(), ws.numel(), _stream_ptr(stream)), "lb_dual_svid")
    return (lin, U, V) if float_factors else lin


def joint_itq(U, V, iters: int, rot0=None, ws=None, stream=None):
    """Joint-ITQ (lb_joint_itq) of one path's float factors U' [d_out][r_p]
    and V' [d_in][r_p] (fp32 device tensors, rotated in place).  Returns
    (R [r_p][r_p] fp32, objective [iters + 1] fp64): the final rotation and the
    objective at the start and after each alternation."""
    torch = _torch()
    _dev_check(U, V)
    if U.dtype != torch.float32 or V.dtype != torch.float32 or U.dim() != 2 or V.dim() != 2:
        raise ValueError("U and V must be 2-D float32 tensors")
    if not (U.is_contiguous() and V.is_contiguous()):
        raise ValueError("U and V must be contiguous (they are rotated in place)")
    d_out, r_p = U.shape
    d_in = V.shape[0]
    if V.shape[1] != r_p:
        raise ValueError("U and V must have the same number of columns")
    if rot0 is not None:
        _dev_check(rot0)
        if rot0.dtype != torch.float32 or tuple(rot0.shape) != (r_p, r_p):
            raise ValueError("rot0 must be a float32 [r_p][r_p] tensor")
        rot0 = rot0.contiguous()
    R = torch.empty((r_p, r_p), dtype=torch.float32, device=U.device)
    obj = torch.empty((iters + 1,), dtype=torch.float64, device=U.device)
    need = lib().lb_joint_itq_workspace_bytes(d_out, d_in, r_p)
    if ws is None or ws.numel() < need:
        ws = workspace(max(need, 1), U.device)
    _check(lib().lb_joint_itq(U.data_ptr(), V.data_ptr(), d_out, d_in, r_p, int(iters),
                              rot0.data_ptr() if rot0 is not None else None, R.data_ptr(), obj.data_ptr(),
                              ws.data_ptr(), ws.numel(), _stream_ptr(stream)), "lb_joint_itq")
    return R, obj


def device_faults(stream=None) -> int:
    """Waits for the stream, then reads and clears the device's fault bits
    (LB_FAULT_*); 0 if no kernel reported a fault."""
    f = ctypes.c_uint32(0)
    rc = lib().lb_device_faults(_stream_ptr(stream), ctypes.byref(f))
    if rc not in (LB_OK, LB_EDEVICE):
        _check(rc, "lb_device_faults")
    return f.value


def linear_path(d_in: int, d_out: int, r: int, T: int, residual: bool, x_dtype, y_dtype,
                flags: int = LB_PATH_AUTO) -> int:
    """The kernel family (LB_PATH_DECODE / LB_PATH_PREFILL / LB_PATH_DECODE_VALU)
    lb_linear_forward would run for these sizes (host only)."""
    rc = lib().lb_linear_path(d_in, d_out, r, T, int(residual), _dtype_code(x_dtype),
                              _dtype_code(y_dtype), flags)
    if rc < 0:
        _check(rc, "lb_linear_path")
    return rc


def _calls(items, flags):
    arr = (lb_linear_call * len(items))()
    for i, (x, y, layer) in enumerate(items):
        _dev_check(x, y)
        if x.shape[-1] != layer.d_in or y.shape[-1] != layer.d_out or x.shape[0] != y.shape[0]:
            raise ValueError("item %d: x/y shapes do not match the layer" % i)
        arr[i] = lb_linear_call(x.data_ptr(), y.data_ptr(), layer.struct(), layer.d_in, layer.d_out,
                                layer.r, x.shape[0], int(layer.residual), _dtype_code(x.dtype),
                                _dtype_code(y.dtype), flags)
    return arr


def grouped_workspace_bytes(items, flags: int = LB_PATH_AUTO) -> int:
    return lib().lb_linear_grouped_workspace_bytes(_calls(items, flags), len(items))


def linear_forward_grouped(items, flags: int = LB_PATH_AUTO, ws=None, stream=None):
    """The stateless grouped call: items is a sequence of (x, y, PackedLinear);
    every y is recomputed from its x (lb_linear_forward_grouped)."""
    arr = _calls(items, flags)
    need = lib().lb_linear_grouped_workspace_bytes(arr, len(items))
    if ws is None or ws.numel() < need:
        ws = workspace(need, items[0][0].device)
    _check(lib().lb_linear_forward_grouped(arr, len(items), ws.data_ptr(), ws.numel(),
                                           _stream_ptr(stream)), "lb_linear_forward_grouped")
    return ws


class Group:
    """Many independent linears run together (layer stacks).  Inputs and
    outputs are bound at construction; run() recomputes every output."""

    def __init__(self, items: Sequence, T: int, x_dtype, y_dtype, flags: int = LB_PATH_AUTO,
                 stream=None):
        """items: sequence of (x tensor, y tensor, PackedLinear)."""
        self.items = list(items)
        n = len(self.items)
        arr = (lb_linear_desc * n)()
        for i, (x, y, layer) in enumerate(self.items):
            arr[i] = lb_linear_desc(x.data_ptr(), y.data_ptr(), layer.struct(), layer.d_in,
                                    layer.d_out, layer.r, int(layer.residual), 0)
        self._descs = arr
        need = lib().lb_grouped_workspace_bytes(arr, n, T, flags)
        if need == 0:
            raise LBError(LB_EINVAL, "lb_grouped_workspace_bytes")
        self.ws = workspace(need, self.items[0][0].device)
        _check(lib().lb_grouped_prepare(arr, n, T, _dtype_code(x_dtype), _dtype_code(y_dtype),
                                        self.ws.data_ptr(), self.ws.numel(), flags,
                                        _stream_ptr(stream)), "lb_grouped_prepare")

    def run(self, stream=None):
        _check(lib().lb_grouped_run(self.ws.data_ptr(), _stream_ptr(stream)), "lb_grouped_run")

    def run_stage(self, stage: int, stream=None):
        _check(lib().lb_grouped_run_stage(self.ws.data_ptr(), stage, _stream_ptr(stream)),
               "lb_grouped_run_stage")

    def release(self):
        """Forget the group's host-side record (lb_grouped_release); idempotent."""
        ws = getattr(self, "ws", None)
        if ws is not None:
            lib().lb_grouped_release(ws.data_ptr())
            self.ws = None

    def __del__(self):
        try:
            self.release()
        except Exception:
            pass
