"""Host-side checks of the C ABI: the library loads without a GPU, exports
every function littlebit.h declares, and rejects bad arguments before it
touches the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import binarized_rank_linear_amd as lb
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "littlebit.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(lb_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_library_loads_and_exports_every_declared_symbol():
    L = lb.lib()
    names = _declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert lb.lib().lb_version() >> 16 >= 1


def test_status_strings():
    for rc in (lb.LB_OK, lb.LB_EINVAL, lb.LB_EUNSUPPORTED, lb.LB_EALIGN, lb.LB_EWORKSPACE, lb.LB_EHIP):
        assert lb.status_string(rc) and lb.status_string(rc) != "unknown status"


@pytest.mark.parametrize("d_in,d_out,bn,bd,res", [
    (1024, 1024, 1, 1, False), (1024, 3072, 55, 100, True), (3072, 1024, 55, 100, True),
    (4096, 4096, 1, 1, True), (4096, 11008, 1, 1, True), (11008, 4096, 1, 1, True),
    (5120, 5120, 55, 100, True), (5120, 1024, 55, 100, True), (5120, 17408, 55, 100, True),
    (17408, 5120, 55, 100, True), (8192, 8192, 1, 10, True), (8192, 1024, 1, 10, True),
    (8192, 28672, 1, 10, True), (28672, 8192, 1, 10, True), (4096, 4096, 1, 10, True),
    (123, 4567, 7, 3, False), (100000, 300, 5, 1, True)])
def test_rank_rule_matches_oracle(d_in, d_out, bn, bd, res):
    assert lb.rank_for_budget(d_in, d_out, bn, bd, res) == oracle.rank_for_budget(d_in, d_out, bn, bd, res)


def test_rank_rule_errors():
    with pytest.raises(lb.LBError) as e:
        lb.rank_for_budget(64, 64, 1, 10, False)
    assert e.value.status == lb.LB_EINVAL
    with pytest.raises(lb.LBError):
        lb.rank_for_budget(0, 64, 1, 1, False)


def test_packed_sizes():
    assert lb.packed_ld(1) == 4 and lb.packed_ld(304) == 304 and lb.packed_ld(305) == 308
    assert lb.packed_ld_aligned(1) == 32 and lb.packed_ld_aligned(304) == 320 and lb.packed_ld_aligned(320) == 320
    assert lb.packed_ld_aligned(0) == 0
    assert lb.packed_words(100, 7, 0, 8) == 4 * 8
    assert lb.packed_words(7, 100, 1, 8) == 4 * 8
    assert lb.packed_words(7, 100, 1, 6) == 0        # ld below the other axis
    assert lb.packed_words(7, 100, 2, 8) == 0        # bad axis


FAKE = 0x10000000   # never dereferenced: every call below fails its checks first


def _factors(ld_v=512, ld_u=1024, **kw):
    f = lb.lb_factors(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000,
                      FAKE + 0x4000000, ld_v, ld_u)
    for k, v in kw.items():
        setattr(f, k, v)
    return f


def _fwd(x=FAKE + 0x5000000, xd=lb.LB_F32, y=FAKE + 0x6000000, yd=lb.LB_F32, f=None, d_in=1024,
         d_out=1024, r=512, T=1, res=0, ws=None, ws_bytes=1 << 20, flags=0):
    f = f if f is not None else _factors()
    return lb.lib().lb_linear_forward(x, xd, y, yd, ctypes.byref(f), d_in, d_out, r, T, res,
                                      ws, ws_bytes, flags, None)


def test_linear_forward_argument_errors():
    L = lb.lib()
    assert _fwd(d_in=0) == lb.LB_EINVAL
    assert _fwd(r=0) == lb.LB_EINVAL
    assert _fwd(T=-1) == lb.LB_EINVAL
    assert _fwd(r=511, res=1, f=_factors(ld_v=256)) == lb.LB_EINVAL     # odd total rank
    assert _fwd(xd=7) == lb.LB_EINVAL
    assert _fwd(x=0) == lb.LB_EINVAL
    assert _fwd(x=0, y=0, T=0) == lb.LB_OK                              # empty tensors
    assert _fwd(f=_factors(ld_v=500)) == lb.LB_EINVAL                   # ld_v < r_p
    assert _fwd(f=_factors(ld_v=514)) == lb.LB_EALIGN                   # ld_v % 4
    assert _fwd(f=_factors(v_bits=FAKE + 4)) == lb.LB_EALIGN            # bits not 16-aligned
    assert _fwd(f=_factors(g=0)) == lb.LB_EINVAL
    assert _fwd(x=FAKE + 0x5000001) == lb.LB_EALIGN                     # fp32 x misaligned
    assert _fwd(y=FAKE + 0x5000000) == lb.LB_EINVAL                     # y overlaps x
    assert _fwd(flags=9) == lb.LB_EINVAL                                # unknown path
    assert _fwd(flags=lb.LB_PATH_PREFILL, T=64) == lb.LB_EUNSUPPORTED   # GEMM path, fp32 out
    assert _fwd(ws=None) == lb.LB_EWORKSPACE
    need = L.lb_linear_workspace_bytes(1024, 1024, 512, 1, 0, 0)
    assert need > 0
    assert _fwd(ws=FAKE + 0x7000000, ws_bytes=need - 1) == lb.LB_EWORKSPACE
    assert _fwd(ws=FAKE + 0x7000001, ws_bytes=need) == lb.LB_EALIGN
    assert _fwd(ws=FAKE + 0x5000000, ws_bytes=need) == lb.LB_EINVAL     # ws overlaps x
    # T == 0 is a no-op that still validates its arguments
    assert _fwd(T=0) == lb.LB_OK
    assert _fwd(T=0, d_in=0) == lb.LB_EINVAL


def test_pack_argument_errors():
    L = lb.lib()
    assert L.lb_pack_signs(FAKE, 10, 10, 2, FAKE + 0x100000, 12, None) == lb.LB_EINVAL
    assert L.lb_pack_signs(FAKE, 10, 10, 0, FAKE + 0x100000, 8, None) == lb.LB_EINVAL   # ld < cols
    assert L.lb_pack_signs(FAKE, 10, 10, 0, FAKE + 0x100000, 14, None) == lb.LB_EALIGN  # ld % 4
    assert L.lb_pack_signs(FAKE, 10, 10, 0, FAKE + 0x100004, 12, None) == lb.LB_EALIGN  # dst align
    assert L.lb_pack_signs(0, 10, 10, 0, FAKE + 0x100000, 12, None) == lb.LB_EINVAL
    assert L.lb_pack_signs(FAKE, 64, 64, 0, FAKE + 8, 64, None) in (lb.LB_EINVAL, lb.LB_EALIGN)


def test_mlp_and_group_argument_errors():
    L = lb.lib()
    f = _factors(ld_v=208, ld_u=3072)
    fd = _factors(ld_v=208, ld_u=1024)
    rc = L.lb_mlp_forward(FAKE + 0x5000000, lb.LB_BF16, FAKE + 0x6000000, lb.LB_BF16,
                          ctypes.byref(f), ctypes.byref(f), ctypes.byref(fd), 1024, 3072, 416,
                          416, 1, 1, None, 0, 0, None)
    assert rc == lb.LB_EWORKSPACE
    assert L.lb_mlp_workspace_bytes(1024, 3072, 416, 416, 16, 1, 0) > 0
    assert L.lb_mlp_workspace_bytes(1024, 3072, 415, 416, 16, 1, 0) == 0   # odd rank, residual
    arr = (lb.lb_linear_desc * 1)()
    arr[0] = lb.lb_linear_desc(FAKE + 0x5000000, FAKE + 0x6000000, _factors(), 1024, 1024, 512, 0, 0)
    assert L.lb_grouped_workspace_bytes(arr, 1, 64, 0) > 0                 # GEMM-path group
    assert L.lb_grouped_workspace_bytes(arr, 1, 0, 0) == 0                 # no tokens
    assert L.lb_grouped_workspace_bytes(arr, 0, 4, 0) == 0                 # no linears
    assert L.lb_grouped_prepare(arr, 1, 1, lb.LB_F32, lb.LB_F32, None, 0, 0, None) == lb.LB_EWORKSPACE
    assert L.lb_grouped_run(FAKE, None) == lb.LB_EINVAL                   # never prepared
    assert L.lb_grouped_release(FAKE) == lb.LB_EINVAL                     # never prepared
