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
    for rc in (lb.LB_OK, lb.LB_EINVAL, lb.LB_EUNSUPPORTED, lb.LB_EALIGN, lb.LB_EWORKSPACE, lb.LB_EHIP,
               lb.LB_EDEVICE):
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


def test_workspace_query_covers_every_path_a_call_can_take():
    """lb_linear_workspace_bytes (flags AUTO) is at least what each path the
    call may end on needs: AUTO sends bf16 outputs of 9-32 tokens to the GEMM
    kernels, but a d_in they do not take (not a multiple of 8) goes to the
    decode kernels, whose workspace is larger here; the query once sized only
    the GEMM form, and the call then refused its own query's workspace."""
    import torch
    L = lb.lib()
    bf, f32 = torch.bfloat16, torch.float32
    for d_in, d_out, r, T, res in [(25, 1662, 692, 19, 1), (1001, 600, 96, 24, 0), (4095, 190, 4, 55, 1),
                                   (1024, 1024, 512, 16, 0), (7, 3000, 40, 32, 1)]:
        auto = L.lb_linear_workspace_bytes(d_in, d_out, r, T, res, 0)
        for flags in (lb.LB_PATH_DECODE, lb.LB_PATH_DECODE_VALU, lb.LB_PATH_PREFILL):
            forced = L.lb_linear_workspace_bytes(d_in, d_out, r, T, res, flags)
            if flags == lb.LB_PATH_PREFILL and d_in % 8:
                continue            # forced GEMM requests of such shapes run the vector-ALU kernels
            if lb.linear_path(d_in, d_out, r, T, bool(res), bf, bf) == flags or \
                    lb.linear_path(d_in, d_out, r, T, bool(res), f32, f32) == flags:
                assert auto >= forced, (d_in, d_out, r, T, res, flags, auto, forced)
        if 9 <= T <= 32:
            # a misaligned x sends even a d_in the GEMM kernels take to the decode kernels
            assert auto >= L.lb_linear_workspace_bytes(d_in, d_out, r, T, res, lb.LB_PATH_DECODE), (d_in, T)


def test_mlp_checks_x_and_y_at_the_block_width():
    """The block's x and y are [T][d_model]: a y placed right after x is not
    an overlap, even when d_ff > d_model (the check once sized x as down's
    input, [T][d_ff], and refused such a y as overlapping)."""
    L = lb.lib()
    T, d_model, d_ff = 115, 641, 2045
    f = _factors(ld_v=68, ld_u=2048)
    fd = _factors(ld_v=12, ld_u=644)
    x = FAKE + 0x5000000
    for y in (x + T * d_model * 4, x + T * d_model * 4 + 4096):
        rc = L.lb_mlp_forward(x, lb.LB_F32, y, lb.LB_F32, ctypes.byref(f), ctypes.byref(f), ctypes.byref(fd),
                              d_model, d_ff, 68, 10, T, 1, None, 0, 0, None)
        assert rc == lb.LB_EWORKSPACE, rc
    rc = L.lb_mlp_forward(x, lb.LB_F32, x + T * d_model * 4 - 4, lb.LB_F32, ctypes.byref(f), ctypes.byref(f),
                          ctypes.byref(fd), d_model, d_ff, 68, 10, T, 1, None, 0, 0, None)
    assert rc == lb.LB_EINVAL                                            # a real overlap


def test_linear_path_choice():
    """Which kernel family a request takes (host only): the decode kernels up
    to 8 tokens, the bf16 GEMM kernels above for bf16 outputs, the decode
    kernels up to 32 tokens for fp32 outputs (or with the decode flag) and the
    vector-ALU kernels above, for shapes the GEMM kernels do not take, and for
    buffers the decode kernels' 32-bit offsets cannot address."""
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    D, G, V = lb.LB_PATH_DECODE, lb.LB_PATH_PREFILL, lb.LB_PATH_DECODE_VALU
    assert lb.linear_path(8192, 28672, 608, 1, True, bf, bf) == D
    assert lb.linear_path(8192, 28672, 608, 8, True, bf, bf) == D
    assert lb.linear_path(8192, 28672, 608, 9, True, bf, bf) == G
    assert lb.linear_path(8192, 28672, 608, 16, True, bf, bf) == G
    assert lb.linear_path(8192, 28672, 608, 32, True, bf, bf) == G
    assert lb.linear_path(8192, 28672, 608, 32, True, bf, bf, lb.LB_PATH_DECODE) == D
    assert lb.linear_path(8192, 28672, 608, 16, True, f32, f32) == D   # fp32 outputs: no GEMM
    assert lb.linear_path(100, 70, 32, 24, True, bf, bf) == D            # d_in % 8 != 0: no GEMM
    assert lb.linear_path(8192, 28672, 608, 33, True, bf, bf) == G
    assert lb.linear_path(8192, 28672, 608, 2048, True, bf, bf) == G
    assert lb.linear_path(1024, 1024, 512, 64, False, f32, f32) == V
    assert lb.linear_path(100, 70, 32, 64, True, bf, bf) == V            # d_in % 8 != 0
    assert lb.linear_path(1024, 1024, 512, 1, False, f32, f32, lb.LB_PATH_DECODE_VALU) == V
    # x of 32 tokens x 2^25 fp32 inputs is 4 GiB: past the decode kernels' offsets
    assert lb.linear_path(1 << 25, 64, 64, 32, False, f32, f32) == V
    assert lb.linear_path(1 << 25, 64, 64, 1, False, f32, f32) == D
    with pytest.raises(lb.LBError) as e:
        lb.linear_path(1024, 1024, 512, 64, False, f32, f32, lb.LB_PATH_PREFILL)
    assert e.value.status == lb.LB_EUNSUPPORTED
    with pytest.raises(lb.LBError):
        lb.linear_path(1024, 1024, 512, 1, False, f32, f32, 1 << 8)     # a group-only flag


def _call(**kw):
    c = lb.lb_linear_call(FAKE + 0x5000000, FAKE + 0x6000000, _factors(), 1024, 1024, 512, 1, 0,
                          lb.LB_BF16, lb.LB_BF16, 0)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_grouped_call_argument_errors():
    L = lb.lib()
    arr = (lb.lb_linear_call * 2)(_call(), _call(x=FAKE + 0x8000000, y=FAKE + 0x9000000, T=64))
    need = L.lb_linear_grouped_workspace_bytes(arr, 2)
    assert need > 0
    # two sub-groups (T = 1 and T = 64) share the workspace: the larger one sizes it
    one = (lb.lb_linear_call * 1)(arr[0])
    two = (lb.lb_linear_call * 1)(arr[1])
    assert need == max(L.lb_linear_grouped_workspace_bytes(one, 1), L.lb_linear_grouped_workspace_bytes(two, 1))
    assert L.lb_linear_forward_grouped(None, 1, FAKE, need, None) == lb.LB_EINVAL
    assert L.lb_linear_forward_grouped(arr, 0, FAKE, need, None) == lb.LB_EINVAL
    assert L.lb_linear_forward_grouped(arr, 2, None, 0, None) == lb.LB_EWORKSPACE
    assert L.lb_linear_forward_grouped(arr, 2, FAKE + 0xa000000, need - 1, None) == lb.LB_EWORKSPACE
    bad = (lb.lb_linear_call * 1)(_call(flags=1 << 9))                  # unknown flag bit
    assert L.lb_linear_forward_grouped(bad, 1, FAKE + 0xa000000, need, None) == lb.LB_EINVAL
    bad = (lb.lb_linear_call * 1)(_call(r=511, residual=1))             # odd total rank
    assert L.lb_linear_forward_grouped(bad, 1, FAKE + 0xa000000, need, None) == lb.LB_EINVAL
    bad = (lb.lb_linear_call * 1)(_call(y=FAKE + 0x5000000))            # y overlaps x
    assert L.lb_linear_forward_grouped(bad, 1, FAKE + 0xa000000, need, None) == lb.LB_EINVAL
    bad = (lb.lb_linear_call * 1)(_call(x_dtype=5))
    assert L.lb_linear_forward_grouped(bad, 1, FAKE + 0xa000000, need, None) == lb.LB_EINVAL
    assert L.lb_linear_grouped_workspace_bytes(None, 1) == 0
    descs = (lb.lb_linear_desc * 1)()
    descs[0] = lb.lb_linear_desc(FAKE + 0x5000000, FAKE + 0x6000000, _factors(), 1024, 1024, 512, 0, 0)
    assert L.lb_grouped_workspace_bytes(descs, 1, 1, 1 << 9) == 0       # unknown flag bit
    assert L.lb_grouped_workspace_bytes(descs, 1, 1, lb.LB_GROUP_FAULT_TEST) > 0
    assert L.lb_grouped_prepare(descs, 1, 1, lb.LB_BF16, lb.LB_BF16, FAKE, 1 << 30, 1 << 9,
                                None) == lb.LB_EINVAL


def test_latent_api_argument_errors():
    L = lb.lib()
    f = _factors()
    X, TT, Y, WS = FAKE + 0x5000000, FAKE + 0x6000000, FAKE + 0x8000000, FAKE + 0xa000000
    need = L.lb_linear_workspace_bytes(1024, 1024, 512, 4, 0, 0)
    s1 = lambda **k: L.lb_linear_stage1(k.get("x", X), k.get("xd", lb.LB_BF16), k.get("t", TT),
                                        k.get("td", lb.LB_F32), k.get("yd", lb.LB_BF16), ctypes.byref(f),
                                        1024, 1024, k.get("r", 512), k.get("T", 4), k.get("res", 0),
                                        k.get("ws", WS), need, k.get("flags", 0), None)
    s2 = lambda **k: L.lb_linear_stage2(k.get("t", TT), k.get("td", lb.LB_F32), k.get("y", Y),
                                        k.get("yd", lb.LB_BF16), ctypes.byref(f), 1024, 1024, k.get("r", 512),
                                        k.get("T", 4), 0, k.get("ws", WS), need, 0, None)
    assert s1(td=7) == lb.LB_EINVAL
    assert s1(yd=7) == lb.LB_EINVAL
    assert s1(t=0) == lb.LB_EINVAL
    assert s1(t=TT + 2) == lb.LB_EALIGN                      # fp32 t misaligned
    assert s1(t=X + 64) == lb.LB_EINVAL                      # t overlaps x
    assert s1(ws=None) == lb.LB_EWORKSPACE
    assert s1(ws=TT) == lb.LB_EINVAL                         # ws overlaps t
    assert s1(flags=1 << 8) == lb.LB_EINVAL                  # a group-only flag
    assert s1(r=511, res=1) == lb.LB_EINVAL
    assert s1(T=0, x=0, t=0) == lb.LB_OK                     # empty: a no-op
    assert s2(y=0) == lb.LB_EINVAL
    assert s2(y=TT) == lb.LB_EINVAL                          # y overlaps t
    assert s2(td=lb.LB_BF16, t=TT + 1) == lb.LB_EALIGN


def test_decoder_layer_argument_errors():
    """lb_decoder_layer_forward's checks, before any launch (fake device
    addresses; a call that got past them would fault, so each one must not)."""
    L = lb.lib()
    f = _factors(ld_v=512, ld_u=2048)
    mk = lambda **k: lb.lb_decoder_layer(f, f, f, f, f, f, f, k.get("d", 1024), k.get("ff", 2048),
                                         k.get("nh", 8), k.get("nkv", 2), 256, 128, 256, 256, 1,
                                         k.get("eps", 1e-6))
    good = mk()
    need = L.lb_decoder_layer_workspace_bytes(ctypes.byref(good), 4)
    assert need > 0
    assert L.lb_decoder_layer_workspace_bytes(ctypes.byref(good), 33) == 0
    assert L.lb_decoder_layer_workspace_bytes(ctypes.byref(good), 0) == 0
    assert L.lb_decoder_layer_workspace_bytes(ctypes.byref(mk(nh=3)), 4) == 0
    X, Y, WS = FAKE + 0x5000000, FAKE + 0x6000000, FAKE + 0xa000000
    run = lambda lay=good, **k: L.lb_decoder_layer_forward(ctypes.byref(lay), k.get("x", X), k.get("y", Y),
                                                           k.get("T", 4), k.get("ws", WS), k.get("n", need), None)
    assert run(T=33) == lb.LB_EUNSUPPORTED
    assert run(T=-1) == lb.LB_EINVAL
    assert run(T=0, x=0, y=0) == lb.LB_OK                    # empty: a no-op
    assert run(mk(nh=3)) == lb.LB_EINVAL                     # heads do not divide d_model
    assert run(mk(nh=8, nkv=3)) == lb.LB_EINVAL              # kv heads do not divide heads
    assert run(mk(eps=float("nan"))) == lb.LB_EINVAL
    assert run(x=0) == lb.LB_EINVAL
    assert run(x=X + 2) == lb.LB_EALIGN
    assert run(y=X + 256) == lb.LB_EINVAL                    # y overlaps x
    assert run(ws=None) == lb.LB_EWORKSPACE
    assert run(n=need - 1) == lb.LB_EWORKSPACE
    assert run(ws=WS + 16) == lb.LB_EALIGN
    assert run(ws=X - 256) == lb.LB_EINVAL                   # ws overlaps x


def test_joint_itq_argument_errors():
    """lb_joint_itq and lb_dual_svid_itq reject bad arguments before any
    launch or copy (fake device addresses)."""
    L = lb.lib()
    U, V, R0, OBJ, WS = FAKE + 0x100000, FAKE + 0x900000, FAKE + 0x1100000, FAKE + 0x1200000, FAKE + 0x2000000
    need = L.lb_joint_itq_workspace_bytes(96, 64, 16)
    assert need >= (96 + 64) * 16 * 4 * 2
    assert L.lb_joint_itq_workspace_bytes(0, 64, 16) == 0
    assert L.lb_joint_itq_workspace_bytes(96, 64, 0) == 0
    run = lambda **k: L.lb_joint_itq(k.get("u", U), k.get("v", V), k.get("d_out", 96), k.get("d_in", 64),
                                     k.get("r_p", 16), k.get("iters", 4), k.get("rot0", None), k.get("rot", None),
                                     k.get("obj", None), k.get("ws", WS), k.get("n", need), None)
    assert run(u=None) == lb.LB_EINVAL
    assert run(v=None) == lb.LB_EINVAL
    assert run(iters=-1) == lb.LB_EINVAL
    assert run(r_p=65) == lb.LB_EINVAL                      # more latents than min(d_out, d_in)
    assert run(r_p=0) == lb.LB_EINVAL
    assert run(u=U + 2) == lb.LB_EALIGN
    assert run(rot0=R0 + 1) == lb.LB_EALIGN
    assert run(obj=OBJ + 4) == lb.LB_EALIGN                 # fp64 objective
    assert run(ws=None) == lb.LB_EWORKSPACE
    assert run(n=need - 1) == lb.LB_EWORKSPACE
    assert run(ws=WS + 64) == lb.LB_EALIGN
    assert run(d_out=1 << 20, d_in=1 << 20, r_p=1024, n=1 << 40) == lb.LB_EUNSUPPORTED
    f = _factors(ld_v=16, ld_u=96)
    Wp = FAKE + 0x3000000
    nsv = L.lb_dual_svid_itq_workspace_bytes(96, 64, 32, 1)
    assert nsv > L.lb_dual_svid_workspace_bytes(96, 64, 32, 1)
    assert L.lb_dual_svid_itq_workspace_bytes(96, 64, 33, 1) == 0      # odd rank with the residual
    sv = lambda **k: L.lb_dual_svid_itq(k.get("w", Wp), 96, 64, k.get("r", 32), 1, k.get("iters", 5),
                                        ctypes.byref(f), None, None, k.get("ws", WS), k.get("n", nsv), None)
    assert sv(iters=-1) == lb.LB_EINVAL
    assert sv(w=None) == lb.LB_EINVAL
    assert sv(r=33) == lb.LB_EINVAL
    assert sv(n=nsv - 1) == lb.LB_EWORKSPACE
    assert sv(ws=WS + 8) == lb.LB_EALIGN
