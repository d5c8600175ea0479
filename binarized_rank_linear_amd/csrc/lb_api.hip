// lb_api.hip -- the C entry points of littlebit.h: argument checks, path
// dispatch, workspace sizing, the SwiGLU block and layer groups.
#include <algorithm>
#include <atomic>
#include <deque>
#include <memory>
#include <mutex>
#include <random>
#include <string.h>
#include <unordered_map>
#include <vector>

#include "lb_internal.h"

using namespace lb;

namespace {

constexpr int64_t kDecodeMaxT = 32;     // token count served by the decode kernels
// With bf16 outputs AUTO takes the GEMM kernels from this many tokens on:
// above 8 tokens the decode kernels' stage 1 no longer runs fused (its
// activation operands take a launch of their own) and their matrix work grows
// with the activation rows, while the bf16 GEMMs on 32-token tiles cost about
// the same from 8 to 32 tokens (a 32-layer Llama2-7B-shaped stack: 0.34 against
// 0.47 ms per pass at T = 8, 0.73 against 0.49 ms at T = 12, 2.09 against 0.55
// ms at T = 32).
constexpr int64_t kGemmFromT = 9;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t act_size(int dtype) { return dtype == LB_F32 ? 4 : 2; }

bool valid_dtype(int d) { return d == LB_F32 || d == LB_BF16; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

enum class Path { Valu, MfmaDecode, Gemm };

// Flag bits a call may carry: the path, and for groups the fault-report test.
constexpr unsigned kLinearFlags = LB_PATH_MASK;
constexpr unsigned kGroupFlags = LB_PATH_MASK | LB_GROUP_FAULT_TEST;

// The path a request runs on (a: its sizes, and its strides when known).
// Returns LB_EINVAL for an invalid path flag, LB_EUNSUPPORTED for a path the
// request cannot take.
int choose_path(unsigned flags, int64_t T, int y_dtype, Path *out, const Linear *a = nullptr) {
    const bool mfma_ok = mfma_decode_supported(T, y_dtype) && (!a || mfma_decode_shape_ok(*a));
    switch (flags & LB_PATH_MASK) {
        case LB_PATH_AUTO:
            if (T <= kDecodeMaxT &&
                (T < kGemmFromT || y_dtype != LB_BF16 || (a && !gemm_linear_supported(*a))))
                *out = mfma_ok ? Path::MfmaDecode : Path::Valu;
            else
                *out = y_dtype == LB_BF16 ? Path::Gemm : Path::Valu;
            return LB_OK;
        case LB_PATH_DECODE:
            *out = mfma_ok ? Path::MfmaDecode : Path::Valu;
            return LB_OK;
        case LB_PATH_PREFILL:
            if (y_dtype != LB_BF16) return LB_EUNSUPPORTED;
            *out = Path::Gemm;
            return LB_OK;
        case LB_PATH_DECODE_VALU:
            *out = Path::Valu;
            return LB_OK;
        default:
            return LB_EINVAL;
    }
}

size_t path_workspace(Path p, const Linear &a) {
    switch (p) {
        case Path::Valu: return valu_workspace_bytes(a);
        case Path::MfmaDecode: return mfma_decode_workspace_bytes(a);
        case Path::Gemm: return gemm_workspace_bytes(a);
    }
    return 0;
}

int run_path(Path p, const Linear &a, void *ws, hipStream_t s) {
    switch (p) {
        case Path::Valu: return valu_forward(a, ws, s);
        case Path::MfmaDecode: return mfma_decode_forward(a, ws, s);
        case Path::Gemm: return gemm_forward(a, ws, s);
    }
    return LB_EINVAL;
}

size_t rup256(size_t n) { return (n + 255) & ~(size_t)255; }

// Shape checks shared by the linear entry points; fills the size fields of *a.
int check_shape(int64_t d_in, int64_t d_out, int64_t r, int64_t T, int residual, Linear *a) {
    if (d_in <= 0 || d_out <= 0 || r <= 0 || T < 0) return LB_EINVAL;
    if (d_in > (1ll << 31) || d_out > (1ll << 31) || r > (1ll << 24) || T > (1ll << 31))
        return LB_EINVAL;
    const int P = residual ? 2 : 1;
    if (r % P) return LB_EINVAL;
    a->d_in = d_in;
    a->d_out = d_out;
    a->r_p = r / P;
    a->P = P;
    a->T = T;
    return LB_OK;
}

int check_factors(const lb_factors *w, Linear *a) {
    if (!w || !w->v_bits || !w->u_bits || !w->g || !w->l || !w->h) return LB_EINVAL;
    if (w->ld_v < a->r_p || w->ld_u < a->d_out) return LB_EINVAL;
    if (w->ld_v % 4 || w->ld_u % 4) return LB_EALIGN;
    if (!aligned(w->v_bits, 16) || !aligned(w->u_bits, 16)) return LB_EALIGN;
    if (!aligned(w->g, 2) || !aligned(w->l, 2) || !aligned(w->h, 2)) return LB_EALIGN;
    a->v_bits = w->v_bits;
    a->u_bits = w->u_bits;
    a->g = w->g;
    a->l = w->l;
    a->h = w->h;
    a->ld_v = w->ld_v;
    a->ld_u = w->ld_u;
    return LB_OK;
}

int check_io(const void *x, int x_dtype, void *y, int y_dtype, Linear *a) {
    if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype)) return LB_EINVAL;
    if ((!x || !y) && a->T > 0) return LB_EINVAL;   // empty tensors may carry null pointers
    if (!aligned(x, act_size(x_dtype)) || !aligned(y, act_size(y_dtype))) return LB_EALIGN;
    if (overlap(x, (size_t)(a->T * a->d_in) * act_size(x_dtype), y,
                (size_t)(a->T * a->d_out) * act_size(y_dtype)))
        return LB_EINVAL;
    a->x = x;
    a->y = y;
    a->x_dtype = x_dtype;
    a->y_dtype = y_dtype;
    return LB_OK;
}

}  // namespace

namespace lb {
static thread_local const char *t_last_hip_error = "no HIP error recorded";
void note_hip_error(hipError_t e) { t_last_hip_error = hipGetErrorString(e); }
}  // namespace lb

extern "C" {

const char *lb_last_hip_error(void) { return lb::t_last_hip_error; }

int lb_version(void) { return (1 << 16) | 0; }

const char *lb_status_string(int status) {
    switch (status) {
        case LB_OK: return "ok";
        case LB_EINVAL: return "invalid argument";
        case LB_EUNSUPPORTED: return "unsupported request";
        case LB_EALIGN: return "misaligned pointer or stride";
        case LB_EWORKSPACE: return "workspace missing or too small";
        case LB_EHIP: return "HIP runtime error";
        case LB_EDEVICE: return "a kernel reported a fault (lb_device_faults)";
        default: return "unknown status";
    }
}

int lb_rank_for_budget(int64_t d_in, int64_t d_out, int64_t b_num, int64_t b_den, int residual,
                       int64_t *r_total, int64_t *r_path) {
    if (!r_total || !r_path) return LB_EINVAL;
    if (d_in <= 0 || d_out <= 0 || b_num <= 0 || b_den <= 0) return LB_EINVAL;
    // floor(b_num*d_in*d_out / (b_den*(d_in+d_out))) in 128-bit integers
    const __int128 num = (__int128)b_num * d_in * d_out;
    const __int128 den = (__int128)b_den * (d_in + d_out);
    const __int128 q = num / den;
    if (q > ((__int128)1 << 40)) return LB_EINVAL;
    const int64_t r = ((int64_t)q / 32) * 32;
    if (r <= 0) return LB_EINVAL;
    *r_total = r;
    *r_path = residual ? r / 2 : r;
    return LB_OK;
}

int64_t lb_packed_ld(int64_t n_other) { return n_other <= 0 ? 0 : rup(n_other, 4); }

int64_t lb_packed_ld_aligned(int64_t n_other) { return n_other <= 0 ? 0 : rup(n_other, 32); }

int64_t lb_packed_words(int64_t rows, int64_t cols, int axis, int64_t ld) {
    if (rows <= 0 || cols <= 0 || (axis != 0 && axis != 1)) return 0;
    const int64_t n_pack = axis == 0 ? rows : cols;
    const int64_t n_other = axis == 0 ? cols : rows;
    if (ld < n_other) return 0;
    return cdiv(n_pack, 32) * ld;
}

int lb_pack_signs(const float *src, int64_t rows, int64_t cols, int axis, uint32_t *dst,
                  int64_t ld, void *stream) {
    if (!src || !dst || rows <= 0 || cols <= 0 || (axis != 0 && axis != 1)) return LB_EINVAL;
    const int64_t n_pack = axis == 0 ? rows : cols;
    const int64_t n_other = axis == 0 ? cols : rows;
    if (ld < n_other) return LB_EINVAL;
    if (ld % 4 || !aligned(dst, 16) || !aligned(src, 4)) return LB_EALIGN;
    if (cdiv(n_pack, 32) >= 65536 && axis == 0) return LB_EUNSUPPORTED;
    if (cdiv(n_pack, 64) >= 65536 && axis == 1) return LB_EUNSUPPORTED;
    if (overlap(src, (size_t)(rows * cols) * 4, dst, (size_t)(cdiv(n_pack, 32) * ld) * 4))
        return LB_EINVAL;
    return launch_pack(src, rows, cols, axis, dst, ld, (hipStream_t)stream);
}

size_t lb_linear_workspace_bytes(int64_t d_in, int64_t d_out, int64_t r, int64_t T,
                                 int residual, unsigned flags) {
    Linear a{};
    if (check_shape(d_in, d_out, r, T, residual, &a)) return 0;
    if (flags & ~kLinearFlags) return 0;
    a.ld_v = lb_packed_ld_aligned(a.r_p);
    a.ld_u = lb_packed_ld_aligned(d_out);
    size_t need = 0;
    // Every path a call of this shape can take, for either activation and
    // output dtype: AUTO picks by the output dtype, and by the shape and the
    // pointers when the GEMM kernels do not take them (so both the choice
    // without the linear and the one with its shape count), and the
    // vector-ALU kernels serve strides the decode kernels do not address.
    for (int xd : {LB_BF16, LB_F32})
        for (int yd : {LB_BF16, LB_F32}) {
            a.x_dtype = xd;
            a.y_dtype = yd;
            for (int with_shape = 0; with_shape < 2; ++with_shape) {
                Path p;
                if (choose_path(flags, T, yd, &p, with_shape ? &a : nullptr)) continue;
                size_t b = path_workspace(p, a);
                if (p == Path::MfmaDecode) b = std::max(b, path_workspace(Path::Valu, a));
                // a misaligned x or g at run time sends AUTO's GEMM requests of
                // up to kDecodeMaxT tokens to the decode kernels
                if (p == Path::Gemm && (flags & LB_PATH_MASK) == LB_PATH_AUTO && T <= kDecodeMaxT) {
                    if (mfma_decode_supported(T, yd) && mfma_decode_shape_ok(a))
                        b = std::max(b, path_workspace(Path::MfmaDecode, a));
                    b = std::max(b, path_workspace(Path::Valu, a));
                }
                if (b > need) need = b;
            }
        }
    return rup256(need);
}

int lb_linear_forward(const void *x, int x_dtype, void *y, int y_dtype, const lb_factors *w,
                      int64_t d_in, int64_t d_out, int64_t r, int64_t T, int residual, void *ws,
                      size_t ws_bytes, unsigned flags, void *stream) {
    Linear a{};
    int rc;
    if ((rc = check_shape(d_in, d_out, r, T, residual, &a))) return rc;
    if ((rc = check_factors(w, &a))) return rc;
    if ((rc = check_io(x, x_dtype, y, y_dtype, &a))) return rc;
    if (flags & ~kLinearFlags) return LB_EINVAL;
    Path p;
    if ((rc = choose_path(flags, T, y_dtype, &p, &a))) return rc;
    if (T == 0) return LB_OK;
    const size_t need = path_workspace(p, a);
    if (need > 0) {
        if (!ws || ws_bytes < need) return LB_EWORKSPACE;
        if (!aligned(ws, 256)) return LB_EALIGN;
        if (overlap(ws, need, x, (size_t)(T * d_in) * act_size(x_dtype)) ||
            overlap(ws, need, y, (size_t)(T * d_out) * act_size(y_dtype)))
            return LB_EINVAL;
    }
    return run_path(p, a, ws, (hipStream_t)stream);
}

// ---- the latent API ----------------------------------------------------------

namespace {
int run_stage(Path p, const Linear &a, void *ws, int stage, void *t, int t_dtype, hipStream_t s) {
    switch (p) {
        case Path::Valu: return valu_stage_forward(a, ws, stage, t, t_dtype, s);
        case Path::MfmaDecode: return mfma_decode_stage(a, ws, stage, t, t_dtype, s);
        case Path::Gemm: return gemm_stage_forward(a, ws, stage, t, t_dtype, s);
    }
    return LB_EINVAL;
}

// Checks shared by both halves: sizes, factors, the latents buffer, the
// workspace and the path.  act/act_bytes: the activation (x or y) the half
// reads or writes besides t.
int stage_common(const lb_factors *w, int64_t d_in, int64_t d_out, int64_t r, int64_t T, int residual,
                 const void *t, int t_dtype, const void *act, size_t act_bytes, int y_dtype, void *ws,
                 size_t ws_bytes, unsigned flags, Linear *a, Path *p) {
    int rc;
    if ((rc = check_shape(d_in, d_out, r, T, residual, a))) return rc;
    if ((rc = check_factors(w, a))) return rc;
    if (!valid_dtype(t_dtype) || !valid_dtype(y_dtype) || (flags & ~kLinearFlags)) return LB_EINVAL;
    if (T > 0 && (!t || !act)) return LB_EINVAL;
    if (!aligned(t, act_size(t_dtype))) return LB_EALIGN;
    const size_t t_bytes = (size_t)(T * r) * act_size(t_dtype);
    if (overlap(t, t_bytes, act, act_bytes)) return LB_EINVAL;
    a->y_dtype = y_dtype;
    if ((rc = choose_path(flags, T, y_dtype, p, a))) return rc;
    if (T == 0) return LB_OK;
    const size_t need = path_workspace(*p, *a);
    if (need > 0) {
        if (!ws || ws_bytes < need) return LB_EWORKSPACE;
        if (!aligned(ws, 256)) return LB_EALIGN;
        if (overlap(ws, need, t, t_bytes) || overlap(ws, need, act, act_bytes)) return LB_EINVAL;
    }
    return LB_OK;
}
}  // namespace

int lb_linear_stage1(const void *x, int x_dtype, void *t, int t_dtype, int y_dtype, const lb_factors *w,
                     int64_t d_in, int64_t d_out, int64_t r, int64_t T, int residual, void *ws, size_t ws_bytes,
                     unsigned flags, void *stream) {
    Linear a{};
    Path p;
    if (!valid_dtype(x_dtype)) return LB_EINVAL;
    if (!aligned(x, act_size(x_dtype))) return LB_EALIGN;
    const size_t x_bytes = (size_t)(T > 0 ? T * d_in : 0) * act_size(x_dtype);
    if (int rc = stage_common(w, d_in, d_out, r, T, residual, t, t_dtype, x, x_bytes, y_dtype, ws, ws_bytes,
                              flags, &a, &p))
        return rc;
    if (T == 0) return LB_OK;
    a.x = x;
    a.x_dtype = x_dtype;
    return run_stage(p, a, ws, 1, t, t_dtype, (hipStream_t)stream);
}

int lb_linear_stage2(const void *t, int t_dtype, void *y, int y_dtype, const lb_factors *w, int64_t d_in,
                     int64_t d_out, int64_t r, int64_t T, int residual, void *ws, size_t ws_bytes, unsigned flags,
                     void *stream) {
    Linear a{};
    Path p;
    if (!valid_dtype(y_dtype)) return LB_EINVAL;
    if (!aligned(y, act_size(y_dtype))) return LB_EALIGN;
    const size_t y_bytes = (size_t)(T > 0 ? T * d_out : 0) * act_size(y_dtype);
    if (int rc = stage_common(w, d_in, d_out, r, T, residual, t, t_dtype, y, y_bytes, y_dtype, ws, ws_bytes,
                              flags, &a, &p))
        return rc;
    if (T == 0) return LB_OK;
    a.y = y;
    a.x_dtype = LB_BF16;
    return run_stage(p, a, ws, 2, const_cast<void *>(t), t_dtype, (hipStream_t)stream);
}

// ---- SwiGLU block ----------------------------------------------------------

static size_t mlp_linear_ws(int64_t d_model, int64_t d_ff, int64_t r_gu, int64_t r_down, int64_t T,
                            int residual, unsigned flags) {
    const size_t a = lb_linear_workspace_bytes(d_model, d_ff, r_gu, T, residual, flags);
    const size_t b = lb_linear_workspace_bytes(d_ff, d_model, r_down, T, residual, flags);
    return a > b ? a : b;
}

// The fused decode form of the block (bf16 output, decode kernels): gate and
// up as one three-launch group writing bf16, then down reading silu(gate) (.)
// up as its input (computed while its stage 1 stages the activations).
// Workspace: gate and up outputs, then the larger of the two runs' scratch.
static size_t mlp_fused_ws(const Linear &ag, const Linear &au, const Linear &ad) {
    const size_t inter = rup256((size_t)(ag.T * ag.d_out) * 2);
    const Linear gu[2] = {ag, au};
    const size_t a = mfma_inline_workspace_bytes(gu, 2), b = mfma_decode_workspace_bytes(ad);
    return 2 * inter + rup256(a > b ? a : b);
}

size_t lb_mlp_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t r_gu, int64_t r_down,
                              int64_t T, int residual, unsigned flags) {
    Linear ag{}, ad{};
    if (check_shape(d_model, d_ff, r_gu, T, residual, &ag)) return 0;
    if (check_shape(d_ff, d_model, r_down, T, residual, &ad)) return 0;
    if (flags & ~kLinearFlags) return 0;
    const size_t inter = rup256((size_t)(T * d_ff) * sizeof(float));
    size_t need = 2 * inter + mlp_linear_ws(d_model, d_ff, r_gu, r_down, T, residual, flags);
    Path p;
    if (T > 0 && !choose_path(flags, T, LB_BF16, &p) && p == Path::MfmaDecode) {
        ag.y_dtype = ag.x_dtype = ad.y_dtype = ad.x_dtype = LB_BF16;
        need = std::max(need, mlp_fused_ws(ag, ag, ad));
    }
    return need;
}

int lb_mlp_forward(const void *x, int x_dtype, void *y, int y_dtype, const lb_factors *gate,
                   const lb_factors *up, const lb_factors *down, int64_t d_model, int64_t d_ff,
                   int64_t r_gu, int64_t r_down, int64_t T, int residual, void *ws,
                   size_t ws_bytes, unsigned flags, void *stream) {
    Linear ag{}, au{}, ad{};
    int rc;
    if ((rc = check_shape(d_model, d_ff, r_gu, T, residual, &ag))) return rc;
    if ((rc = check_shape(d_model, d_ff, r_gu, T, residual, &au))) return rc;
    if ((rc = check_shape(d_ff, d_model, r_down, T, residual, &ad))) return rc;
    if ((rc = check_factors(gate, &ag)) || (rc = check_factors(up, &au)) ||
        (rc = check_factors(down, &ad)))
        return rc;
    // x and y are the block's [T][d_model] (down's own input is the SwiGLU,
    // in the workspace)
    Linear io{};
    io.T = T;
    io.d_in = io.d_out = d_model;
    if ((rc = check_io(x, x_dtype, y, y_dtype, &io))) return rc;
    ad.y = y;
    ad.y_dtype = y_dtype;
    Path p;
    if (flags & ~kLinearFlags) return LB_EINVAL;
    if ((rc = choose_path(flags, T, y_dtype, &p, &ad))) return rc;
    if (T == 0) return LB_OK;
    const size_t need = lb_mlp_workspace_bytes(d_model, d_ff, r_gu, r_down, T, residual, flags);
    if (!ws || ws_bytes < need) return LB_EWORKSPACE;
    if (!aligned(ws, 256)) return LB_EALIGN;
    if (overlap(ws, need, x, (size_t)(T * d_model) * act_size(x_dtype)) ||
        overlap(ws, need, y, (size_t)(T * d_model) * act_size(y_dtype)))
        return LB_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    if (p == Path::MfmaDecode && y_dtype == LB_BF16 && mfma_decode_shape_ok(ag) && mfma_decode_shape_ok(au)) {
        // the fused form: gate and up (bf16) as one group, down reads the SwiGLU
        const size_t inter = rup256((size_t)(T * d_ff) * 2);
        uint16_t *yg = (uint16_t *)ws, *yu = (uint16_t *)((char *)ws + inter);
        void *lws = (char *)ws + 2 * inter;
        ag.x = au.x = x;
        ag.x_dtype = au.x_dtype = x_dtype;
        ag.y = yg;
        au.y = yu;
        ag.y_dtype = au.y_dtype = LB_BF16;
        ad.x = yg;
        ad.x2 = yu;
        ad.x_dtype = LB_BF16;
        const Linear gu[2] = {ag, au};
        if ((rc = mfma_inline_forward(gu, 2, lws, s))) return rc;
        return mfma_decode_forward(ad, lws, s);
    }
    const size_t inter = rup256((size_t)(T * d_ff) * sizeof(float));
    float *zg = (float *)ws;
    float *zu = (float *)((char *)ws + inter);
    void *lws = (char *)ws + 2 * inter;
    // gate and up read the same x; the intermediate stays fp32.
    ag.x = au.x = x;
    ag.x_dtype = au.x_dtype = x_dtype;
    ag.y = zg;
    au.y = zu;
    ag.y_dtype = au.y_dtype = LB_F32;
    Path pi;
    if ((rc = choose_path(flags, T, LB_F32, &pi, &ag))) pi = Path::Valu;
    if (p == Path::Gemm) pi = Path::Gemm;
    if ((rc = run_path(pi, ag, lws, s))) return rc;
    if ((rc = run_path(pi, au, lws, s))) return rc;
    if ((rc = launch_swiglu_f32(zg, zu, T * d_ff, s))) return rc;
    ad.x = zg;
    ad.x_dtype = LB_F32;
    return run_path(p, ad, lws, s);
}

}  // extern "C"

// ---- layer groups ----------------------------------------------------------

namespace {
enum class GroupKind { Loop, Decode, Gemm };

// Everything a run of a group needs: the linears (for the linear-by-linear
// form), the launch state of the whole-group kernels, and the image its
// workspace must hold (header with the stamp, tables, zeroed counters).
struct GroupPlan {
    std::vector<lb_linear_desc> descs;
    int64_t T = 0;
    int x_dtype = 0, y_dtype = 0;
    unsigned flags = 0;
    void *ws = nullptr;
    size_t ws_bytes = 0;
    GroupKind kind = GroupKind::Loop;
    std::vector<uint8_t> state;
    GroupImage img;
};

// A tag no other group set-up in this process has (and, with its random
// half, unlikely to be any earlier contents of the memory it stamps).
uint64_t new_tag() {
    static std::atomic<uint64_t> counter{1};
    static const uint64_t salt = [] {
        std::random_device rd;
        return ((uint64_t)rd() << 32) ^ (uint64_t)rd();
    }();
    return salt ^ (counter.fetch_add(1) * 0x9e3779b97f4a7c15ull);
}

int group_linear(const lb_linear_desc &d, int64_t T, int x_dtype, int y_dtype, Linear *a) {
    int rc;
    if ((rc = check_shape(d.d_in, d.d_out, d.r, T, d.residual, a))) return rc;
    if ((rc = check_factors(&d.w, a))) return rc;
    if ((rc = check_io(d.x, x_dtype, d.y, y_dtype, a))) return rc;
    return LB_OK;
}

// Shapes only (pointers unset): enough for sizing and path choice.
bool group_shapes(const lb_linear_desc *descs, int n, int64_t T, std::vector<Linear> *ls) {
    ls->assign((size_t)n, Linear{});
    for (int i = 0; i < n; ++i) {
        Linear &a = (*ls)[(size_t)i];
        if (check_shape(descs[i].d_in, descs[i].d_out, descs[i].r, T, descs[i].residual, &a)) return false;
        a.x_dtype = a.y_dtype = LB_BF16;
        a.ld_v = descs[i].w.ld_v;
        a.ld_u = descs[i].w.ld_u;
    }
    return true;
}

GroupKind group_kind(unsigned flags, int64_t T, int y_dtype, const std::vector<Linear> &ls) {
    Path p;
    if (choose_path(flags, T, y_dtype, &p)) return GroupKind::Loop;
    if (p == Path::MfmaDecode) {
        for (const Linear &a : ls)
            if (!mfma_decode_shape_ok(a)) return GroupKind::Loop;
        return GroupKind::Decode;
    }
    if (p == Path::Gemm && gemm_group_supported(ls.data(), (int)ls.size())) return GroupKind::Gemm;
    return GroupKind::Loop;
}

size_t group_ws_bytes(const lb_linear_desc *descs, int n, int64_t T, unsigned flags) {
    if (!descs || n <= 0 || T <= 0 || (flags & ~kGroupFlags)) return 0;
    std::vector<Linear> ls;
    if (!group_shapes(descs, n, T, &ls)) return 0;
    size_t need = 0;
    // whole-group kernels' tables and per-linear scratch, for either output dtype
    for (int yd : {LB_BF16, LB_F32}) {
        const GroupKind k = group_kind(flags, T, yd, ls);
        size_t b = 0;
        if (k == GroupKind::Decode) b = mfma_group_workspace_bytes(ls.data(), n, T, yd);
        if (k == GroupKind::Gemm) b = gemm_group_workspace_bytes(ls.data(), n);
        if (b > need) need = b;
    }
    // the linear-by-linear loop (after a 256-byte header)
    for (int i = 0; i < n; ++i) {
        const size_t b = lb_linear_workspace_bytes(descs[i].d_in, descs[i].d_out, descs[i].r, T,
                                                   descs[i].residual, flags & kLinearFlags);
        if (b + 256 > need) need = b + 256;
    }
    return rup256(need);
}

// Checks a group and plans it on ws (nothing is enqueued).
int build_plan(const lb_linear_desc *descs, int n, int64_t T, int x_dtype, int y_dtype, void *ws,
               size_t ws_bytes, unsigned flags, GroupPlan *gp) {
    if (!descs || n <= 0 || T <= 0) return LB_EINVAL;
    if (flags & ~kGroupFlags) return LB_EINVAL;
    Path p;
    int rc;
    if ((rc = choose_path(flags, T, y_dtype, &p))) return rc;
    std::vector<Linear> ls((size_t)n);
    for (int i = 0; i < n; ++i)
        if ((rc = group_linear(descs[i], T, x_dtype, y_dtype, &ls[(size_t)i]))) return rc;
    const size_t need = group_ws_bytes(descs, n, T, flags);
    if (!ws || ws_bytes < need) return LB_EWORKSPACE;
    if (!aligned(ws, 256)) return LB_EALIGN;
    for (int i = 0; i < n; ++i) {
        const Linear &a = ls[(size_t)i];
        if (overlap(ws, need, a.x, (size_t)(T * a.d_in) * act_size(x_dtype)) ||
            overlap(ws, need, a.y, (size_t)(T * a.d_out) * act_size(y_dtype)))
            return LB_EINVAL;
    }
    gp->descs.assign(descs, descs + n);
    gp->T = T;
    gp->x_dtype = x_dtype;
    gp->y_dtype = y_dtype;
    gp->flags = flags;
    gp->ws = ws;
    gp->ws_bytes = ws_bytes;
    gp->kind = group_kind(flags, T, y_dtype, ls);
    const uint64_t tag = new_tag();
    if (gp->kind == GroupKind::Decode) {
        gp->state.assign(mfma_group_state_bytes(), 0);
        return mfma_group_plan(ls.data(), n, T, y_dtype, ws, ws_bytes, tag, (flags & LB_GROUP_FAULT_TEST) != 0,
                               gp->state.data(), &gp->img);
    }
    if (gp->kind == GroupKind::Gemm) {
        gp->state.assign(gemm_group_state_bytes(), 0);
        return gemm_group_plan(ls.data(), n, ws, ws_bytes, tag, gp->state.data(), &gp->img);
    }
    return LB_OK;
}

// Enqueues the set-up of a planned group on s: its workspace image from
// `src` (host memory that stays valid until the copy is done), the zeroed
// scratch and, for the GEMM kernels, the factor preparation.
int enqueue_setup(const GroupPlan &gp, const void *src, hipStream_t s) {
    if (gp.kind == GroupKind::Loop) return LB_OK;
    if (hipMemcpyAsync(gp.ws, src, gp.img.bytes.size(), hipMemcpyHostToDevice, s) != hipSuccess)
        return hip_status(hipGetLastError());
    if (int rc = fill_words((char *)gp.ws + gp.img.zero_off, gp.img.zero_bytes, 0u, s)) return rc;
    if (gp.kind == GroupKind::Gemm) return gemm_group_run(gp.state.data(), s, 4);
    return LB_OK;
}

int run_plan(const GroupPlan &gp, int stage_mask, hipStream_t s) {
    if (gp.kind == GroupKind::Decode) return mfma_group_run(gp.state.data(), s, stage_mask);
    if (gp.kind == GroupKind::Gemm) return gemm_group_run(gp.state.data(), s, stage_mask);
    if (stage_mask != 3) return LB_EUNSUPPORTED;
    void *lws = (char *)gp.ws + 256;
    for (const lb_linear_desc &d : gp.descs) {
        const int rc = lb_linear_forward(d.x, gp.x_dtype, d.y, gp.y_dtype, &d.w, d.d_in, d.d_out, d.r, gp.T,
                                         d.residual, lws, gp.ws_bytes - 256, gp.flags & kLinearFlags, s);
        if (rc) return rc;
    }
    return LB_OK;
}

// Prepared groups, by workspace address.  A record is looked up under the
// lock and used outside it; runs read it only.
std::mutex g_groups_mu;
std::unordered_map<void *, std::shared_ptr<const GroupPlan>> g_groups;

std::shared_ptr<const GroupPlan> find_group(void *ws) {
    std::lock_guard<std::mutex> lk(g_groups_mu);
    auto it = g_groups.find(ws);
    return it == g_groups.end() ? nullptr : it->second;
}

// ---- the stateless grouped call: plans cached by their arguments ----------

uint64_t fnv1a(const void *p, size_t n, uint64_t h = 1469598103934665603ull) {
    const uint8_t *b = (const uint8_t *)p;
    for (size_t i = 0; i < n; ++i) h = (h ^ b[i]) * 1099511628211ull;
    return h;
}

// One cached plan: its key (the call's bytes), the plan, a pinned copy of its
// workspace image and an event after the last copy out of it.
struct CachedPlan {
    std::vector<uint8_t> key;
    uint64_t hash = 0;
    std::shared_ptr<GroupPlan> plan;
    void *pinned = nullptr;
    hipEvent_t copied = nullptr;
    uint64_t used = 0;
    bool captured = false;    // a captured graph copies from `pinned`: kept until the process ends
};

constexpr size_t kPlanCache = 8;
std::mutex g_cache_mu;
std::deque<CachedPlan> g_cache;      // deque: slots keep their address as it grows
uint64_t g_cache_clock = 0;

void drop_cached(CachedPlan &c) {
    if (c.copied) {
        (void)hipEventSynchronize(c.copied);
        (void)hipEventDestroy(c.copied);
    }
    if (c.pinned) (void)hipHostFree(c.pinned);
    c = CachedPlan{};
}

// Plans a sub-group (or finds its plan) and enqueues its set-up and run.
int run_stateless(const lb_linear_desc *descs, int n, int64_t T, int x_dtype, int y_dtype, void *ws,
                  size_t ws_bytes, unsigned flags, hipStream_t s) {
    std::vector<uint8_t> key(sizeof(lb_linear_desc) * n + 64);
    memcpy(key.data(), descs, sizeof(lb_linear_desc) * n);
    uint8_t *tail = key.data() + sizeof(lb_linear_desc) * n;
    memcpy(tail, &T, 8);
    memcpy(tail + 8, &x_dtype, 4);
    memcpy(tail + 12, &y_dtype, 4);
    memcpy(tail + 16, &flags, 4);
    memcpy(tail + 24, &ws, sizeof(void *));
    memcpy(tail + 32, &ws_bytes, sizeof(size_t));
    int dev = 0;
    (void)hipGetDevice(&dev);
    memcpy(tail + 40, &dev, 4);
    const uint64_t h = fnv1a(key.data(), key.size());
    std::lock_guard<std::mutex> lk(g_cache_mu);
    CachedPlan *hit = nullptr;
    for (CachedPlan &c : g_cache)
        if (c.plan && c.hash == h && c.key == key) hit = &c;
    if (!hit) {
        auto gp = std::make_shared<GroupPlan>();
        if (int rc = build_plan(descs, n, T, x_dtype, y_dtype, ws, ws_bytes, flags, gp.get())) return rc;
        // a free slot, else the least recently used one no graph copies from
        CachedPlan *slot = nullptr;
        size_t live = 0;
        for (CachedPlan &c : g_cache) live += c.captured ? 0 : 1;
        if (live < kPlanCache) {
            for (CachedPlan &c : g_cache)
                if (!c.plan) { slot = &c; break; }
            if (!slot) slot = &g_cache.emplace_back();
        } else {
            for (CachedPlan &c : g_cache)
                if (!c.captured && (!slot || c.used < slot->used)) slot = &c;
        }
        drop_cached(*slot);
        slot->key = std::move(key);
        slot->hash = h;
        slot->plan = gp;
        if (!gp->img.bytes.empty()) {
            if (hipHostMalloc(&slot->pinned, gp->img.bytes.size(), hipHostMallocDefault) != hipSuccess ||
                hipEventCreateWithFlags(&slot->copied, hipEventDisableTiming) != hipSuccess) {
                const int rc = hip_status(hipGetLastError());
                drop_cached(*slot);
                return rc;
            }
            memcpy(slot->pinned, gp->img.bytes.data(), gp->img.bytes.size());
        }
        hit = slot;
    }
    hit->used = ++g_cache_clock;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return hip_status(hipGetLastError());
    if (cs != hipStreamCaptureStatusNone) hit->captured = true;
    const GroupPlan &gp = *hit->plan;
    if (int rc = enqueue_setup(gp, hit->pinned, s)) return rc;
    // (a captured copy is never waited for: its slot is kept)
    if (hit->copied && cs == hipStreamCaptureStatusNone && hipEventRecord(hit->copied, s) != hipSuccess)
        return hip_status(hipGetLastError());
    return run_plan(gp, 3, s);
}

lb_linear_desc desc_of(const lb_linear_call &c) {
    lb_linear_desc d{};
    d.x = c.x;
    d.y = c.y;
    d.w = c.w;
    d.d_in = c.d_in;
    d.d_out = c.d_out;
    d.r = c.r;
    d.residual = c.residual;
    return d;
}

bool same_group(const lb_linear_call &a, const lb_linear_call &b) {
    return a.T == b.T && a.x_dtype == b.x_dtype && a.y_dtype == b.y_dtype && a.flags == b.flags;
}

// The calls' sub-groups (equal T, dtypes and flags), in order of first appearance.
std::vector<std::vector<int>> sub_groups(const lb_linear_call *calls, int n) {
    std::vector<std::vector<int>> gs;
    for (int i = 0; i < n; ++i) {
        bool placed = false;
        for (auto &g : gs)
            if (same_group(calls[g[0]], calls[i])) { g.push_back(i); placed = true; break; }
        if (!placed) gs.push_back({i});
    }
    return gs;
}
}  // namespace

extern "C" {

size_t lb_grouped_workspace_bytes(const lb_linear_desc *descs, int n, int64_t T, unsigned flags) {
    return group_ws_bytes(descs, n, T, flags);
}

int lb_grouped_prepare(const lb_linear_desc *descs, int n, int64_t T, int x_dtype, int y_dtype,
                       void *ws, size_t ws_bytes, unsigned flags, void *stream) {
    auto gp = std::make_shared<GroupPlan>();
    if (int rc = build_plan(descs, n, T, x_dtype, y_dtype, ws, ws_bytes, flags, gp.get())) return rc;
    hipStream_t s = (hipStream_t)stream;
    // blocking: the host image is copied out before this returns
    if (int rc = enqueue_setup(*gp, gp->img.bytes.data(), s)) return rc;
    if (int rc = hip_status(hipStreamSynchronize(s))) return rc;
    gp->img.bytes.clear();
    gp->img.bytes.shrink_to_fit();
    std::lock_guard<std::mutex> lk(g_groups_mu);
    g_groups[ws] = std::move(gp);
    return LB_OK;
}

int lb_grouped_release(void *ws) {
    std::lock_guard<std::mutex> lk(g_groups_mu);
    auto it = g_groups.find(ws);
    if (it == g_groups.end()) return LB_EINVAL;
    g_groups.erase(it);
    return LB_OK;
}

int lb_grouped_run(void *ws, void *stream) {
    const std::shared_ptr<const GroupPlan> gp = find_group(ws);
    if (!gp) return LB_EINVAL;
    return run_plan(*gp, 3, (hipStream_t)stream);
}

int lb_grouped_run_stage(void *ws, int stage, void *stream) {
    if (stage != 1 && stage != 2) return LB_EINVAL;
    const std::shared_ptr<const GroupPlan> gp = find_group(ws);
    if (!gp) return LB_EINVAL;
    if (gp->kind == GroupKind::Loop) return LB_EUNSUPPORTED;
    return run_plan(*gp, stage, (hipStream_t)stream);
}

size_t lb_linear_grouped_workspace_bytes(const lb_linear_call *calls, int n) {
    if (!calls || n <= 0) return 0;
    size_t need = 0;
    for (const std::vector<int> &g : sub_groups(calls, n)) {
        const lb_linear_call &c0 = calls[g[0]];
        if (c0.T == 0) continue;
        std::vector<lb_linear_desc> ds;
        for (int i : g) ds.push_back(desc_of(calls[i]));
        const size_t b = group_ws_bytes(ds.data(), (int)ds.size(), c0.T, c0.flags);
        if (b == 0) return 0;
        need = std::max(need, b);
    }
    return need;
}

int lb_linear_forward_grouped(const lb_linear_call *calls, int n, void *ws, size_t ws_bytes, void *stream) {
    if (!calls || n <= 0) return LB_EINVAL;
    const std::vector<std::vector<int>> gs = sub_groups(calls, n);
    // every call is checked before anything is enqueued
    for (int i = 0; i < n; ++i) {
        const lb_linear_call &c = calls[i];
        if (c.T < 0 || (c.flags & ~kGroupFlags)) return LB_EINVAL;
        Linear a{};
        int rc;
        if ((rc = check_shape(c.d_in, c.d_out, c.r, c.T, c.residual, &a))) return rc;
        if ((rc = check_factors(&c.w, &a))) return rc;
        if ((rc = check_io(c.x, c.x_dtype, c.y, c.y_dtype, &a))) return rc;
        Path p;
        if ((rc = choose_path(c.flags & kLinearFlags, c.T, c.y_dtype, &p))) return rc;
    }
    const size_t need = lb_linear_grouped_workspace_bytes(calls, n);
    if (need > 0 && (!ws || ws_bytes < need)) return LB_EWORKSPACE;
    for (const std::vector<int> &g : gs) {
        const lb_linear_call &c0 = calls[g[0]];
        if (c0.T == 0) continue;
        std::vector<lb_linear_desc> ds;
        for (int i : g) ds.push_back(desc_of(calls[i]));
        if (int rc = run_stateless(ds.data(), (int)ds.size(), c0.T, c0.x_dtype, c0.y_dtype, ws, ws_bytes,
                                   c0.flags, (hipStream_t)stream))
            return rc;
    }
    return LB_OK;
}

int lb_device_faults(void *stream, uint32_t *faults) {
    uint32_t f = 0;
    if (int rc = take_faults((hipStream_t)stream, &f)) return rc;
    if (faults) *faults = f;
    return f ? LB_EDEVICE : LB_OK;
}

int lb_linear_path(int64_t d_in, int64_t d_out, int64_t r, int64_t T, int residual, int x_dtype, int y_dtype,
                   unsigned flags) {
    Linear a{};
    int rc;
    if ((rc = check_shape(d_in, d_out, r, T, residual, &a))) return rc;
    if (!valid_dtype(x_dtype) || !valid_dtype(y_dtype) || (flags & ~kLinearFlags)) return LB_EINVAL;
    a.x_dtype = x_dtype;
    a.y_dtype = y_dtype;
    a.ld_v = lb_packed_ld_aligned(a.r_p);
    a.ld_u = lb_packed_ld_aligned(d_out);
    Path p;
    if ((rc = choose_path(flags, T, y_dtype, &p, &a))) return rc;
    if (p == Path::Gemm && !gemm_linear_supported(a)) p = Path::Valu;
    return p == Path::MfmaDecode ? (int)LB_PATH_DECODE : p == Path::Gemm ? (int)LB_PATH_PREFILL
                                                                          : (int)LB_PATH_DECODE_VALU;
}

}  // extern "C"
