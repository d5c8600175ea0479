// lb_api.hip -- the C entry points of littlebit.h: argument checks, path
// dispatch, workspace sizing, the SwiGLU block and layer groups.
#include <mutex>
#include <string.h>
#include <unordered_map>
#include <vector>

#include "lb_internal.h"

using namespace lb;

namespace {

constexpr int64_t kDecodeMaxT = 32;     // token count served by the decode kernels

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t act_size(int dtype) { return dtype == LB_F32 ? 4 : 2; }

bool valid_dtype(int d) { return d == LB_F32 || d == LB_BF16; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

enum class Path { Valu, MfmaDecode, Gemm };

// The path a request runs on.  Returns false for an invalid or unsupported flag.
int choose_path(unsigned flags, int64_t T, int y_dtype, Path *out) {
    switch (flags & LB_PATH_MASK) {
        case LB_PATH_AUTO:
            if (T <= kDecodeMaxT)
                *out = mfma_decode_supported(T, y_dtype) ? Path::MfmaDecode : Path::Valu;
            else
                *out = y_dtype == LB_BF16 ? Path::Gemm : Path::Valu;
            return LB_OK;
        case LB_PATH_DECODE:
            *out = mfma_decode_supported(T, y_dtype) ? Path::MfmaDecode : Path::Valu;
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
    a.x_dtype = a.y_dtype = LB_BF16;
    size_t need = 0;
    // AUTO may pick either path for T > 32 depending on the output dtype.
    const int ys[2] = {LB_BF16, LB_F32};
    for (int yi = 0; yi < 2; ++yi) {
        Path p;
        if (choose_path(flags, T, ys[yi], &p)) continue;
        const size_t b = path_workspace(p, a);
        if (b > need) need = b;
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
    Path p;
    if ((rc = choose_path(flags, T, y_dtype, &p))) return rc;
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

// ---- SwiGLU block ----------------------------------------------------------

static size_t mlp_linear_ws(int64_t d_model, int64_t d_ff, int64_t r_gu, int64_t r_down, int64_t T,
                            int residual, unsigned flags) {
    const size_t a = lb_linear_workspace_bytes(d_model, d_ff, r_gu, T, residual, flags);
    const size_t b = lb_linear_workspace_bytes(d_ff, d_model, r_down, T, residual, flags);
    return a > b ? a : b;
}

size_t lb_mlp_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t r_gu, int64_t r_down,
                              int64_t T, int residual, unsigned flags) {
    Linear a{};
    if (check_shape(d_model, d_ff, r_gu, T, residual, &a)) return 0;
    if (check_shape(d_ff, d_model, r_down, T, residual, &a)) return 0;
    const size_t inter = rup256((size_t)(T * d_ff) * sizeof(float));
    return 2 * inter + mlp_linear_ws(d_model, d_ff, r_gu, r_down, T, residual, flags);
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
    if ((rc = check_io(x, x_dtype, y, y_dtype, &ad))) return rc;
    if (overlap(x, (size_t)(T * d_model) * act_size(x_dtype), y,
                (size_t)(T * d_model) * act_size(y_dtype)))
        return LB_EINVAL;
    Path p;
    if ((rc = choose_path(flags, T, y_dtype, &p))) return rc;
    if (T == 0) return LB_OK;
    const size_t need = lb_mlp_workspace_bytes(d_model, d_ff, r_gu, r_down, T, residual, flags);
    if (!ws || ws_bytes < need) return LB_EWORKSPACE;
    if (!aligned(ws, 256)) return LB_EALIGN;
    if (overlap(ws, need, x, (size_t)(T * d_model) * act_size(x_dtype)) ||
        overlap(ws, need, y, (size_t)(T * d_model) * act_size(y_dtype)))
        return LB_EINVAL;
    const size_t inter = rup256((size_t)(T * d_ff) * sizeof(float));
    float *zg = (float *)ws;
    float *zu = (float *)((char *)ws + inter);
    void *lws = (char *)ws + 2 * inter;
    hipStream_t s = (hipStream_t)stream;
    // gate and up read the same x; the intermediate stays fp32.
    ag.x = au.x = x;
    ag.x_dtype = au.x_dtype = x_dtype;
    ag.y = zg;
    au.y = zu;
    ag.y_dtype = au.y_dtype = LB_F32;
    Path pi;
    if ((rc = choose_path(flags, T, LB_F32, &pi))) pi = Path::Valu;
    if (p == Path::Gemm) pi = Path::Gemm;
    if ((rc = run_path(pi, ag, lws, s))) return rc;
    if ((rc = run_path(pi, au, lws, s))) return rc;
    if ((rc = launch_swiglu_f32(zg, zu, T * d_ff, s))) return rc;
    ad.x = zg;
    ad.x_dtype = LB_F32;
    return run_path(p, ad, lws, s);
}

// ---- layer groups ----------------------------------------------------------

namespace {
enum class GroupKind { Loop, Decode, Gemm };

struct GroupRecord {
    std::vector<lb_linear_desc> descs;
    int64_t T;
    int x_dtype, y_dtype;
    unsigned flags;
    size_t ws_bytes;
    GroupKind kind;                   // Decode / Gemm: whole-group kernels
    std::vector<uint8_t> state;       // their host-side launch state
};

std::mutex g_groups_mu;
std::unordered_map<void *, GroupRecord> g_groups;

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
    }
    return true;
}

GroupKind group_kind(unsigned flags, int64_t T, int y_dtype, const std::vector<Linear> &ls) {
    Path p;
    if (choose_path(flags, T, y_dtype, &p)) return GroupKind::Loop;
    if (p == Path::MfmaDecode) return GroupKind::Decode;
    if (p == Path::Gemm && gemm_group_supported(ls.data(), (int)ls.size())) return GroupKind::Gemm;
    return GroupKind::Loop;
}
}  // namespace

size_t lb_grouped_workspace_bytes(const lb_linear_desc *descs, int n, int64_t T, unsigned flags) {
    if (!descs || n <= 0 || T <= 0) return 0;
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
    // the linear-by-linear loop
    for (int i = 0; i < n; ++i) {
        const size_t b = lb_linear_workspace_bytes(descs[i].d_in, descs[i].d_out, descs[i].r, T,
                                                   descs[i].residual, flags);
        if (b > need) need = b;
    }
    return rup256(need) + 256;
}

int lb_grouped_prepare(const lb_linear_desc *descs, int n, int64_t T, int x_dtype, int y_dtype,
                       void *ws, size_t ws_bytes, unsigned flags, void *stream) {
    if (!descs || n <= 0 || T <= 0) return LB_EINVAL;
    Path p;
    int rc;
    if ((rc = choose_path(flags, T, y_dtype, &p))) return rc;
    std::vector<Linear> ls((size_t)n);
    for (int i = 0; i < n; ++i)
        if ((rc = group_linear(descs[i], T, x_dtype, y_dtype, &ls[(size_t)i]))) return rc;
    const size_t need = lb_grouped_workspace_bytes(descs, n, T, flags);
    if (!ws || ws_bytes < need) return LB_EWORKSPACE;
    if (!aligned(ws, 256)) return LB_EALIGN;
    GroupRecord rec;
    rec.descs.assign(descs, descs + n);
    rec.T = T;
    rec.x_dtype = x_dtype;
    rec.y_dtype = y_dtype;
    rec.flags = flags;
    rec.ws_bytes = ws_bytes;
    rec.kind = group_kind(flags, T, y_dtype, ls);
    if (rec.kind == GroupKind::Decode) {
        rec.state.assign(mfma_group_state_bytes(), 0);
        if ((rc = mfma_group_prepare(ls.data(), n, T, y_dtype, ws, ws_bytes, rec.state.data(),
                                     (hipStream_t)stream)))
            return rc;
    } else if (rec.kind == GroupKind::Gemm) {
        rec.state.assign(gemm_group_state_bytes(), 0);
        if ((rc = gemm_group_prepare(ls.data(), n, ws, ws_bytes, rec.state.data(),
                                     (hipStream_t)stream)))
            return rc;
    }
    std::lock_guard<std::mutex> lk(g_groups_mu);
    g_groups[ws] = std::move(rec);
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
    GroupRecord g;
    {
        std::lock_guard<std::mutex> lk(g_groups_mu);
        auto it = g_groups.find(ws);
        if (it == g_groups.end()) return LB_EINVAL;
        GroupRecord &rec = it->second;
        // whole-group kernels launch from the record itself, under the lock:
        // their host state advances with every run (the decode pass numbers
        // its runs)
        if (rec.kind == GroupKind::Decode) return mfma_group_run(rec.state.data(), (hipStream_t)stream);
        if (rec.kind == GroupKind::Gemm) return gemm_group_run(rec.state.data(), (hipStream_t)stream);
        g = rec;
    }
    void *lws = (char *)ws + 256;
    for (const lb_linear_desc &d : g.descs) {
        const int rc = lb_linear_forward(d.x, g.x_dtype, d.y, g.y_dtype, &d.w, d.d_in, d.d_out, d.r,
                                         g.T, d.residual, lws, g.ws_bytes - 256, g.flags, stream);
        if (rc) return rc;
    }
    return LB_OK;
}

int lb_grouped_run_stage(void *ws, int stage, void *stream) {
    if (stage != 1 && stage != 2) return LB_EINVAL;
    std::lock_guard<std::mutex> lk(g_groups_mu);
    auto it = g_groups.find(ws);
    if (it == g_groups.end()) return LB_EINVAL;
    GroupRecord &rec = it->second;
    if (rec.kind == GroupKind::Loop) return LB_EUNSUPPORTED;
    if (rec.kind == GroupKind::Gemm) return gemm_group_run(rec.state.data(), (hipStream_t)stream, stage);
    return mfma_group_run(rec.state.data(), (hipStream_t)stream, stage);
}

}  // extern "C"
