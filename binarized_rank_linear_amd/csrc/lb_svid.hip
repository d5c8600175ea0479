// lb_svid.hip -- Dual-SVID initialisation of a LittleBit linear from a dense
// weight (sesamedisk, "How low-rank binarization works", the Dual-SVID
// paragraph; mlsanity, abstract): a truncated SVD gives the starting latent
// factors, the binary factors are their signs, rank-1 fits of the factor
// magnitudes give the scales, and a residual path is fitted the same way to
// what the first path leaves.  Off the forward path: it produces the packed
// factors the forward kernels read.
//
// The SVD is one-sided Jacobi (Hestenes): the columns of A (W or W^T, the
// longer side down the columns) are rotated pairwise until every pair is
// orthogonal; then A = U S and the accumulated rotations are V.  A round
// rotates n/2 disjoint column pairs (the circle schedule), one workgroup per
// pair; n - 1 rounds are a sweep; sweeps repeat until no pair needed a
// rotation.  Dot products accumulate in fp64, the columns stay fp32.
#include <math.h>

#include "lb_internal.h"

namespace lb {
namespace {

constexpr int kT = 256;
constexpr double kOrthTol = 1e-6;        // a pair is orthogonal when |a_p.a_q| <= tol |a_p| |a_q|
// A column whose squared norm is below kZeroRel |A|_F^2 is numerically zero
// (rank deficiency): pairs with one are left alone.  Without this, null-space
// columns keep rotating among themselves at ever smaller (finally subnormal)
// scales and the sweeps never settle.
constexpr double kZeroRel = 1e-12;
constexpr int kMaxSweeps = 40;
constexpr int kPowerIters = 100;         // rank-1 fits: power iterations

__device__ __forceinline__ double block_sum(double v, double *red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < kT / 64; ++w) t += red[w];
    return t;
}

// A [n][m] column-major (column c = m floats): from row-major W [d_out][d_in],
// A = W (m = d_out, n = d_in) or A = W^T (m = d_in, n = d_out).
__global__ __launch_bounds__(kT) void k_load_columns(const float *__restrict__ w, int64_t d_out, int64_t d_in,
                                                     int transpose, float *__restrict__ a) {
    const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
    if (e >= d_out * d_in) return;
    const int64_t i = e / d_in, j = e - i * d_in;        // W[i][j]
    if (transpose) a[i * d_in + j] = w[e];               // column i of W^T is row i of W
    else a[j * d_out + i] = w[e];                        // column j of W
}

__global__ __launch_bounds__(kT) void k_identity(float *__restrict__ v, int64_t n) {
    const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
    if (e < n * n) v[e] = (e / n == e % n) ? 1.0f : 0.0f;
}

// One round of the circle schedule over N (= n rounded up to even) slots:
// pair 0 is (N-1, r), pair k is ((r+k) mod (N-1), (r-k) mod (N-1)); slot n
// (when n is odd) is empty.  Workgroup k rotates pair k of round r.
__global__ __launch_bounds__(kT) void k_jacobi_round(float *__restrict__ a, float *__restrict__ v, int64_t m,
                                                     int64_t n, int64_t N, int64_t r, const double *__restrict__ zero,
                                                     int *__restrict__ rotated) {
    const int64_t k = blockIdx.x;
    int64_t p, q;
    if (k == 0) {
        p = N - 1;
        q = r;
    } else {
        p = (r + k) % (N - 1);
        q = (r - k + (N - 1)) % (N - 1);
    }
    if (p >= n || q >= n) return;                        // the empty slot (uniform)
    float *ap = a + p * m, *aq = a + q * m;
    double al = 0.0, be = 0.0, ga = 0.0;
    for (int64_t i = threadIdx.x; i < m; i += kT) {
        const double x = ap[i], y = aq[i];
        al += x * x;
        be += y * y;
        ga += x * y;
    }
    __shared__ double red[kT / 64];
    al = block_sum(al, red);
    be = block_sum(be, red);
    ga = block_sum(ga, red);
    if (al <= *zero || be <= *zero) return;              // a numerically zero column (uniform)
    if (!(fabs(ga) > kOrthTol * sqrt(al * be))) return;  // orthogonal already (uniform)
    if (threadIdx.x == 0) atomicOr(rotated, 1);
    const double zeta = (be - al) / (2.0 * ga);
    const double t = (zeta >= 0.0 ? 1.0 : -1.0) / (fabs(zeta) + sqrt(1.0 + zeta * zeta));
    const double cd = 1.0 / sqrt(1.0 + t * t);
    const float c = (float)cd, s = (float)(cd * t);
    for (int64_t i = threadIdx.x; i < m; i += kT) {
        const float x = ap[i], y = aq[i];
        ap[i] = c * x - s * y;
        aq[i] = s * x + c * y;
    }
    float *vp = v + p * n, *vq = v + q * n;
    for (int64_t i = threadIdx.x; i < n; i += kT) {
        const float x = vp[i], y = vq[i];
        vp[i] = c * x - s * y;
        vq[i] = s * x + c * y;
    }
}

// *zero = kZeroRel |A|_F^2 (one workgroup, fixed summation order).
__global__ __launch_bounds__(kT) void k_zero_level(const float *__restrict__ a, int64_t n, double *__restrict__ zero) {
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += kT) s += (double)a[i] * a[i];
    __shared__ double red[kT / 64];
    s = block_sum(s, red);
    if (threadIdx.x == 0) *zero = kZeroRel * s;
}

// sigma[j] = |column j of A|; one workgroup per column.
__global__ __launch_bounds__(kT) void k_column_norms(const float *__restrict__ a, int64_t m,
                                                     float *__restrict__ sigma) {
    const float *c = a + (int64_t)blockIdx.x * m;
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < m; i += kT) s += (double)c[i] * c[i];
    __shared__ double red[kT / 64];
    s = block_sum(s, red);
    if (threadIdx.x == 0) sigma[blockIdx.x] = (float)sqrt(s);
}

// order[rank] = j, ranks by decreasing sigma (ties by index).
__global__ __launch_bounds__(kT) void k_rank(const float *__restrict__ sigma, int64_t n, int32_t *__restrict__ order) {
    const int64_t j = (int64_t)blockIdx.x * kT + threadIdx.x;
    if (j >= n) return;
    const float sj = sigma[j];
    int64_t rank = 0;
    for (int64_t k = 0; k < n; ++k) {
        const float sk = sigma[k];
        rank += (sk > sj || (sk == sj && k < j)) ? 1 : 0;
    }
    order[rank] = (int32_t)j;
}

// The top r_p triplets as the two latent factors, each holding sqrt(sigma):
// U' [d_out][r_p] and V' [d_in][r_p], row-major.  A = W: U' column = a_j /
// sqrt(s_j), V' column = v_j sqrt(s_j); A = W^T: the two roles swap.
__global__ __launch_bounds__(kT) void k_take_factors(const float *__restrict__ a, const float *__restrict__ v,
                                                     const float *__restrict__ sigma, const int32_t *__restrict__ order,
                                                     int64_t m, int64_t n, int transpose, int64_t d_out,
                                                     int64_t d_in, int64_t r_p, float *__restrict__ up,
                                                     float *__restrict__ vp) {
    const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
    const int64_t nu = d_out * r_p;
    if (e >= nu + d_in * r_p) return;
    const bool is_u = e < nu;
    const int64_t row = is_u ? e / r_p : (e - nu) / r_p;
    const int64_t k = is_u ? e % r_p : (e - nu) % r_p;
    const int64_t j = order[k];
    const float s = sigma[j];
    const float root = sqrtf(s);
    // from A (left vectors scaled by s): divide by sqrt(s); from V: multiply
    const bool from_a = is_u != (transpose != 0);
    float val;
    if (from_a) val = s > 0.0f ? a[j * m + row] / root : 0.0f;
    else val = v[j * n + row] * root;
    if (is_u) up[e] = val;
    else vp[e - nu] = val;
}

// Rank-1 fit of |M| (M [rows][cols] row-major) by power iteration:
// y = |M|^T x, normalised; x = |M| y, its norm the singular value, normalised.
__global__ __launch_bounds__(kT) void k_abs_mtv(const float *__restrict__ mtx, int64_t rows, int64_t cols,
                                                const float *__restrict__ x, float *__restrict__ y) {
    const int64_t k = (int64_t)blockIdx.x * kT + threadIdx.x;
    if (k >= cols) return;
    double s = 0.0;
    for (int64_t i = 0; i < rows; ++i) s += (double)fabsf(mtx[i * cols + k]) * x[i];
    y[k] = (float)s;
}

__global__ __launch_bounds__(kT) void k_abs_mv(const float *__restrict__ mtx, int64_t rows, int64_t cols,
                                               const float *__restrict__ y, float *__restrict__ x) {
    const int64_t i = blockIdx.x;
    double s = 0.0;
    for (int64_t k = threadIdx.x; k < cols; k += kT) s += (double)fabsf(mtx[i * cols + k]) * y[k];
    __shared__ double red[kT / 64];
    s = block_sum(s, red);
    if (threadIdx.x == 0) x[i] = (float)s;
}

// v /= |v| (one workgroup); the norm goes to *norm when given.
__global__ __launch_bounds__(kT) void k_normalise(float *__restrict__ v, int64_t n, float *__restrict__ norm) {
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += kT) s += (double)v[i] * v[i];
    __shared__ double red[kT / 64];
    s = block_sum(s, red);
    const double nr = sqrt(s);
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += kT) v[i] = nr > 0.0 ? (float)(v[i] / nr) : 0.0f;
    if (norm && threadIdx.x == 0) *norm = (float)nr;
}

__global__ __launch_bounds__(kT) void k_fill(float *__restrict__ v, int64_t n, float val) {
    const int64_t i = (int64_t)blockIdx.x * kT + threadIdx.x;
    if (i < n) v[i] = val;
}

// The stored scales: h = sqrt(s_u) a, g = sqrt(s_v) c, l = (sqrt(s_u) b) (.)
// (sqrt(s_v) d), rounded to fp16 (nearest even); also as fp32 for the
// remainder.
__global__ __launch_bounds__(kT) void k_scales(const float *__restrict__ xa, const float *__restrict__ yb,
                                               const float *__restrict__ su, const float *__restrict__ xc,
                                               const float *__restrict__ yd, const float *__restrict__ sv,
                                               int64_t d_out, int64_t d_in, int64_t r_p, uint16_t *__restrict__ h,
                                               uint16_t *__restrict__ g, uint16_t *__restrict__ l,
                                               float *__restrict__ h32, float *__restrict__ g32,
                                               float *__restrict__ l32) {
    const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
    const float ru = sqrtf(*su), rv = sqrtf(*sv);
    auto f16 = [](float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); };
    auto back = [](uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); };
    if (e < d_out) {
        const uint16_t b = f16(ru * xa[e]);
        h[e] = b;
        h32[e] = back(b);
    } else if (e < d_out + d_in) {
        const int64_t j = e - d_out;
        const uint16_t b = f16(rv * xc[j]);
        g[j] = b;
        g32[j] = back(b);
    } else if (e < d_out + d_in + r_p) {
        const int64_t k = e - d_out - d_in;
        const uint16_t b = f16((ru * yb[k]) * (rv * yd[k]));
        l[k] = b;
        l32[k] = back(b);
    }
}

// R = W - h_i g_j sum_k l_k sign(U'[i][k]) sign(V'[j][k]): the remainder the
// residual path fits.  64 x 64 outputs per workgroup, 4 x 4 per thread; the
// signs (l folded into the V side) of 16 latents at a time in LDS.
constexpr int kRT = 64, kRK = 16;
__global__ __launch_bounds__(kT) void k_remainder(const float *__restrict__ w, const float *__restrict__ up,
                                                  const float *__restrict__ vp, const float *__restrict__ h32,
                                                  const float *__restrict__ g32, const float *__restrict__ l32,
                                                  int64_t d_out, int64_t d_in, int64_t r_p, float *__restrict__ r) {
    __shared__ float su[kRK][kRT], sv[kRK][kRT];
    const int64_t i0 = (int64_t)blockIdx.y * kRT, j0 = (int64_t)blockIdx.x * kRT;
    const int ti = threadIdx.x / 16, tj = threadIdx.x % 16;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < r_p; k0 += kRK) {
        for (int e = threadIdx.x; e < kRK * kRT; e += kT) {
            const int kk = e / kRT, rr = e % kRT;
            const int64_t k = k0 + kk, i = i0 + rr, j = j0 + rr;
            su[kk][rr] = (k < r_p && i < d_out) ? (up[i * r_p + k] < 0.0f ? -1.0f : 1.0f) : 0.0f;
            sv[kk][rr] = (k < r_p && j < d_in) ? (vp[j * r_p + k] < 0.0f ? -l32[k] : l32[k]) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kRK; ++kk) {
            float a4[4], b4[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a4[q] = su[kk][ti * 4 + q];
                b4[q] = sv[kk][tj * 4 + q];
            }
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[x][y] += a4[x] * b4[y];
        }
        __syncthreads();
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            const int64_t i = i0 + ti * 4 + x, j = j0 + tj * 4 + y;
            if (i < d_out && j < d_in) r[i * d_in + j] = w[i * d_in + j] - h32[i] * g32[j] * acc[x][y];
        }
}

size_t rup256(size_t n) { return (n + 255) & ~(size_t)255; }

struct SvidLayout {
    int64_t m, n;
    size_t a, v, sigma, order, up, vp, rem, x, y, s, h32, g32, l32, flag, zero, itq, total;
};

// up and vp are adjacent (U' then V': the matrix F = [U'; V'] Joint-ITQ turns).
SvidLayout svid_layout(int64_t d_out, int64_t d_in, int64_t r_p, bool residual, bool itq) {
    SvidLayout L;
    L.m = d_out >= d_in ? d_out : d_in;
    L.n = d_out >= d_in ? d_in : d_out;
    size_t at = 0;
    auto take = [&](size_t b) { const size_t o = at; at += rup256(b); return o; };
    L.a = take((size_t)(L.m * L.n) * 4);
    L.v = take((size_t)(L.n * L.n) * 4);
    L.sigma = take((size_t)L.n * 4);
    L.order = take((size_t)L.n * 4);
    L.up = take((size_t)((d_out + d_in) * r_p) * 4);
    L.vp = L.up + (size_t)(d_out * r_p) * 4;
    L.rem = residual ? take((size_t)(d_out * d_in) * 4) : 0;
    L.x = take((size_t)(d_out + d_in) * 4);               // a (rows of U') then c (rows of V')
    L.y = take((size_t)(2 * r_p) * 4);                   // b then d
    L.s = take(4 * 4);                                    // the two fits' singular values
    L.h32 = take((size_t)d_out * 4);
    L.g32 = take((size_t)d_in * 4);
    L.l32 = take((size_t)r_p * 4);
    L.flag = take(4);
    L.zero = take(8);
    L.itq = itq ? take(itq_workspace_bytes(d_out + d_in, r_p)) : 0;
    L.total = at;
    return L;
}

unsigned grid_of(int64_t n) { return (unsigned)cdiv(n, kT); }

// Rank-1 fit of |M|: x (rows, unit), y (cols, unit) and the singular value.
int rank1_fit(const float *mtx, int64_t rows, int64_t cols, float *x, float *y, float *s, hipStream_t st) {
    k_fill<<<grid_of(rows), kT, 0, st>>>(x, rows, 1.0f);
    k_normalise<<<1, kT, 0, st>>>(x, rows, nullptr);
    for (int it = 0; it < kPowerIters; ++it) {
        k_abs_mtv<<<grid_of(cols), kT, 0, st>>>(mtx, rows, cols, x, y);
        k_normalise<<<1, kT, 0, st>>>(y, cols, nullptr);
        k_abs_mv<<<(unsigned)rows, kT, 0, st>>>(mtx, rows, cols, y, x);
        k_normalise<<<1, kT, 0, st>>>(x, rows, s);
    }
    return last_launch_status();
}

// One path on the weight at `w` (row-major [d_out][d_in]): factors, scales and
// packed signs of path p of `out`.
int svid_path(const float *w, int64_t d_out, int64_t d_in, int64_t r_p, int p, const lb_factors *out,
              float *u_out, float *v_out, int itq_iters, uint8_t *ws, const SvidLayout &L, hipStream_t st) {
    float *a = (float *)(ws + L.a), *v = (float *)(ws + L.v), *sigma = (float *)(ws + L.sigma);
    int32_t *order = (int32_t *)(ws + L.order);
    float *up = (float *)(ws + L.up), *vp = (float *)(ws + L.vp);
    int *flag = (int *)(ws + L.flag);
    const int64_t m = L.m, n = L.n;
    const int transpose = d_out >= d_in ? 0 : 1;
    k_load_columns<<<grid_of(d_out * d_in), kT, 0, st>>>(w, d_out, d_in, transpose, a);
    k_identity<<<grid_of(n * n), kT, 0, st>>>(v, n);
    double *zero = (double *)(ws + L.zero);
    k_zero_level<<<1, kT, 0, st>>>(a, m * n, zero);
    if (int rc = last_launch_status()) return rc;
    const int64_t N = n + (n & 1);
    bool converged = n < 2;
    for (int sweep = 0; sweep < kMaxSweeps && !converged; ++sweep) {
        if (int rc = fill_words(flag, 4, 0u, st)) return rc;
        for (int64_t r = 0; r < N - 1; ++r)
            k_jacobi_round<<<(unsigned)(N / 2), kT, 0, st>>>(a, v, m, n, N, r, zero, flag);
        if (int rc = last_launch_status()) return rc;
        int h = 0;
        if (hipMemcpyAsync(&h, flag, 4, hipMemcpyDeviceToHost, st) != hipSuccess || hipStreamSynchronize(st) != hipSuccess)
            return hip_status(hipGetLastError());
        converged = h == 0;
    }
    if (!converged) return LB_EUNSUPPORTED;
    k_column_norms<<<(unsigned)n, kT, 0, st>>>(a, m, sigma);
    k_rank<<<grid_of(n), kT, 0, st>>>(sigma, n, order);
    k_take_factors<<<grid_of((d_out + d_in) * r_p), kT, 0, st>>>(a, v, sigma, order, m, n, transpose, d_out, d_in,
                                                                   r_p, up, vp);
    if (int rc = last_launch_status()) return rc;
    // LittleBit-2: turn both factors by the Joint-ITQ rotation before the signs
    if (itq_iters > 0)
        if (int rc = itq_rotate(up, d_out + d_in, r_p, itq_iters, nullptr, nullptr, nullptr, ws + L.itq, st))
            return rc;
    // rank-1 fits of |U'| and |V'|
    float *xa = (float *)(ws + L.x), *xc = xa + d_out, *yb = (float *)(ws + L.y), *yd = yb + r_p;
    float *s = (float *)(ws + L.s);
    if (int rc = rank1_fit(up, d_out, r_p, xa, yb, s, st)) return rc;
    if (int rc = rank1_fit(vp, d_in, r_p, xc, yd, s + 1, st)) return rc;
    uint16_t *h = (uint16_t *)out->h + (int64_t)p * d_out, *g = (uint16_t *)out->g + (int64_t)p * d_in;
    uint16_t *l = (uint16_t *)out->l + (int64_t)p * r_p;
    k_scales<<<grid_of(d_out + d_in + r_p), kT, 0, st>>>(xa, yb, s, xc, yd, s + 1, d_out, d_in, r_p, h, g, l,
                                                         (float *)(ws + L.h32), (float *)(ws + L.g32),
                                                         (float *)(ws + L.l32));
    if (int rc = last_launch_status()) return rc;
    // signs, packed as the forward kernels read them
    const int64_t kw_v = cdiv(d_in, 32), kw_u = cdiv(r_p, 32);
    if (int rc = launch_pack(vp, d_in, r_p, 0, (uint32_t *)out->v_bits + (int64_t)p * kw_v * out->ld_v, out->ld_v, st))
        return rc;
    if (int rc = launch_pack(up, d_out, r_p, 1, (uint32_t *)out->u_bits + (int64_t)p * kw_u * out->ld_u, out->ld_u, st))
        return rc;
    if (u_out && hipMemcpyAsync(u_out + (int64_t)p * d_out * r_p, up, (size_t)(d_out * r_p) * 4,
                                hipMemcpyDeviceToDevice, st) != hipSuccess)
        return hip_status(hipGetLastError());
    if (v_out && hipMemcpyAsync(v_out + (int64_t)p * d_in * r_p, vp, (size_t)(d_in * r_p) * 4,
                                hipMemcpyDeviceToDevice, st) != hipSuccess)
        return hip_status(hipGetLastError());
    return LB_OK;
}

int svid_check(const float *w, int64_t d_out, int64_t d_in, int64_t r, int residual, const lb_factors *out) {
    if (!w || !out || d_out <= 0 || d_in <= 0 || r <= 0) return LB_EINVAL;
    const int P = residual ? 2 : 1;
    if (r % P) return LB_EINVAL;
    const int64_t r_p = r / P;
    if (r_p > (d_out < d_in ? d_out : d_in)) return LB_EINVAL;    // at most the rank of W
    if (!out->v_bits || !out->u_bits || !out->g || !out->l || !out->h) return LB_EINVAL;
    if (out->ld_v < r_p || out->ld_u < d_out) return LB_EINVAL;
    if (((uintptr_t)w & 3) || ((uintptr_t)out->v_bits & 3) || ((uintptr_t)out->u_bits & 3)) return LB_EALIGN;
    // column-major A and every buffer's 32-bit element offsets
    if (d_out * d_in >= (1ll << 31) || d_out >= (1 << 24) || d_in >= (1 << 24)) return LB_EUNSUPPORTED;
    return LB_OK;
}

}  // namespace
}  // namespace lb

namespace lb {
namespace {

int dual_svid_run(const float *w, int64_t d_out, int64_t d_in, int64_t r, int residual, int itq_iters,
                  const lb_factors *out, float *u_out, float *v_out, void *ws, size_t ws_bytes, void *stream) {
    if (int rc = svid_check(w, d_out, d_in, r, residual, out)) return rc;
    if (itq_iters < 0) return LB_EINVAL;
    const int64_t r_p = r / (residual ? 2 : 1);
    const SvidLayout L = svid_layout(d_out, d_in, r_p, residual != 0, itq_iters > 0);
    if (!ws || ws_bytes < L.total) return LB_EWORKSPACE;
    if ((uintptr_t)ws & 255) return LB_EALIGN;
    hipStream_t st = (hipStream_t)stream;
    uint8_t *wsb = (uint8_t *)ws;
    if (int rc = svid_path(w, d_out, d_in, r_p, 0, out, u_out, v_out, itq_iters, wsb, L, st)) return rc;
    if (!residual) return LB_OK;
    float *rem = (float *)(wsb + L.rem);
    dim3 grid((unsigned)cdiv(d_in, kRT), (unsigned)cdiv(d_out, kRT));
    k_remainder<<<grid, kT, 0, st>>>(w, (const float *)(wsb + L.up), (const float *)(wsb + L.vp),
                                     (const float *)(wsb + L.h32), (const float *)(wsb + L.g32),
                                     (const float *)(wsb + L.l32), d_out, d_in, r_p, rem);
    if (int rc = last_launch_status()) return rc;
    return svid_path(rem, d_out, d_in, r_p, 1, out, u_out, v_out, itq_iters, wsb, L, st);
}

}  // namespace
}  // namespace lb

extern "C" size_t lb_dual_svid_workspace_bytes(int64_t d_out, int64_t d_in, int64_t r, int residual) {
    if (d_out <= 0 || d_in <= 0 || r <= 0 || r % (residual ? 2 : 1)) return 0;
    return lb::svid_layout(d_out, d_in, r / (residual ? 2 : 1), residual != 0, false).total;
}

extern "C" int lb_dual_svid(const float *w, int64_t d_out, int64_t d_in, int64_t r, int residual,
                            const lb_factors *out, float *u_out, float *v_out, void *ws, size_t ws_bytes,
                            void *stream) {
    return lb::dual_svid_run(w, d_out, d_in, r, residual, 0, out, u_out, v_out, ws, ws_bytes, stream);
}

extern "C" size_t lb_dual_svid_itq_workspace_bytes(int64_t d_out, int64_t d_in, int64_t r, int residual) {
    if (d_out <= 0 || d_in <= 0 || r <= 0 || r % (residual ? 2 : 1)) return 0;
    return lb::svid_layout(d_out, d_in, r / (residual ? 2 : 1), residual != 0, true).total;
}

extern "C" int lb_dual_svid_itq(const float *w, int64_t d_out, int64_t d_in, int64_t r, int residual,
                                int itq_iters, const lb_factors *out, float *u_out, float *v_out, void *ws,
                                size_t ws_bytes, void *stream) {
    return lb::dual_svid_run(w, d_out, d_in, r, residual, itq_iters, out, u_out, v_out, ws, ws_bytes, stream);
}
