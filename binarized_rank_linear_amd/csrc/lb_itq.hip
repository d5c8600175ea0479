// lb_itq.hip -- Joint-ITQ rotation of a layer's latent factors (LittleBit-2:
// littlebitllm, hero and "The method"; trove, "How it works", step 2;
// deniz.in, "LittleBit-2 fixes the initialization").  Off the forward path: it
// turns the SVD-derived factors U' [d_out][r] and V' [d_in][r] by one shared
// orthogonal R before their signs are taken.  (U'R)(V'R)^T = U'V'^T, so the
// rotation changes only how well the signs fit the factors, and it folds into
// them: the deployed layer keeps its form.
//
// R minimises ||sign(U'R) - U'R||^2 + ||sign(V'R) - V'R||^2 by iterative
// quantisation: with R fixed the codes are the signs; with the codes B fixed
// the best orthogonal R is the polar factor of Z = U'^T B_u + V'^T B_v (the
// orthogonal Procrustes solution).  The two factors are kept as one matrix
// F = [U'; V'] ([D][r], D = d_out + d_in), so each step is
//     A = F R,  Z = F^T sign(A),  R = polar(Z)
// -- two fp32 GEMMs over the long side (on the fp32 matrix cores) and a polar
// decomposition of an r x r matrix.  The polar factor comes from the Newton-Schulz iteration
// X <- X (3 I - X^T X) / 2, started from Z / ||Z^T Z||_F^(1/2) (largest
// singular value at most 1): GEMMs only, no SVD.
#include <math.h>

#include "lb_internal.h"

namespace lb {
namespace {

constexpr int NT = 256;                 // threads per workgroup
constexpr int BM = 128, BN = 128, BK = 16;
constexpr int kRedBlocks = 256;         // fixed grid of the reductions (a fixed summation order)
constexpr int kMaxPolarIters = 64;
constexpr int kPolarCheckEvery = 8;     // host reads the polar state every this many iterations
constexpr float kPolarNear = 1e-2f;     // max |X^T X - I| below which two more iterations finish

// Polar-iteration states (one int in the workspace).
enum : int { kRunning = 0, kStop = 3, kKeep = 4 };

typedef float f32x16 __attribute__((ext_vector_type(16)));

// C = alpha * op(A) * s(B) over the K range of this split (blockIdx.z):
// op(A) = A ([M][K], lda) or, with TA, A^T with A stored [K][M] (lda); B is
// [K][N] (ldb); s(B) = B, or its signs (+1 for zero) with SIGNB.  128 x 128
// outputs per workgroup, K in steps of 16 through double-buffered LDS; each
// wave computes 64 x 64 of them as 2 x 2 blocks of v_mfma_f32_32x32x2_f32
// (fp32 matrix cores: lane l supplies row l%32 of the A block and column
// l%32 of the B block at k = l/32; it holds D[8(v/4) + 4(l/32) + v%4][l%32]
// in accumulator v).  Split z writes C + z * split_stride.  Does nothing
// once *stop >= kStop.
template <bool TA, bool SIGNB>
__global__ __launch_bounds__(NT) void k_sgemm(int64_t M, int64_t N, int64_t K, int64_t kchunk,
                                              const float *__restrict__ A, int64_t lda,
                                              const float *__restrict__ B, int64_t ldb, float *__restrict__ C,
                                              int64_t ldc, int64_t split_stride, float alpha,
                                              const int *__restrict__ stop) {
    if (stop && *stop >= kStop) return;
    __shared__ __align__(16) float As[2][BK][BM + 4];
    __shared__ __align__(16) float Bs[2][BK][BN + 4];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;
    const int l32 = lane & 31, kh = lane >> 5;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int64_t kb = (int64_t)blockIdx.z * kchunk;
    const int64_t ke = kb + kchunk < K ? kb + kchunk : K;
    C += (int64_t)blockIdx.z * split_stride;
    constexpr int PER = BM * BK / NT;   // 8 elements of each operand per thread and K step
    float ra[PER], rb[PER];
    auto load = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + NT * i;
            int kk, mm;
            if (TA) {
                kk = e / BM;
                mm = e % BM;
            } else {
                mm = e / BK;
                kk = e % BK;
            }
            const int64_t k = k0 + kk, m = m0 + mm;
            ra[i] = (k < ke && m < M) ? (TA ? A[k * lda + m] : A[m * lda + k]) : 0.0f;
            const int kb2 = e / BN, nn = e % BN;
            const int64_t k2 = k0 + kb2, n = n0 + nn;
            float v = 0.0f;
            if (k2 < ke && n < N) {
                v = B[k2 * ldb + n];
                if (SIGNB) v = v < 0.0f ? -1.0f : 1.0f;
            }
            rb[i] = v;
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + NT * i;
            if (TA) As[buf][e / BM][e % BM] = ra[i];
            else As[buf][e % BK][e / BK] = ra[i];
            Bs[buf][e / BN][e % BN] = rb[i];
        }
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    load(kb);
    store(0);
    __syncthreads();
    int buf = 0;
    for (int64_t k0 = kb; k0 < ke; k0 += BK) {
        const bool more = k0 + BK < ke;
        if (more) load(k0 + BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 2) {
            const float a0 = As[buf][kk + kh][wm + l32], a1 = As[buf][kk + kh][wm + 32 + l32];
            const float b0 = Bs[buf][kk + kh][wn + l32], b1 = Bs[buf][kk + kh][wn + 32 + l32];
            acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        if (more) store(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }
#pragma unroll
    for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            const int64_t col = n0 + wn + 32 * bj + l32;
            if (col >= N) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = m0 + wm + 32 * bi + 8 * (v >> 2) + 4 * kh + (v & 3);
                if (row < M) C[row * ldc + col] = alpha * acc[bi][bj][v];
            }
        }
}

// C[i][j] = alpha * sum_z parts[z][i][j] (z in order).
__global__ __launch_bounds__(NT) void k_reduce_splits(const float *__restrict__ parts, int S, int64_t M, int64_t N,
                                                      float *__restrict__ C, int64_t ldc, float alpha,
                                                      const int *__restrict__ stop) {
    if (stop && *stop >= kStop) return;
    const int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (e >= M * N) return;
    float s = 0.0f;
    for (int z = 0; z < S; ++z) s += parts[(int64_t)z * M * N + e];
    C[(e / N) * ldc + e % N] = alpha * s;
}

__device__ __forceinline__ double block_sum(double v, double *red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < NT / 64; ++w) t += red[w];
    return t;
}

__device__ __forceinline__ float block_max(float v, float *red) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float t = 0.0f;
    for (int w = 0; w < NT / 64; ++w) t = fmaxf(t, red[w]);
    return t;
}

// Partial sums (one per workgroup of a fixed grid) of (1 - |a|)^2 = (sign(a) - a)^2
// (kind 0) or of a^2 (kind 1), in fp64.
__global__ __launch_bounds__(NT) void k_sum_partial(const float *__restrict__ a, int64_t n, int kind,
                                                    double *__restrict__ part) {
    double s = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < n; i += (int64_t)kRedBlocks * NT) {
        const double v = a[i];
        const double d = kind == 0 ? 1.0 - fabs(v) : v;
        s += d * d;
    }
    __shared__ double red[NT / 64];
    s = block_sum(s, red);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// *out = sum of the partials (the objective).
__global__ __launch_bounds__(NT) void k_objective_final(const double *__restrict__ part, double *__restrict__ out) {
    __shared__ double red[NT / 64];
    const double s = block_sum(threadIdx.x < kRedBlocks ? part[threadIdx.x] : 0.0, red);
    if (threadIdx.x == 0) *out = s;
}

// Start of a polar decomposition: from sum(G^2) (G = Z^T Z) the scale
// c = ||G||_F^(1/2) >= sigma_max(Z): scal[0] = 1/c, scal[1] = 1/c^2; the state
// becomes kRunning, or kKeep when Z is zero (any R is then optimal: keep it).
__global__ __launch_bounds__(NT) void k_polar_begin(const double *__restrict__ part, float *__restrict__ scal,
                                                    int *__restrict__ state) {
    __shared__ double red[NT / 64];
    const double s = block_sum(threadIdx.x < kRedBlocks ? part[threadIdx.x] : 0.0, red);
    if (threadIdx.x == 0) {
        const double ng = sqrt(s);
        if (!(ng > 0.0) || !isfinite(ng)) {
            *state = kKeep;
            scal[0] = scal[1] = 0.0f;
        } else {
            *state = kRunning;
            scal[0] = (float)(1.0 / sqrt(ng));
            scal[1] = (float)(1.0 / ng);
        }
    }
}

// X *= scal[0], G *= scal[1] (the scaled start).
__global__ __launch_bounds__(NT) void k_polar_scale(float *__restrict__ x, float *__restrict__ g, int64_t n,
                                                    const float *__restrict__ scal, const int *__restrict__ state) {
    if (*state >= kStop) return;
    const int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (e >= n) return;
    x[e] *= scal[0];
    g[e] *= scal[1];
}

// Partial maxima of |G - I| (G [r][r]).
__global__ __launch_bounds__(NT) void k_dev_partial(const float *__restrict__ g, int64_t r, float *__restrict__ part,
                                                    const int *__restrict__ state) {
    if (*state >= kStop) return;
    float m = 0.0f;
    for (int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x; e < r * r; e += (int64_t)kRedBlocks * NT) {
        const float d = fabsf(g[e] - (e / r == e % r ? 1.0f : 0.0f));
        m = fmaxf(m, d != d ? INFINITY : d);          // a NaN counts as far away
    }
    __shared__ float red[NT / 64];
    m = block_max(m, red);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// The state after this iteration's check: once max |G - I| < kPolarNear, two
// more iterations run (the error roughly squares in each), then it stops.
__global__ __launch_bounds__(NT) void k_polar_check(const float *__restrict__ part, int *__restrict__ state) {
    if (*state >= kStop) return;
    __shared__ float red[NT / 64];
    const float m = block_max(threadIdx.x < kRedBlocks ? part[threadIdx.x] : 0.0f, red);
    if (threadIdx.x == 0) {
        const int s = *state;
        *state = s == kRunning ? (m < kPolarNear ? 1 : kRunning) : s + 1;
    }
}

// X = 1.5 X - 0.5 T, T = X G (one Newton-Schulz step).
__global__ __launch_bounds__(NT) void k_polar_combine(float *__restrict__ x, const float *__restrict__ t, int64_t n,
                                                      const int *__restrict__ state) {
    if (*state >= kStop) return;
    const int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (e < n) x[e] = 1.5f * x[e] - 0.5f * t[e];
}

// R = X when the iteration finished (kStop); kept when Z was zero (kKeep); a
// decomposition that did not finish keeps R and counts a failure.
__global__ __launch_bounds__(NT) void k_polar_end(const float *__restrict__ x, float *__restrict__ rot, int64_t n,
                                                  const int *__restrict__ state, int *__restrict__ fails) {
    const int s = *state;
    const int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (s == kStop) {
        if (e < n) rot[e] = x[e];
    } else if (s != kKeep && e == 0) {
        atomicAdd(fails, 1);
    }
}

__global__ __launch_bounds__(NT) void k_eye(float *__restrict__ v, int64_t r) {
    const int64_t e = (int64_t)blockIdx.x * NT + threadIdx.x;
    if (e < r * r) v[e] = (e / r == e % r) ? 1.0f : 0.0f;
}

__global__ __launch_bounds__(NT) void k_zero_int(int *__restrict__ p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0;
}

size_t rup256(size_t n) { return (n + 255) & ~(size_t)255; }
unsigned grid_of(int64_t n) { return (unsigned)cdiv(n, NT); }

// Split count of a GEMM with an M x N output over K: enough workgroups to
// fill the chip (about 1024), each split at least 256 deep, at most 32.
int splits_for(int64_t M, int64_t N, int64_t K) {
    const int64_t tiles = cdiv(M, BM) * cdiv(N, BN);
    int64_t s = 1024 / tiles;
    s = imin(s, K / 256);
    return (int)imax(1, imin(32, s));
}

struct ItqLayout {
    size_t af, rot, x, g, t, parts, red, redf, scal, state, fails, total;
    int s_z, s_ns;
};

ItqLayout itq_layout(int64_t D, int64_t r) {
    ItqLayout L;
    size_t at = 0;
    auto take = [&](size_t b) { const size_t o = at; at += rup256(b); return o; };
    const size_t rr = (size_t)(r * r) * 4;
    L.af = take((size_t)(D * r) * 4);
    L.rot = take(rr);
    L.x = take(rr);
    L.g = take(rr);
    L.t = take(rr);
    L.s_z = splits_for(r, r, D);
    L.s_ns = splits_for(r, r, r);
    const int sm = L.s_z > L.s_ns ? L.s_z : L.s_ns;
    L.parts = take(sm > 1 ? (size_t)sm * rr : 4);
    L.red = take(kRedBlocks * 8);
    L.redf = take(kRedBlocks * 4);
    L.scal = take(2 * 4);
    L.state = take(4);
    L.fails = take(4);
    L.total = at;
    return L;
}

// C = alpha op(A) s(B), split over K into S pieces when S > 1 (then summed in
// split order by k_reduce_splits).
template <bool TA, bool SIGNB>
int sgemm(int64_t M, int64_t N, int64_t K, const float *A, int64_t lda, const float *B, int64_t ldb, float *C,
          int64_t ldc, float alpha, int S, float *parts, const int *stop, hipStream_t st) {
    if (S <= 1) {
        dim3 grid((unsigned)cdiv(N, BN), (unsigned)cdiv(M, BM), 1);
        k_sgemm<TA, SIGNB><<<grid, NT, 0, st>>>(M, N, K, rup(K, BK), A, lda, B, ldb, C, ldc, 0, alpha, stop);
        return last_launch_status();
    }
    const int64_t kchunk = rup(cdiv(K, S), BK);
    dim3 grid((unsigned)cdiv(N, BN), (unsigned)cdiv(M, BM), (unsigned)S);
    k_sgemm<TA, SIGNB><<<grid, NT, 0, st>>>(M, N, K, kchunk, A, lda, B, ldb, parts, N, M * N, 1.0f, stop);
    k_reduce_splits<<<grid_of(M * N), NT, 0, st>>>(parts, S, M, N, C, ldc, alpha, stop);
    return last_launch_status();
}

int objective_into(const float *af, int64_t n, double *out, uint8_t *ws, const ItqLayout &L, hipStream_t st) {
    double *part = (double *)(ws + L.red);
    k_sum_partial<<<kRedBlocks, NT, 0, st>>>(af, n, 0, part);
    k_objective_final<<<1, NT, 0, st>>>(part, out);
    return last_launch_status();
}

// rot = polar(X) (X holds Z on entry and is overwritten).
int polar(int64_t r, uint8_t *ws, const ItqLayout &L, hipStream_t st) {
    float *x = (float *)(ws + L.x), *g = (float *)(ws + L.g), *t = (float *)(ws + L.t);
    float *parts = (float *)(ws + L.parts), *rot = (float *)(ws + L.rot);
    float *scal = (float *)(ws + L.scal), *redf = (float *)(ws + L.redf);
    int *state = (int *)(ws + L.state), *fails = (int *)(ws + L.fails);
    double *red = (double *)(ws + L.red);
    const int64_t n = r * r;
    // G = Z^T Z, then the scaled start
    if (int rc = sgemm<true, false>(r, r, r, x, r, x, r, g, r, 1.0f, L.s_ns, parts, nullptr, st)) return rc;
    k_sum_partial<<<kRedBlocks, NT, 0, st>>>(g, n, 1, red);
    k_polar_begin<<<1, NT, 0, st>>>(red, scal, state);
    k_polar_scale<<<grid_of(n), NT, 0, st>>>(x, g, n, scal, state);
    if (int rc = last_launch_status()) return rc;
    for (int it = 0; it < kMaxPolarIters; ++it) {
        k_dev_partial<<<kRedBlocks, NT, 0, st>>>(g, r, redf, state);
        k_polar_check<<<1, NT, 0, st>>>(redf, state);
        if (int rc = sgemm<false, false>(r, r, r, x, r, g, r, t, r, 1.0f, L.s_ns, parts, state, st)) return rc;
        k_polar_combine<<<grid_of(n), NT, 0, st>>>(x, t, n, state);
        if (int rc = sgemm<true, false>(r, r, r, x, r, x, r, g, r, 1.0f, L.s_ns, parts, state, st)) return rc;
        if ((it + 1) % kPolarCheckEvery == 0) {
            int h = 0;
            if (hipMemcpyAsync(&h, state, 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
                hipStreamSynchronize(st) != hipSuccess)
                return hip_status(hipGetLastError());
            if (h >= kStop) break;
        }
    }
    k_polar_end<<<grid_of(n), NT, 0, st>>>(x, rot, n, state, fails);
    return last_launch_status();
}

}  // namespace

size_t itq_workspace_bytes(int64_t D, int64_t r) { return itq_layout(D, r).total; }

int itq_rotate(float *F, int64_t D, int64_t r, int iters, const float *rot0, float *rot_out, double *objective,
               void *ws_, hipStream_t st) {
    const ItqLayout L = itq_layout(D, r);
    uint8_t *ws = (uint8_t *)ws_;
    float *af = (float *)(ws + L.af), *rot = (float *)(ws + L.rot), *x = (float *)(ws + L.x);
    float *parts = (float *)(ws + L.parts);
    int *fails = (int *)(ws + L.fails);
    const size_t rr = (size_t)(r * r) * 4;
    k_zero_int<<<1, 1, 0, st>>>(fails);
    if (rot0) {
        if (hipMemcpyAsync(rot, rot0, rr, hipMemcpyDeviceToDevice, st) != hipSuccess)
            return hip_status(hipGetLastError());
    } else {
        k_eye<<<grid_of(r * r), NT, 0, st>>>(rot, r);
    }
    if (int rc = sgemm<false, false>(D, r, r, F, r, rot, r, af, r, 1.0f, 1, parts, nullptr, st)) return rc;
    if (objective)
        if (int rc = objective_into(af, D * r, objective, ws, L, st)) return rc;
    for (int it = 1; it <= iters; ++it) {
        // Z = F^T sign(F R) into X, R = polar(Z), then A = F R
        if (int rc = sgemm<true, true>(r, r, D, F, r, af, r, x, r, 1.0f, L.s_z, parts, nullptr, st)) return rc;
        if (int rc = polar(r, ws, L, st)) return rc;
        if (int rc = sgemm<false, false>(D, r, r, F, r, rot, r, af, r, 1.0f, 1, parts, nullptr, st)) return rc;
        if (objective)
            if (int rc = objective_into(af, D * r, objective + it, ws, L, st)) return rc;
    }
    if (hipMemcpyAsync(F, af, (size_t)(D * r) * 4, hipMemcpyDeviceToDevice, st) != hipSuccess)
        return hip_status(hipGetLastError());
    if (rot_out && hipMemcpyAsync(rot_out, rot, rr, hipMemcpyDeviceToDevice, st) != hipSuccess)
        return hip_status(hipGetLastError());
    int h = 0;
    if (hipMemcpyAsync(&h, fails, 4, hipMemcpyDeviceToHost, st) != hipSuccess || hipStreamSynchronize(st) != hipSuccess)
        return hip_status(hipGetLastError());
    return h ? LB_EUNSUPPORTED : LB_OK;
}

}  // namespace lb

extern "C" size_t lb_joint_itq_workspace_bytes(int64_t d_out, int64_t d_in, int64_t r_p) {
    if (d_out <= 0 || d_in <= 0 || r_p <= 0) return 0;
    const int64_t D = d_out + d_in;
    return lb::rup256((size_t)(D * r_p) * 4) + lb::itq_workspace_bytes(D, r_p);
}

extern "C" int lb_joint_itq(float *u, float *v, int64_t d_out, int64_t d_in, int64_t r_p, int iters,
                            const float *rot0, float *rot, double *objective, void *ws, size_t ws_bytes,
                            void *stream) {
    using namespace lb;
    if (!u || !v || d_out <= 0 || d_in <= 0 || r_p <= 0 || iters < 0) return LB_EINVAL;
    if (r_p > (d_out < d_in ? d_out : d_in)) return LB_EINVAL;
    const int64_t D = d_out + d_in;
    if (D * r_p >= (1ll << 31) || r_p >= (1 << 15)) return LB_EUNSUPPORTED;
    if (((uintptr_t)u & 3) || ((uintptr_t)v & 3) || ((uintptr_t)rot0 & 3) || ((uintptr_t)rot & 3) ||
        ((uintptr_t)objective & 7))
        return LB_EALIGN;
    if (!ws || ws_bytes < lb_joint_itq_workspace_bytes(d_out, d_in, r_p)) return LB_EWORKSPACE;
    if ((uintptr_t)ws & 255) return LB_EALIGN;
    hipStream_t st = (hipStream_t)stream;
    uint8_t *wsb = (uint8_t *)ws;
    float *F = (float *)wsb;
    const size_t nu = (size_t)(d_out * r_p) * 4, nv = (size_t)(d_in * r_p) * 4;
    if (hipMemcpyAsync(F, u, nu, hipMemcpyDeviceToDevice, st) != hipSuccess ||
        hipMemcpyAsync((uint8_t *)F + nu, v, nv, hipMemcpyDeviceToDevice, st) != hipSuccess)
        return hip_status(hipGetLastError());
    const int rc = itq_rotate(F, D, r_p, iters, rot0, rot, objective, wsb + rup256(nu + nv), st);
    if (rc && rc != LB_EUNSUPPORTED) return rc;
    if (hipMemcpyAsync(u, F, nu, hipMemcpyDeviceToDevice, st) != hipSuccess ||
        hipMemcpyAsync(v, (uint8_t *)F + nu, nv, hipMemcpyDeviceToDevice, st) != hipSuccess)
        return hip_status(hipGetLastError());
    return rc;
}
