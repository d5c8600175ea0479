/*
 * lb_oracle.c -- plain fp64 CPU oracle of the LittleBit linear layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  It shares no
 * code, header, table or constant with the HIP library: every definition here
 * is written from the pages' description of the layer.
 *
 * What the layer computes (sesamedisk page, "What the method actually
 * computes", Proposition 1): for an input row x,
 *     y = h * ( sign(U) . ( l * ( sign(V)^T . ( g * x ) ) ) )
 * where sign(U) is d_out x r and sign(V) is d_in x r with +-1 entries, and
 * h (d_out), g (d_in), l (r) are FP16 scale vectors (same page, "How
 * low-rank binarization works").  A second "residual" binarised path of the
 * same form is added when enabled (same page, Dual-SVID paragraph; littlebitllm
 * page, "Pipeline" step 04).  Both binary products are plain matrix products
 * with floating-point accumulation (sesamedisk, the note after Proposition 1).
 *
 * Everything is evaluated in fp64 with sums in plain index order.  Nothing is
 * blocked, fused or reordered.  Threads (OpenMP) only split independent output
 * elements; each output element is one sequential loop, so the result does
 * not depend on the thread count.
 *
 * Readings taken where the pages are silent (each listed in the design notes):
 *  - sign(v) is -1 exactly when v < 0, else +1 (so sign(+-0) = sign(NaN) = +1);
 *  - packed bit b of word w along the packed axis stands for element 32*w + b,
 *    bit value 1 means -1; tail and padding bits are 0;
 *  - the residual path has its own h, g and l;
 *  - rank r = floor(b * d_in * d_out / (d_in + d_out)) rounded down to a
 *    multiple of 32; with the residual each path gets r / 2;
 *  - the SwiGLU block is y = down( silu(gate(x)) * up(x) ),
 *    silu(z) = z / (1 + exp(-z)).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* rank from the bit budget                                                  */
/* ------------------------------------------------------------------------ */

/* The budget counts only factor bits (littlebitllm page, "How small": scale
 * vectors are not counted).  One path of rank r stores r*(d_in + d_out) sign
 * bits against d_in*d_out weights, so the largest r within b bits per weight is
 * floor(b*d_in*d_out/(d_in+d_out)) (sesamedisk, "How low-rank binarization
 * works": the rank sets the bit budget).  The residual path fits inside the
 * same budget (same page and section), so the two paths split r.  Exact
 * integer arithmetic: b = b_num / b_den.
 * Returns 0 on success, -1 if the rank rounds to zero or inputs are bad. */
int oracle_rank_for_budget(int64_t d_in, int64_t d_out, int64_t b_num, int64_t b_den,
                           int residual, int64_t *r_total, int64_t *r_path)
{
    if (d_in <= 0 || d_out <= 0 || b_num <= 0 || b_den <= 0) return -1;
    /* numerator and denominator of b*d_in*d_out/(d_in+d_out) */
    __int128 num = (__int128)b_num * d_in * d_out;
    __int128 den = (__int128)b_den * (d_in + d_out);
    int64_t r = (int64_t)(num / den);   /* floor: both positive */
    r = (r / 32) * 32;
    if (r <= 0) return -1;
    *r_total = r;
    *r_path = residual ? r / 2 : r;
    return 0;
}

/* ------------------------------------------------------------------------ */
/* sign packing                                                              */
/* ------------------------------------------------------------------------ */

static int is_negative(float v) { return v < 0.0f; }

/* Pack the signs of a row-major float matrix src[rows][cols].
 * axis 0: words run down the rows; dst is [ceil(rows/32)][ld], word (w, c)
 *         holds src[32w + b][c] in bit b.
 * axis 1: words run along the columns; dst is [ceil(cols/32)][ld], word (w, r)
 *         holds src[r][32w + b] in bit b.
 * ld >= the length of the other axis; words beyond it and bits beyond the end
 * of the packed axis are 0. */
void oracle_pack_signs(const float *src, int64_t rows, int64_t cols, int axis,
                       uint32_t *dst, int64_t ld)
{
    int64_t n_pack = axis == 0 ? rows : cols;   /* length of the packed axis */
    int64_t n_other = axis == 0 ? cols : rows;
    int64_t planes = (n_pack + 31) / 32;
    for (int64_t w = 0; w < planes; ++w) {
        for (int64_t o = 0; o < ld; ++o) {
            uint32_t word = 0;
            if (o < n_other) {
                for (int b = 0; b < 32; ++b) {
                    int64_t e = 32 * w + b;
                    if (e >= n_pack) break;
                    float v = axis == 0 ? src[e * cols + o] : src[o * cols + e];
                    if (is_negative(v)) word |= (uint32_t)1 << b;
                }
            }
            dst[w * ld + o] = word;
        }
    }
}

/* Inverse of the above for testing: +1/-1 doubles, dst[rows][cols]. */
void oracle_unpack_signs(const uint32_t *src, int64_t rows, int64_t cols, int axis,
                         int64_t ld, double *dst)
{
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < cols; ++j) {
            int64_t e = axis == 0 ? i : j;      /* index along the packed axis */
            int64_t o = axis == 0 ? j : i;
            uint32_t word = src[(e / 32) * ld + o];
            dst[i * cols + j] = ((word >> (e % 32)) & 1u) ? -1.0 : 1.0;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* factorised forward                                                        */
/* ------------------------------------------------------------------------ */

static double sgn(float v) { return is_negative(v) ? -1.0 : 1.0; }

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* One path of Proposition 1, added into y.
 *   x [T][d_in], U [d_out][r], V [d_in][r] (float factors; only signs used),
 *   h [d_out], g [d_in], l [r] (fp64), y [T][d_out] accumulated. */
static void path_forward(const double *x, int64_t T, int64_t d_in, int64_t d_out, int64_t r,
                         const float *U, const float *V,
                         const double *h, const double *g, const double *l, double *y)
{
    double *t = (double *)calloc((size_t)(T * r), sizeof(double));
    /* a = g * x ; u_k = sum_i sign(V[i][k]) * a_i ; t_k = l_k * u_k */
    #pragma omp parallel for schedule(static)
    for (int64_t nk = 0; nk < T * r; ++nk) {
        int64_t n = nk / r, k = nk % r;
        double u = 0.0;
        for (int64_t i = 0; i < d_in; ++i)
            u += sgn(V[i * r + k]) * (g[i] * x[n * d_in + i]);
        t[n * r + k] = l[k] * u;
    }
    /* z_j = sum_k sign(U[j][k]) * t_k ; y_j += h_j * z_j */
    #pragma omp parallel for schedule(static)
    for (int64_t nj = 0; nj < T * d_out; ++nj) {
        int64_t n = nj / d_out, j = nj % d_out;
        double z = 0.0;
        for (int64_t k = 0; k < r; ++k)
            z += sgn(U[j * r + k]) * t[n * r + k];
        y[n * d_out + j] += h[j] * z;
    }
    free(t);
}

/* y = sum over paths p of the layer of Proposition 1.
 *   U [P][d_out][r_p], V [P][d_in][r_p], h [P][d_out], g [P][d_in], l [P][r_p]. */
void oracle_linear_forward(const double *x, int64_t T, int64_t d_in, int64_t d_out,
                           int64_t r_p, int P, const float *U, const float *V,
                           const double *h, const double *g, const double *l,
                           double *y, int nthreads)
{
    set_threads(nthreads);
    memset(y, 0, sizeof(double) * (size_t)(T * d_out));
    for (int p = 0; p < P; ++p)
        path_forward(x, T, d_in, d_out, r_p,
                     U + (size_t)p * d_out * r_p, V + (size_t)p * d_in * r_p,
                     h + (size_t)p * d_out, g + (size_t)p * d_in, l + (size_t)p * r_p, y);
}

/* The same layer for a bounded subset of output rows: y[T][n_rows] gets rows
 * rows[0..n_rows) of the full output.  Used to check very large layers on a
 * sample of outputs; the latent t is still computed in full. */
void oracle_linear_forward_rows(const double *x, int64_t T, int64_t d_in, int64_t d_out,
                                int64_t r_p, int P, const float *U, const float *V,
                                const double *h, const double *g, const double *l,
                                const int64_t *rows, int64_t n_rows, double *y, int nthreads)
{
    set_threads(nthreads);
    memset(y, 0, sizeof(double) * (size_t)(T * n_rows));
    double *t = (double *)calloc((size_t)(T * r_p), sizeof(double));
    for (int p = 0; p < P; ++p) {
        const float *Up = U + (size_t)p * d_out * r_p, *Vp = V + (size_t)p * d_in * r_p;
        const double *hp = h + (size_t)p * d_out, *gp = g + (size_t)p * d_in, *lp = l + (size_t)p * r_p;
        #pragma omp parallel for schedule(static)
        for (int64_t nk = 0; nk < T * r_p; ++nk) {
            int64_t n = nk / r_p, k = nk % r_p;
            double u = 0.0;
            for (int64_t i = 0; i < d_in; ++i)
                u += sgn(Vp[i * r_p + k]) * (gp[i] * x[n * d_in + i]);
            t[n * r_p + k] = lp[k] * u;
        }
        #pragma omp parallel for schedule(static)
        for (int64_t nq = 0; nq < T * n_rows; ++nq) {
            int64_t n = nq / n_rows, q = nq % n_rows, j = rows[q];
            double z = 0.0;
            for (int64_t k = 0; k < r_p; ++k)
                z += sgn(Up[j * r_p + k]) * t[n * r_p + k];
            y[n * n_rows + q] += hp[j] * z;
        }
    }
    free(t);
}

/* The two halves of the layer around the rank-r intermediate, which the
 * sesamedisk page ("The real result") names as what a k/v projection can
 * cache instead of its d_out-wide output.
 * Latents: t [T][P*r_p], path p in columns p*r_p .. p*r_p + r_p - 1,
 *   t[n][p*r_p + k] = l_p[k] * sum_i sign(V_p[i][k]) * (g_p[i] * x[n][i]),
 * the same loop as the first half of path_forward. */
void oracle_linear_latents(const double *x, int64_t T, int64_t d_in, int64_t r_p, int P,
                           const float *V, const double *g, const double *l, double *t, int nthreads)
{
    set_threads(nthreads);
    int64_t R = (int64_t)P * r_p;
    for (int p = 0; p < P; ++p) {
        const float *Vp = V + (size_t)p * d_in * r_p;
        const double *gp = g + (size_t)p * d_in, *lp = l + (size_t)p * r_p;
        #pragma omp parallel for schedule(static)
        for (int64_t nk = 0; nk < T * r_p; ++nk) {
            int64_t n = nk / r_p, k = nk % r_p;
            double u = 0.0;
            for (int64_t i = 0; i < d_in; ++i)
                u += sgn(Vp[i * r_p + k]) * (gp[i] * x[n * d_in + i]);
            t[n * R + (int64_t)p * r_p + k] = lp[k] * u;
        }
    }
}

/* Output from given latents t [T][P*r_p] (layout as above):
 *   y[n][j] = sum_p h_p[j] * sum_k sign(U_p[j][k]) * t[n][p*r_p + k],
 * the paths added in order, as path_forward adds them. */
void oracle_linear_from_latents(const double *t, int64_t T, int64_t d_out, int64_t r_p, int P,
                                const float *U, const double *h, double *y, int nthreads)
{
    set_threads(nthreads);
    int64_t R = (int64_t)P * r_p;
    memset(y, 0, sizeof(double) * (size_t)(T * d_out));
    for (int p = 0; p < P; ++p) {
        const float *Up = U + (size_t)p * d_out * r_p;
        const double *hp = h + (size_t)p * d_out;
        #pragma omp parallel for schedule(static)
        for (int64_t nj = 0; nj < T * d_out; ++nj) {
            int64_t n = nj / d_out, j = nj % d_out;
            double z = 0.0;
            for (int64_t k = 0; k < r_p; ++k)
                z += sgn(Up[j * r_p + k]) * t[n * R + (int64_t)p * r_p + k];
            y[n * d_out + j] += hp[j] * z;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* SwiGLU block                                                              */
/* ------------------------------------------------------------------------ */

/* silu(z) = z / (1 + exp(-z)); for z below about -709 exp overflows to +inf
 * and the quotient is -0, so no NaN arises for finite z. */
double oracle_silu(double z) { return z / (1.0 + exp(-z)); }

/* y = down( silu(gate(x)) * up(x) ): gate and up map d_model -> d_ff with
 * per-path rank r_gu_p, down maps d_ff -> d_model with per-path rank r_dn_p. */
void oracle_mlp_forward(const double *x, int64_t T, int64_t d_model, int64_t d_ff, int P,
                        int64_t r_gu_p, int64_t r_dn_p,
                        const float *Ug, const float *Vg, const double *hg, const double *gg, const double *lg,
                        const float *Uu, const float *Vu, const double *hu, const double *gu, const double *lu,
                        const float *Ud, const float *Vd, const double *hd, const double *gd, const double *ld,
                        double *y, int nthreads)
{
    double *zg = (double *)malloc(sizeof(double) * (size_t)(T * d_ff));
    double *zu = (double *)malloc(sizeof(double) * (size_t)(T * d_ff));
    oracle_linear_forward(x, T, d_model, d_ff, r_gu_p, P, Ug, Vg, hg, gg, lg, zg, nthreads);
    oracle_linear_forward(x, T, d_model, d_ff, r_gu_p, P, Uu, Vu, hu, gu, lu, zu, nthreads);
    for (int64_t e = 0; e < T * d_ff; ++e) zg[e] = oracle_silu(zg[e]) * zu[e];
    oracle_linear_forward(zg, T, d_ff, d_model, r_dn_p, P, Ud, Vd, hd, gd, ld, y, nthreads);
    free(zg);
    free(zu);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
