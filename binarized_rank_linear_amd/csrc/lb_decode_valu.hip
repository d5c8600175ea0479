// lb_decode_valu.hip -- plain vector-ALU decode path of the LittleBit forward.
//
// Proposition 1 (sesamedisk page, "What the method actually computes") as two
// binary matrix-vector products with fp32 accumulation; each +-1 is applied as
// a flip of the fp32 sign bit (the page's note that a +-1 multiply is a sign
// flip).  This path favours clarity over speed: it is the cross-check for the
// matrix-core decode kernels and serves any token count in chunks of <= 32.
//
//   stage 1: part[z][n][p*r_p + k] = sum_{i in chunk z} sign(V_p[i][k]) g_p[i] x[n][i]
//   stage 2: y[n][j] = sum_p h_p[j] sum_k sign(U_p[j][k]) (l_p[k] sum_z part[z][n][p*r_p+k])
// for the tokens n of one launch pair (at most 32); the pairs run one after
// the other on the stream and reuse part, so the workspace does not grow
// with the token count.
//
// One thread per latent row (stage 1) or output row (stage 2); the packed
// word planes make the 64 lanes of a wave read 256 consecutive bytes.
#include "lb_internal.h"

namespace lb {

namespace {

constexpr int kBlock = 256;     // threads per block = rows per block
constexpr int kSpan = 256;      // activations staged per round (8 words)

struct ValuPlan {
    int nt;          // tokens per launch (template width)
    int nsplit;      // K-chunks of stage 1
    int64_t kchunk;  // elements of d_in per chunk (multiple of kSpan)
};

ValuPlan plan_valu(const Linear &a) {
    ValuPlan pl;
    pl.nt = a.T >= 32 ? 32 : a.T > 16 ? 32 : a.T > 8 ? 16 : a.T > 4 ? 8 : a.T > 2 ? 4 : a.T > 1 ? 2 : 1;
    const int64_t spans = cdiv(a.d_in, kSpan);
    const int64_t blocks1 = cdiv(a.r_p, kBlock) * a.P;
    int64_t ns = 1024 / (blocks1 > 0 ? blocks1 : 1);
    if (ns < 1) ns = 1;
    if (ns > spans) ns = spans;
    if (ns > 256) ns = 256;
    const int64_t spans_per = cdiv(spans, ns);
    pl.kchunk = spans_per * kSpan;
    pl.nsplit = (int)cdiv(a.d_in, pl.kchunk);
    return pl;
}

template <int NT>
__global__ __launch_bounds__(kBlock) void k_s1_valu(Linear a, int64_t n0, int ntok,
                                                    int64_t kchunk, float *__restrict__ part) {
    __shared__ float sa[NT][kSpan];
    const int p = blockIdx.y;
    const int64_t k = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t i_begin = (int64_t)blockIdx.z * kchunk;
    const int64_t i_end = imin(a.d_in, i_begin + kchunk);
    const uint32_t *vb = a.v_bits + (int64_t)p * a.kw_v() * a.ld_v;
    const uint16_t *g = a.g + (int64_t)p * a.d_in;
    float acc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[n] = 0.0f;

    for (int64_t i0 = i_begin; i0 < i_end; i0 += kSpan) {
        __syncthreads();
        for (int e = threadIdx.x; e < NT * kSpan; e += kBlock) {
            const int n = e / kSpan, ii = e % kSpan;
            const int64_t i = i0 + ii;
            float v = 0.0f;
            if (n < ntok && i < i_end)
                v = f16_to_f32(g[i]) * load_act(a.x, a.x_dtype, (n0 + n) * a.d_in + i);
            sa[n][ii] = v;
        }
        __syncthreads();
        if (k < a.r_p) {
            const int nw = (int)imin(kSpan / 32, cdiv(i_end - i0, 32));
            for (int ww = 0; ww < nw; ++ww) {
                const uint32_t word = vb[(i0 / 32 + ww) * a.ld_v + k];
                for (int b = 0; b < 32; ++b) {
                    const uint32_t s = (word << (31 - b)) & 0x80000000u;
#pragma unroll
                    for (int n = 0; n < NT; ++n) acc[n] += flip(sa[n][ww * 32 + b], s);
                }
            }
        }
    }
    if (k < a.r_p) {
        const int64_t R = a.P * a.r_p;
        for (int n = 0; n < ntok; ++n)
            part[((int64_t)blockIdx.z * NT + n) * R + p * a.r_p + k] = acc[n];
    }
}

// The latents of one launch pair's tokens, t [T][P*r_p] (t_dtype), summed as
// k_s2_valu sums them: l * (sum of the pieces in order).  One thread per
// (token, latent).
template <int NT>
__global__ __launch_bounds__(kBlock) void k_t_valu(Linear a, int64_t n0, int ntok, int nsplit,
                                                   const float *__restrict__ part, void *t, int t_dtype) {
    const int64_t R = a.P * a.r_p;
    const int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (e >= ntok * R) return;
    const int n = (int)(e / R);
    const int64_t pk = e - n * R;
    const int p = (int)(pk / a.r_p);
    const int64_t kx = pk - (int64_t)p * a.r_p;
    float s = 0.0f;
    for (int z = 0; z < nsplit; ++z) s += part[((int64_t)z * NT + n) * R + pk];
    const float v = f16_to_f32(a.l[p * a.r_p + kx]) * s;
    const int64_t o = (n0 + n) * R + pk;
    if (t_dtype == LB_F32) ((float *)t)[o] = v;
    else ((uint16_t *)t)[o] = f32_to_bf16(v);
}

// t_in (null: the latents come from part): the latents t [T][P*r_p] given.
template <int NT>
__global__ __launch_bounds__(kBlock) void k_s2_valu(Linear a, int64_t n0, int ntok, int nsplit,
                                                    const float *__restrict__ part, const void *t_in,
                                                    int t_dtype) {
    __shared__ float st[NT][kSpan];
    const int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    const int64_t R = a.P * a.r_p;
    float yacc[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) yacc[n] = 0.0f;

    for (int p = 0; p < a.P; ++p) {
        const uint32_t *ub = a.u_bits + (int64_t)p * a.kw_u() * a.ld_u;
        float acc[NT];
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[n] = 0.0f;
        for (int64_t k0 = 0; k0 < a.r_p; k0 += kSpan) {
            __syncthreads();
            for (int e = threadIdx.x; e < NT * kSpan; e += kBlock) {
                const int n = e / kSpan, kk = e % kSpan;
                const int64_t kx = k0 + kk;
                float v = 0.0f;
                if (n < ntok && kx < a.r_p) {
                    if (t_in) {
                        const int64_t o = (n0 + n) * R + p * a.r_p + kx;
                        v = t_dtype == LB_F32 ? ((const float *)t_in)[o]
                                              : bf16_to_f32(((const uint16_t *)t_in)[o]);
                    } else {
                        float s = 0.0f;
                        for (int z = 0; z < nsplit; ++z)
                            s += part[((int64_t)z * NT + n) * R + p * a.r_p + kx];
                        v = f16_to_f32(a.l[p * a.r_p + kx]) * s;
                    }
                }
                st[n][kk] = v;
            }
            __syncthreads();
            if (j < a.d_out) {
                const int nw = (int)imin(kSpan / 32, cdiv(a.r_p - k0, 32));
                for (int ww = 0; ww < nw; ++ww) {
                    const uint32_t word = ub[(k0 / 32 + ww) * a.ld_u + j];
                    for (int b = 0; b < 32; ++b) {
                        const uint32_t s = (word << (31 - b)) & 0x80000000u;
#pragma unroll
                        for (int n = 0; n < NT; ++n) acc[n] += flip(st[n][ww * 32 + b], s);
                    }
                }
            }
        }
        if (j < a.d_out) {
            const float hv = f16_to_f32(a.h[p * a.d_out + j]);
#pragma unroll
            for (int n = 0; n < NT; ++n) yacc[n] += hv * acc[n];
        }
    }
    if (j < a.d_out)
        for (int n = 0; n < ntok; ++n) store_act(a.y, a.y_dtype, (n0 + n) * a.d_out + j, yacc[n]);
}

// stage: 3 = the whole layer; 1 = the latents to t; 2 = the output from t.
template <int NT>
int run_valu(const Linear &a, const ValuPlan &pl, float *part, hipStream_t s, int stage = 3,
             void *t = nullptr, int t_dtype = LB_F32) {
    for (int64_t n0 = 0; n0 < a.T; n0 += NT) {
        const int ntok = (int)imin(NT, a.T - n0);
        if (stage & 1) {
            dim3 g1((unsigned)cdiv(a.r_p, kBlock), (unsigned)a.P, (unsigned)pl.nsplit);
            k_s1_valu<NT><<<g1, kBlock, 0, s>>>(a, n0, ntok, pl.kchunk, part);
            if (int rc = last_launch_status()) return rc;
        }
        if (stage == 1) {
            k_t_valu<NT><<<(unsigned)cdiv(ntok * a.P * a.r_p, kBlock), kBlock, 0, s>>>(a, n0, ntok, pl.nsplit,
                                                                                   part, t, t_dtype);
            if (int rc = last_launch_status()) return rc;
        }
        if (stage & 2) {
            dim3 g2((unsigned)cdiv(a.d_out, kBlock));
            k_s2_valu<NT><<<g2, kBlock, 0, s>>>(a, n0, ntok, pl.nsplit, part, stage == 2 ? t : nullptr, t_dtype);
            if (int rc = last_launch_status()) return rc;
        }
    }
    return LB_OK;
}

}  // namespace

size_t valu_workspace_bytes(const Linear &a) {
    const ValuPlan pl = plan_valu(a);
    return (size_t)pl.nsplit * (size_t)pl.nt * (size_t)(a.P * a.r_p) * sizeof(float);
}

int valu_forward(const Linear &a, void *ws, hipStream_t s) {
    const ValuPlan pl = plan_valu(a);
    float *part = (float *)ws;
    switch (pl.nt) {
        case 1: return run_valu<1>(a, pl, part, s);
        case 2: return run_valu<2>(a, pl, part, s);
        case 4: return run_valu<4>(a, pl, part, s);
        case 8: return run_valu<8>(a, pl, part, s);
        case 16: return run_valu<16>(a, pl, part, s);
        default: return run_valu<32>(a, pl, part, s);
    }
}

int valu_stage_forward(const Linear &a, void *ws, int stage, void *t, int t_dtype, hipStream_t s) {
    const ValuPlan pl = plan_valu(a);
    float *part = (float *)ws;
    switch (pl.nt) {
        case 1: return run_valu<1>(a, pl, part, s, stage, t, t_dtype);
        case 2: return run_valu<2>(a, pl, part, s, stage, t, t_dtype);
        case 4: return run_valu<4>(a, pl, part, s, stage, t, t_dtype);
        case 8: return run_valu<8>(a, pl, part, s, stage, t, t_dtype);
        case 16: return run_valu<16>(a, pl, part, s, stage, t, t_dtype);
        default: return run_valu<32>(a, pl, part, s, stage, t, t_dtype);
    }
}

}  // namespace lb
