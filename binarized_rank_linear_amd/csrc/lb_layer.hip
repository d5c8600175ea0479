// lb_layer.hip -- lb_decoder_layer_forward: one decoder layer of a LittleBit
// model at decode time, its seven linears replaced by LittleBit linears (the
// architecture is otherwise unchanged: littlebitllm page, hero; deniz.in,
// "Factorize first, then binarize"), minus attention over a KV cache:
//
//   a  = x / rms(x)                          RMSNorm (its weight folded into g)
//   q, k, v = Q(a), K(a), V(a)               one group, one staged input
//   o_in = v, each kv head serving its group of query heads
//                                            (attention over one token: the
//                                            softmax of a single score is 1)
//   x1 = x + O(o_in)                         residual added in O's epilogue
//   b  = x1 / rms(x1)
//   y  = x1 + Down(silu(Gate(b)) * Up(b))    gate and up one group; the SwiGLU
//                                            computed in Down's input staging
//
// The RMSNorms' 1/rms(x) is a per-token scale of the next linears' input,
// applied where their stage 1 stages it.
#include <math.h>

#include "lb_internal.h"

namespace lb {
namespace {

constexpr int kT = 256;

// inv[n] = 1 / sqrt(mean(x[n]^2) + eps), bf16 x [T][d]: workgroup n < T sums
// token n's squares (16-byte loads, all in flight, when rows are 16-byte
// aligned), the waves by shuffles, then across the waves in LDS.  Workgroups
// from T on clear `zn` 32-bit words at `zero` (a run's scratch) meanwhile.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__global__ __launch_bounds__(kT) void k_rms(const uint16_t *__restrict__ x, int64_t T, int64_t d, float eps,
                                            float *__restrict__ inv, uint32_t *__restrict__ zero, int64_t zn) {
    const int64_t b = blockIdx.x;
    if (b >= T) {                                             // the clearing workgroups
        const int64_t nz = (int64_t)gridDim.x - T;
        for (int64_t i = (b - T) * kT + threadIdx.x; i < zn; i += nz * kT) zero[i] = 0u;
        return;
    }
    const uint16_t *xr = x + b * d;
    float s = 0.0f;
    if ((d & 7) == 0 && ((uintptr_t)x & 15) == 0) {
        const uint4 *xv = (const uint4 *)xr;
        const int64_t nv = d >> 3;
        for (int64_t i0 = 0; i0 < nv; i0 += 4 * kT) {
            uint4 q[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t i = i0 + k * kT + threadIdx.x;
                q[k] = i < nv ? xv[i] : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t w[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float lo = __uint_as_float(w[j] << 16), hi = __uint_as_float(w[j] & 0xffff0000u);
                    s += lo * lo + hi * hi;
                }
            }
        }
    } else {
        for (int64_t i = threadIdx.x; i < d; i += kT) {
            const float v = bf16_to_f32(xr[i]);
            s += v * v;
        }
    }
    __shared__ float red[kT / 64];
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int w = 0; w < kT / 64; ++w) t += red[w];
        inv[b] = 1.0f / sqrtf(t / (float)d + eps);
    }
}

// o_in[n][h*dh + e] = v[n][(h / grp)*dh + e]: each kv head serves grp query heads.
__global__ __launch_bounds__(kT) void k_expand_heads(const uint16_t *__restrict__ v, uint16_t *__restrict__ o,
                                                     int64_t T, int64_t d_model, int64_t d_kv, int64_t dh,
                                                     int64_t grp) {
    const int64_t e = (int64_t)blockIdx.x * kT + threadIdx.x;
    if (e >= T * d_model) return;
    const int64_t n = e / d_model, c = e - n * d_model;
    const int64_t h = c / dh;
    o[e] = v[n * d_kv + (h / grp) * dh + (c - h * dh)];
}

size_t rup256(size_t n) { return (n + 255) & ~(size_t)255; }

struct LayerPlan {
    Linear q, k, v, o, gate, up, down;
    size_t off_s, off_q, off_k, off_v, off_oin, off_x1, off_g, off_u;
    size_t off_qkv, off_o, off_gu, off_dn, total;   // the four runs' scratch (cleared together)
};

int check_factors_of(const lb_factors *w, Linear *a) {
    if (!w->v_bits || !w->u_bits || !w->g || !w->l || !w->h) return LB_EINVAL;
    if (w->ld_v < a->r_p || w->ld_u < a->d_out) return LB_EINVAL;
    if (w->ld_v % 4 || w->ld_u % 4) return LB_EALIGN;
    if (((uintptr_t)w->v_bits | (uintptr_t)w->u_bits) & 15) return LB_EALIGN;
    a->v_bits = w->v_bits;
    a->u_bits = w->u_bits;
    a->g = w->g;
    a->l = w->l;
    a->h = w->h;
    a->ld_v = w->ld_v;
    a->ld_u = w->ld_u;
    return LB_OK;
}

int shape_of(int64_t d_in, int64_t d_out, int64_t r, int P, int64_t T, const lb_factors *w, Linear *a) {
    if (d_in <= 0 || d_out <= 0 || r <= 0 || r % P) return LB_EINVAL;
    *a = Linear{};
    a->d_in = d_in;
    a->d_out = d_out;
    a->r_p = r / P;
    a->P = P;
    a->T = T;
    a->x_dtype = a->y_dtype = LB_BF16;
    return w ? check_factors_of(w, a) : LB_OK;
}

// Sizes, factors and the workspace layout of a layer at T tokens.
int plan_layer(const lb_decoder_layer *L, int64_t T, bool with_factors, LayerPlan *p) {
    if (!L || T < 1) return LB_EINVAL;
    if (T > 32) return LB_EUNSUPPORTED;
    if (L->d_model <= 0 || L->d_ff <= 0 || L->n_heads <= 0 || L->n_kv_heads <= 0) return LB_EINVAL;
    if (L->d_model % L->n_heads || L->n_heads % L->n_kv_heads || !(L->eps >= 0.0f)) return LB_EINVAL;
    const int P = L->residual ? 2 : 1;
    const int64_t dkv = L->d_model / L->n_heads * L->n_kv_heads;
    int rc;
    if ((rc = shape_of(L->d_model, L->d_model, L->r_qo, P, T, with_factors ? &L->q : nullptr, &p->q)) ||
        (rc = shape_of(L->d_model, dkv, L->r_kv, P, T, with_factors ? &L->k : nullptr, &p->k)) ||
        (rc = shape_of(L->d_model, dkv, L->r_kv, P, T, with_factors ? &L->v : nullptr, &p->v)) ||
        (rc = shape_of(L->d_model, L->d_model, L->r_qo, P, T, with_factors ? &L->o : nullptr, &p->o)) ||
        (rc = shape_of(L->d_model, L->d_ff, L->r_gu, P, T, with_factors ? &L->gate : nullptr, &p->gate)) ||
        (rc = shape_of(L->d_model, L->d_ff, L->r_gu, P, T, with_factors ? &L->up : nullptr, &p->up)) ||
        (rc = shape_of(L->d_ff, L->d_model, L->r_down, P, T, with_factors ? &L->down : nullptr, &p->down)))
        return rc;
    const Linear *all[7] = {&p->q, &p->k, &p->v, &p->o, &p->gate, &p->up, &p->down};
    for (const Linear *a : all)
        if (!mfma_decode_supported(T, LB_BF16) || !mfma_decode_shape_ok(*a)) return LB_EUNSUPPORTED;
    size_t at = 0;
    auto take = [&](size_t b) { const size_t o = at; at += rup256(b); return o; };
    p->off_s = take((size_t)T * 4);
    p->off_q = take((size_t)(T * L->d_model) * 2);
    p->off_k = take((size_t)(T * dkv) * 2);
    p->off_v = take((size_t)(T * dkv) * 2);
    p->off_oin = take((size_t)(T * L->d_model) * 2);
    p->off_x1 = take((size_t)(T * L->d_model) * 2);
    p->off_g = take((size_t)(T * L->d_ff) * 2);
    p->off_u = take((size_t)(T * L->d_ff) * 2);
    const Linear qkv[3] = {p->q, p->k, p->v}, gu[2] = {p->gate, p->up};
    p->off_qkv = take(mfma_inline_workspace_bytes(qkv, 3));
    p->off_o = take(mfma_inline_workspace_bytes(&p->o, 1));
    p->off_gu = take(mfma_inline_workspace_bytes(gu, 2));
    p->off_dn = take(mfma_inline_workspace_bytes(&p->down, 1));
    p->total = at;
    return LB_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a && b && na && nb && a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace
}  // namespace lb

extern "C" size_t lb_decoder_layer_workspace_bytes(const lb_decoder_layer *L, int64_t T) {
    lb::LayerPlan p;
    return lb::plan_layer(L, T, false, &p) ? 0 : p.total;
}

extern "C" int lb_decoder_layer_forward(const lb_decoder_layer *L, const void *x, void *y, int64_t T, void *ws,
                                        size_t ws_bytes, void *stream) {
    using namespace lb;
    LayerPlan p;
    int rc;
    if (T < 0) return LB_EINVAL;
    if ((rc = plan_layer(L, T ? T : 1, true, &p))) return rc;
    if (T == 0) return LB_OK;
    if (!x || !y || ((uintptr_t)x & 15) || ((uintptr_t)y & 15)) return x && y ? LB_EALIGN : LB_EINVAL;
    const size_t xb = (size_t)(T * L->d_model) * 2;
    if (overlaps(x, xb, y, xb)) return LB_EINVAL;
    if (!ws || ws_bytes < p.total) return LB_EWORKSPACE;
    if ((uintptr_t)ws & 255) return LB_EALIGN;
    if (overlaps(ws, p.total, x, xb) || overlaps(ws, p.total, y, xb)) return LB_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    uint8_t *w = (uint8_t *)ws;
    float *inv = (float *)(w + p.off_s);
    uint16_t *q = (uint16_t *)(w + p.off_q), *k = (uint16_t *)(w + p.off_k), *v = (uint16_t *)(w + p.off_v);
    uint16_t *oin = (uint16_t *)(w + p.off_oin), *x1 = (uint16_t *)(w + p.off_x1);
    uint16_t *yg = (uint16_t *)(w + p.off_g), *yu = (uint16_t *)(w + p.off_u);
    const int64_t dh = L->d_model / L->n_heads, dkv = dh * L->n_kv_heads;
    // a = x / rms(x); the same launch clears the four runs' scratch (their
    // one-launch forms start from zero); q, k, v
    const int64_t zn = (int64_t)(p.total - p.off_qkv) / 4;
    k_rms<<<(unsigned)(T + imin(512, cdiv(zn, kT))), kT, 0, s>>>((const uint16_t *)x, T, L->d_model, L->eps, inv,
                                                                 (uint32_t *)(w + p.off_qkv), zn);
    if ((rc = last_launch_status())) return rc;
    p.q.x = p.k.x = p.v.x = x;
    p.q.xs = p.k.xs = p.v.xs = inv;
    p.q.y = q;
    p.k.y = k;
    p.v.y = v;
    const Linear qkv[3] = {p.q, p.k, p.v};
    if ((rc = mfma_inline_forward(qkv, 3, w + p.off_qkv, s, true))) return rc;
    // attention over one token, then x1 = x + O(o_in): without kv grouping
    // o_in is v; with it, the fused stage 1 of o reads v through the head map,
    // else the heads are expanded into o_in first
    const int64_t grp = L->n_heads / L->n_kv_heads;
    if (grp == 1) {
        p.o.x = v;
    } else if (mfma_fused_stage1(T, LB_BF16)) {
        p.o.x = v;
        p.o.xm_dh = (int32_t)dh;
        p.o.xm_grp = (int32_t)grp;
    } else {
        k_expand_heads<<<(unsigned)cdiv(T * L->d_model, kT), kT, 0, s>>>(v, oin, T, L->d_model, dkv, dh, grp);
        if ((rc = last_launch_status())) return rc;
        p.o.x = oin;
    }
    p.o.resid = x;
    p.o.y = x1;
    if ((rc = mfma_inline_forward(&p.o, 1, w + p.off_o, s, true))) return rc;
    // b = x1 / rms(x1); gate, up; y = x1 + Down(silu(gate) * up)
    k_rms<<<(unsigned)T, kT, 0, s>>>(x1, T, L->d_model, L->eps, inv, nullptr, 0);
    if ((rc = last_launch_status())) return rc;
    p.gate.x = p.up.x = x1;
    p.gate.xs = p.up.xs = inv;
    p.gate.y = yg;
    p.up.y = yu;
    const Linear gu[2] = {p.gate, p.up};
    if ((rc = mfma_inline_forward(gu, 2, w + p.off_gu, s, true))) return rc;
    p.down.x = yg;
    p.down.x2 = yu;
    p.down.resid = x1;
    p.down.y = y;
    return mfma_inline_forward(&p.down, 1, w + p.off_dn, s, true);
}
