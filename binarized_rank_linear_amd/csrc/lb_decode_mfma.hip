// lb_decode_mfma.hip -- matrix-core decode path (T <= 32) of the LittleBit forward.
//
// Proposition 1 (sesamedisk page, "What the method actually computes") is two
// binary contractions with floating-point scaling between them.  Multiplying
// by +-1 is a sign flip (same page, the note after the proposition), so each
// packed bit becomes an fp4 (e2m1) +-1.0 whose sign bit is the packed bit:
//   nibble = ((word << (3 - q)) & 0x88888888) | 0x22222222
// turns bits 4i+q of a word into the sign bits of eight +-1.0 nibbles in two
// VALU operations (a quarter of an operation per weight bit).  The
// activations enter as NL fp8 (e4m3) "limbs" with one power-of-two scale per
// 32-element block, so the block-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4
// (fp4 A x fp8 B, fp32 accumulate) multiplies 16 rows x 128 weight bits by up
// to 16 (token, limb) columns per instruction.  Two limbs keep the relative
// error near 1e-3 (bf16 outputs), three near 2e-5 (fp32 outputs).
//
// Data layout: packed planes (littlebit.h) put word (w, row) at w*ld + row, so
// one 16-byte load gives a lane four consecutive rows of one plane and a wave
// covers 64 rows x 4 planes (four 16-row MFMA instances share one B operand).
//
// Two launches per call or per group of linears:
//   stage 1: item = (linear, path, chunk of d_in, group of 256 latents).  The
//            workgroup turns g (.) x for its chunk into fp8 limbs in LDS, streams
//            the V planes and writes partial latent sums.  The last workgroup
//            of each (linear, path, latent group) -- found with an atomic
//            counter -- adds the chunk partials in chunk order, scales by l and
//            writes the stage-2 B operand (limbs of t) in MFMA lane order.
//   stage 2: item = (linear, block of output rows).  The workgroup copies the
//            B operand of its linear into LDS, streams the U planes of both
//            paths and writes y = sum_p h_p * z_p.
#include "lb_internal.h"

namespace lb {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;                 // rows per wave tile (4 MFMA instances of 16)
constexpr int kRG = kWaves * kTile;       // stage-1 latent rows per workgroup
constexpr int kBop = 64 * 32;             // bytes of one fp8 B operand (64 lanes x 32)
constexpr int kBopS = kBop + 64;          // plus one scale byte per lane
constexpr int kLdsBudget = 64 * 1024;

// Per-linear schedule and workspace pointers (device-resident for groups).
struct MLin {
    const void *x;
    void *y;
    const uint32_t *v_bits, *u_bits;
    const uint16_t *g, *l, *h;
    int64_t ld_v, ld_u, d_in, d_out;
    int32_t r_p, P;
    int32_t kw_v, kw_u;   // planes of V (per path) and of U (per path)
    int32_t kcg;          // K-groups (128 inputs) per stage-1 chunk
    int32_t nchunks;      // stage-1 chunks along d_in
    int32_t nrg;          // 256-latent groups per path
    int32_t kg2;          // stage-2 K-groups per path
    int32_t rows2;        // output rows per stage-2 item
    int32_t n2;           // stage-2 items
    int64_t item1, item2; // first item of this linear in each stage
    float *part;          // [nchunks][T][P*r_p]
    uint8_t *tb;          // [P][kg2][NB] operands of kBopS bytes
    uint32_t *cnt;        // [P][nrg]
};

struct MRun {
    int T, NL, NB, x_dtype, y_dtype;
    int64_t items1, items2;
    const MLin *table;         // null: the single linear passed by value
    const int32_t *lin1;       // item -> linear (stage 1), null for one linear
    const int32_t *lin2;
};

__device__ __forceinline__ float ldexp2(float v, int e) { return __builtin_amdgcn_ldexpf(v, e); }

// fp32 -> OCP e4m3 byte (round to nearest even, in range by construction)
__device__ __forceinline__ uint32_t to_fp8(float v) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xffu;
}
__device__ __forceinline__ float from_fp8(uint32_t b) {
    return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// Byte offset of (element e of a 128-element K-group, column c) inside one B
// operand, and the lane whose scale byte covers it.  The A operand holds bit
// 4i+q of plane word g in MFMA slot s = 8q+i (fp4 lanes carry K = 32g+s); the
// fp8 B operand of the same K sits in lane group (K mod 64)/16 at slot
// (K mod 16) + 16*(K >= 64) (measured layout of the f8f6f4 instruction).
__device__ __forceinline__ int bop_offset(int e, int c) {
    const int g = e >> 5, bit = e & 31;
    const int s = ((bit & 3) << 3) | (bit >> 2);
    const int K = (g << 5) | s;
    const int gp = (K & 63) >> 4;
    const int sp = (K & 15) | ((K >> 6) << 4);
    return ((c + (gp << 4)) << 5) + sp;
}

// The NL limbs of v (element e of a K-group, token n) into an operand set laid
// out [nb][kBopS].  Called by whole waves: each 32-lane half handles one
// 32-element block (one plane word), whose largest magnitude sets the scales
// 2^(E-7-4q).  Lanes with ok == false take part in the reduction with v = 0
// and store nothing.
template <int NL>
__device__ __forceinline__ void emit_limbs(float v, int e, int n, bool ok, uint8_t *ops) {
    constexpr int TPB = 16 / NL;
    float m = fabsf(v);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const int E = (int)((__float_as_uint(m) >> 23) & 0xff) - 127;   // floor(log2 m); m == 0 -> -127
    const int nb = n / TPB;
    const int c0 = (n % TPB) * NL;
    uint8_t *op = ops + nb * kBopS;
    float r = v;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
        const int eq = E - 7 - 4 * q;
        const uint32_t b = to_fp8(ldexp2(r, -eq));
        r -= ldexp2(from_fp8(b), eq);
        if (ok) {
            op[bop_offset(e, c0 + q)] = (uint8_t)b;
            if ((e & 31) == 0) {
                int sc = eq + 127;
                sc = sc < 0 ? 0 : (sc > 254 ? 254 : sc);
                op[kBop + c0 + q + ((e >> 5) << 4)] = (uint8_t)sc;
            }
        }
    }
}

// Zero the fp8 bytes and set scales to 1.0 for `count` operands at ops (LDS).
__device__ __forceinline__ void clear_ops(uint8_t *ops, int count) {
    uint32_t *w = (uint32_t *)ops;
    const int words = count * kBopS / 4;
    for (int i = threadIdx.x; i < words; i += kThreads) {
        const int off = (i * 4) % kBopS;
        w[i] = off >= kBop ? 0x7f7f7f7fu : 0u;
    }
}

// fp4 A operands of one plane word: slot 8q+i <- bit 4i+q, as +-1.0.
__device__ __forceinline__ v8i unpack_word(uint32_t w) {
    v8i a;
    a[0] = (int)(((w << 3) & 0x88888888u) | 0x22222222u);
    a[1] = (int)(((w << 2) & 0x88888888u) | 0x22222222u);
    a[2] = (int)(((w << 1) & 0x88888888u) | 0x22222222u);
    a[3] = (int)((w & 0x88888888u) | 0x22222222u);
    a[4] = a[5] = a[6] = a[7] = 0;
    return a;
}

__device__ __forceinline__ v8i load_bop(const uint8_t *op) {
    const int4 *p = (const int4 *)(op + (threadIdx.x & 63) * 32);
    const int4 lo = p[0], hi = p[1];
    v8i b;
    b[0] = lo.x; b[1] = lo.y; b[2] = lo.z; b[3] = lo.w;
    b[4] = hi.x; b[5] = hi.y; b[6] = hi.z; b[7] = hi.w;
    return b;
}

__device__ __forceinline__ v4f mfma(const v8i &a, const v8i &b, v4f c, int sb) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 0, 0, 127, 0, sb);
}

// Four consecutive rows of one plane (16-byte load), or zeros when out of range.
__device__ __forceinline__ v4u load_rows(const uint32_t *p, bool ok) {
    if (!ok) return v4u{0u, 0u, 0u, 0u};
    return __builtin_nontemporal_load((const v4u *)p);
}

// Sum of the NL limb columns of one token: after this, lanes whose column is
// the token's first limb hold z for 16 rows.
template <int NL>
__device__ __forceinline__ float limb_sum(float v) {
    float s = v + __shfl_down(v, 1, 16);
    if (NL == 3) s += __shfl_down(v, 2, 16);
    return s;
}

// The linear of a work item, as a value: both sources are wave-uniform, so the
// copy stays uniform (matrix instructions ignore the exec mask, so every branch
// around them must be uniform).
__device__ __forceinline__ MLin pick(const MRun &run, const MLin &single, const int32_t *map) {
    MLin m = run.table ? run.table[map[blockIdx.x]] : single;
    static_assert(sizeof(MLin) % 4 == 0, "MLin is copied as 32-bit words");
    int w[sizeof(MLin) / 4];
    __builtin_memcpy(w, &m, sizeof(MLin));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(MLin) / 4); ++i) w[i] = __builtin_amdgcn_readfirstlane(w[i]);
    __builtin_memcpy(&m, w, sizeof(MLin));
    return m;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// stage 1
// ---------------------------------------------------------------------------

template <int NL, int NB>
__global__ __launch_bounds__(kThreads) void k_stage1(MRun run, MLin single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ int s_last;
    const MLin L = pick(run, single, run.lin1);
    const int64_t local = (int64_t)blockIdx.x - L.item1;
    const int rg = (int)(local % L.nrg);
    const int c = (int)((local / L.nrg) % L.nchunks);
    const int p = (int)(local / ((int64_t)L.nrg * L.nchunks));
    const int T = run.T;
    const int lane = threadIdx.x & 63, wave = wave_id();
    constexpr int TPB = 16 / NL;

    // ---- B operands: fp8 limbs of g_p (.) x over this chunk -----------------
    clear_ops(smem, L.kcg * NB);
    __syncthreads();
    {
        const int blocks = L.kcg * 4;                       // 32-element blocks
        const int units = T * blocks;
        const int64_t i0 = (int64_t)c * L.kcg * 128;
        const uint16_t *gp = L.g + (int64_t)p * L.d_in;
        for (int u0 = 2 * wave; u0 < units; u0 += 2 * kWaves) {
            const int u = u0 + (lane >> 5);
            const bool ok = u < units;
            const int n = ok ? u / blocks : 0;
            const int e = ok ? (u % blocks) * 32 + (lane & 31) : 0;   // element in chunk
            const int64_t i = i0 + e;
            float v = 0.0f;
            if (ok && i < L.d_in) v = f16_to_f32(gp[i]) * load_act(L.x, run.x_dtype, (int64_t)n * L.d_in + i);
            emit_limbs<NL>(v, e & 127, n, ok, smem + (e >> 7) * NB * kBopS);
        }
    }
    __syncthreads();

    // ---- stream V planes of this chunk for one 64-latent tile per wave ------
    const int row0 = rg * kRG + wave * kTile;
    const int r16 = lane & 15, gq = lane >> 4;
    const int row = row0 + 4 * r16;
    if (row0 < L.r_p) {
        v4f acc[4][NB];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[m][b] = v4f{0.f, 0.f, 0.f, 0.f};
        const uint32_t *vb = L.v_bits + (int64_t)p * L.kw_v * L.ld_v;
        const int plane0 = c * L.kcg * 4;
        for (int k0 = 0; k0 < L.kcg; k0 += 8) {
            v4u w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int plane = plane0 + 4 * (k0 + j) + gq;
                const bool ok = (k0 + j) < L.kcg && plane < L.kw_v && row < L.r_p;
                w[j] = load_rows(vb + (int64_t)plane * L.ld_v + row, ok);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (k0 + j >= L.kcg) break;
                const uint8_t *ops = smem + (k0 + j) * NB * kBopS;
                v8i bo[NB];
                int sb[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    bo[b] = load_bop(ops + b * kBopS);
                    sb[b] = ops[b * kBopS + kBop + lane];
                }
                const uint32_t ws[4] = {w[j][0], w[j][1], w[j][2], w[j][3]};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const v8i a = unpack_word(ws[m]);
#pragma unroll
                    for (int b = 0; b < NB; ++b) acc[m][b] = mfma(a, bo[b], acc[m][b], sb[b]);
                }
            }
        }
        // ---- partial latent sums: lanes holding a token's first limb write 16 rows
        const int64_t R = (int64_t)L.P * L.r_p;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int cin = r16;
            const int n = b * TPB + cin / NL;
            const bool writer = (cin % NL) == 0 && cin / NL < TPB && n < T;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float s = limb_sum<NL>(acc[m][b][i]);
                    const int k = row0 + 16 * gq + 4 * i + m;
                    if (writer && k < L.r_p)
                        L.part[((int64_t)c * T + n) * R + (int64_t)p * L.r_p + k] = s;
                }
        }
    }

    // ---- the last chunk of this (path, latent group) builds the stage-2 operands
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old = atomicAdd(&L.cnt[p * L.nrg + rg], 1u);
        s_last = (old == (unsigned)(L.nchunks - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    const int kg_first = rg * 2;                                  // 256 latents = 2 K-groups
    const int kg_count = (int)imin(2, L.kg2 - kg_first);
    clear_ops(smem, kg_count * NB);
    __syncthreads();
    {
        const int64_t R = (int64_t)L.P * L.r_p;
        const int blocks = kg_count * 4;
        const int units = T * blocks;
        const uint16_t *lp = L.l + (int64_t)p * L.r_p;
        for (int u0 = 2 * wave; u0 < units; u0 += 2 * kWaves) {
            const int u = u0 + (lane >> 5);
            const bool ok = u < units;
            const int n = ok ? u / blocks : 0;
            const int e = ok ? (u % blocks) * 32 + (lane & 31) : 0;   // latent in group
            const int k = rg * kRG + e;
            float v = 0.0f;
            if (ok && k < L.r_p) {
                float s = 0.0f;
                for (int cc = 0; cc < L.nchunks; ++cc)
                    s += L.part[((int64_t)cc * T + n) * R + (int64_t)p * L.r_p + k];
                v = f16_to_f32(lp[k]) * s;
            }
            emit_limbs<NL>(v, e & 127, n, ok, smem + (e >> 7) * NB * kBopS);
        }
    }
    __syncthreads();
    {
        const int4 *src = (const int4 *)smem;
        int4 *dst = (int4 *)(L.tb + ((int64_t)p * L.kg2 + kg_first) * NB * kBopS);
        const int vecs = kg_count * NB * kBopS / 16;
        for (int i = threadIdx.x; i < vecs; i += kThreads) dst[i] = src[i];
    }
    if (threadIdx.x == 0) L.cnt[p * L.nrg + rg] = 0u;   // ready for the next call
}

// ---------------------------------------------------------------------------
// stage 2
// ---------------------------------------------------------------------------

template <int NL, int NB, int TW>
__global__ __launch_bounds__(kThreads) void k_stage2(MRun run, MLin single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const MLin L = pick(run, single, run.lin2);
    const int64_t local = (int64_t)blockIdx.x - L.item2;
    const int T = run.T;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r16 = lane & 15, gq = lane >> 4;
    constexpr int TPB = 16 / NL;
    const int64_t base = local * L.rows2 + (int64_t)wave * TW * kTile;

    v4f acc[TW][2][4][NB];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[t][p][m][b] = v4f{0.f, 0.f, 0.f, 0.f};

    const int chunk = kLdsBudget / (NB * kBopS);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        if (p >= L.P) break;                            // uniform
        for (int k0 = 0; k0 < L.kg2; k0 += chunk) {
            const int ns = (int)imin(chunk, L.kg2 - k0);
            __syncthreads();
            {
                const int4 *src = (const int4 *)(L.tb + ((int64_t)p * L.kg2 + k0) * NB * kBopS);
                int4 *dst = (int4 *)smem;
                const int vecs = ns * NB * kBopS / 16;
                for (int i = threadIdx.x; i < vecs; i += kThreads) dst[i] = src[i];
            }
            __syncthreads();
            const uint32_t *ub = L.u_bits + (int64_t)p * L.kw_u * L.ld_u;
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const int64_t row = base + t * kTile + 4 * r16;
                const bool row_ok = row < L.d_out;
                for (int j0 = 0; j0 < ns; j0 += 8) {
                    v4u w[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int plane = 4 * (k0 + j0 + j) + gq;
                        const bool ok = (j0 + j) < ns && plane < L.kw_u && row_ok;
                        w[j] = load_rows(ub + (int64_t)plane * L.ld_u + row, ok);
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        if (j0 + j >= ns) break;                    // uniform
                        const uint8_t *ops = smem + (j0 + j) * NB * kBopS;
                        v8i bo[NB];
                        int sb[NB];
#pragma unroll
                        for (int b = 0; b < NB; ++b) {
                            bo[b] = load_bop(ops + b * kBopS);
                            sb[b] = ops[b * kBopS + kBop + lane];
                        }
                        const uint32_t ws[4] = {w[j][0], w[j][1], w[j][2], w[j][3]};
#pragma unroll
                        for (int m = 0; m < 4; ++m) {
                            const v8i a = unpack_word(ws[m]);
#pragma unroll
                            for (int b = 0; b < NB; ++b) acc[t][p][m][b] = mfma(a, bo[b], acc[t][p][m][b], sb[b]);
                        }
                    }
                }
            }
        }
    }

    // ---- epilogue: y = sum_p h_p z_p, one lane per (token, 16 rows) -----------
#pragma unroll
    for (int t = 0; t < TW; ++t) {
        const int64_t rowb = base + t * kTile + 16 * gq;    // this lane's 16 rows
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int cin = r16;
            const int n = b * TPB + cin / NL;
            const bool writer = (cin % NL) == 0 && cin / NL < TPB && n < T;
            float z[2][16];
#pragma unroll
            for (int p = 0; p < 2; ++p)
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int i = 0; i < 4; ++i) z[p][4 * i + m] = limb_sum<NL>(acc[t][p][m][b][i]);
            if (writer) {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int64_t j = rowb + q;
                    if (j < L.d_out) {
                        float y = f16_to_f32(L.h[j]) * z[0][q];
                        if (L.P == 2) y += f16_to_f32(L.h[L.d_out + j]) * z[1][q];
                        store_act(L.y, run.y_dtype, (int64_t)n * L.d_out + j, y);
                    }
                }
            }
        }
    }
}

__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct Shape {
    int NL, NB, TW;
};

bool shape_for(int64_t T, int y_dtype, Shape *s) {
    s->NL = y_dtype == LB_F32 ? 3 : 2;
    const int tpb = 16 / s->NL;
    s->NB = (int)cdiv(T, tpb);
    if (s->NB == 3) s->NB = 4;
    if (s->NB > 4 || T < 1) return false;
    s->TW = s->NB == 1 ? 2 : 1;
    return true;
}

size_t rup256(size_t n) { return (n + 255) & ~(size_t)255; }

// Fill the schedule fields of m and return the workspace bytes it needs.
size_t plan_linear(const Linear &a, const Shape &s, bool many, MLin *m) {
    m->x = a.x;
    m->y = a.y;
    m->v_bits = a.v_bits;
    m->u_bits = a.u_bits;
    m->g = a.g;
    m->l = a.l;
    m->h = a.h;
    m->ld_v = a.ld_v;
    m->ld_u = a.ld_u;
    m->d_in = a.d_in;
    m->d_out = a.d_out;
    m->r_p = (int32_t)a.r_p;
    m->P = a.P;
    m->kw_v = (int32_t)a.kw_v();
    m->kw_u = (int32_t)a.kw_u();
    m->nrg = (int32_t)cdiv(a.r_p, kRG);
    int kcg = (int)imin(8, kLdsBudget / (s.NB * kBopS));
    const int64_t kgv = cdiv(m->kw_v, 4);
    if (!many)   // a lone linear: smaller chunks until the chip has work
        while (kcg > 1 && a.P * m->nrg * cdiv(kgv, kcg) < 512) kcg = (kcg + 1) / 2;
    if (kcg > kgv) kcg = (int)kgv;
    m->kcg = kcg;
    m->nchunks = (int32_t)cdiv(kgv, kcg);
    m->kg2 = (int32_t)cdiv(m->kw_u, 4);
    m->rows2 = kWaves * s.TW * kTile;
    m->n2 = (int32_t)cdiv(a.d_out, m->rows2);
    const size_t cnt = rup256((size_t)a.P * m->nrg * 4);
    const size_t part = rup256((size_t)m->nchunks * a.T * a.P * a.r_p * 4);
    const size_t tb = rup256((size_t)a.P * m->kg2 * s.NB * kBopS);
    return cnt + part + tb;
}

void bind_ws(MLin *m, const Linear &a, const Shape &s, uint8_t *ws) {
    const size_t cnt = rup256((size_t)a.P * m->nrg * 4);
    const size_t part = rup256((size_t)m->nchunks * a.T * a.P * a.r_p * 4);
    m->cnt = (uint32_t *)ws;
    m->part = (float *)(ws + cnt);
    m->tb = ws + cnt + part;
}

size_t lds1(const Shape &s, int kcg) { return (size_t)(kcg > 2 ? kcg : 2) * s.NB * kBopS; }
size_t lds2(const Shape &s) { return (size_t)(kLdsBudget / (s.NB * kBopS)) * s.NB * kBopS; }

template <int NL, int NB, int TW>
int launch_pair(const MRun &run, const MLin &single, int kcg_max, hipStream_t st) {
    Shape s{NL, NB, TW};
    k_stage1<NL, NB><<<(unsigned)run.items1, kThreads, lds1(s, kcg_max), st>>>(run, single);
    if (int rc = last_launch_status()) return rc;
    k_stage2<NL, NB, TW><<<(unsigned)run.items2, kThreads, lds2(s), st>>>(run, single);
    return last_launch_status();
}

int launch_shape(const Shape &s, const MRun &run, const MLin &single, int kcg_max, hipStream_t st) {
    if (s.NL == 2) {
        switch (s.NB) {
            case 1: return launch_pair<2, 1, 2>(run, single, kcg_max, st);
            case 2: return launch_pair<2, 2, 1>(run, single, kcg_max, st);
            case 4: return launch_pair<2, 4, 1>(run, single, kcg_max, st);
        }
    } else {
        switch (s.NB) {
            case 1: return launch_pair<3, 1, 2>(run, single, kcg_max, st);
            case 2: return launch_pair<3, 2, 1>(run, single, kcg_max, st);
            case 4: return launch_pair<3, 4, 1>(run, single, kcg_max, st);
        }
    }
    return LB_EUNSUPPORTED;
}

}  // namespace

bool mfma_decode_supported(int64_t T, int y_dtype) {
    Shape s;
    return shape_for(T, y_dtype, &s);
}

size_t mfma_decode_workspace_bytes(const Linear &a) {
    // sized for the larger of the two output dtypes' limb counts
    size_t need = 0;
    for (int yd : {LB_BF16, LB_F32}) {
        Shape s;
        if (!shape_for(a.T, yd, &s)) continue;
        MLin m{};
        const size_t b = plan_linear(a, s, false, &m);
        if (b > need) need = b;
    }
    return need;
}

int mfma_decode_forward(const Linear &a, void *ws, hipStream_t st) {
    Shape s;
    if (!shape_for(a.T, a.y_dtype, &s)) return LB_EUNSUPPORTED;
    MLin m{};
    plan_linear(a, s, false, &m);
    bind_ws(&m, a, s, (uint8_t *)ws);
    m.item1 = 0;
    m.item2 = 0;
    MRun run{};
    run.T = (int)a.T;
    run.NL = s.NL;
    run.NB = s.NB;
    run.x_dtype = a.x_dtype;
    run.y_dtype = a.y_dtype;
    run.items1 = (int64_t)a.P * m.nchunks * m.nrg;
    run.items2 = m.n2;
    run.table = nullptr;
    const int64_t ncnt = (int64_t)a.P * m.nrg;
    k_fill_u32<<<(unsigned)cdiv(ncnt, 256), 256, 0, st>>>(m.cnt, ncnt, 0u);
    if (int rc = last_launch_status()) return rc;
    return launch_shape(s, run, m, m.kcg, st);
}

// ---- groups ------------------------------------------------------------------

struct MGroupHost {
    Shape s;
    MRun run;
    int kcg_max;
};

size_t mfma_group_workspace_bytes(const Linear *ls, int n, int64_t T, int y_dtype) {
    Shape s;
    if (!shape_for(T, y_dtype, &s)) return 0;
    size_t need = 256 + rup256(sizeof(MLin) * n);
    int64_t i1 = 0, i2 = 0;
    for (int j = 0; j < n; ++j) {
        MLin m{};
        need += plan_linear(ls[j], s, true, &m);
        i1 += (int64_t)ls[j].P * m.nchunks * m.nrg;
        i2 += m.n2;
    }
    need += rup256((size_t)i1 * 4) + rup256((size_t)i2 * 4);
    return need;
}

int mfma_group_prepare(const Linear *ls, int n, int64_t T, int y_dtype, void *ws, size_t ws_bytes,
                       void *host_state, hipStream_t st) {
    MGroupHost *hs = (MGroupHost *)host_state;
    if (!shape_for(T, y_dtype, &hs->s)) return LB_EUNSUPPORTED;
    if (ws_bytes < mfma_group_workspace_bytes(ls, n, T, y_dtype)) return LB_EWORKSPACE;
    uint8_t *w = (uint8_t *)ws;
    MLin *table_dev = (MLin *)(w + 256);
    uint8_t *cur = w + 256 + rup256(sizeof(MLin) * n);
    MLin *tab = new MLin[n];
    int64_t i1 = 0, i2 = 0;
    int kcg_max = 1;
    for (int j = 0; j < n; ++j) {
        MLin &m = tab[j];
        const size_t b = plan_linear(ls[j], hs->s, true, &m);
        bind_ws(&m, ls[j], hs->s, cur);
        cur += b;
        m.item1 = i1;
        m.item2 = i2;
        i1 += (int64_t)ls[j].P * m.nchunks * m.nrg;
        i2 += m.n2;
        if (m.kcg > kcg_max) kcg_max = m.kcg;
    }
    int32_t *lin1 = (int32_t *)cur;
    int32_t *lin2 = (int32_t *)(cur + rup256((size_t)i1 * 4));
    int32_t *h1 = new int32_t[i1], *h2 = new int32_t[i2];
    for (int j = 0; j < n; ++j) {
        const int64_t c1 = (int64_t)ls[j].P * tab[j].nchunks * tab[j].nrg;
        for (int64_t k = 0; k < c1; ++k) h1[tab[j].item1 + k] = j;
        for (int64_t k = 0; k < tab[j].n2; ++k) h2[tab[j].item2 + k] = j;
    }
    int rc = LB_OK;
    if (hipMemcpy(table_dev, tab, sizeof(MLin) * n, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(lin1, h1, (size_t)i1 * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(lin2, h2, (size_t)i2 * 4, hipMemcpyHostToDevice) != hipSuccess)
        rc = LB_EHIP;
    // counters start at zero; every run leaves them at zero
    for (int j = 0; j < n && rc == LB_OK; ++j)
        if (hipMemsetAsync(tab[j].cnt, 0, (size_t)ls[j].P * tab[j].nrg * 4, st) != hipSuccess)
            rc = LB_EHIP;
    if (rc == LB_OK && hipStreamSynchronize(st) != hipSuccess) rc = LB_EHIP;
    delete[] tab;
    delete[] h1;
    delete[] h2;
    if (rc) return rc;
    MRun &run = hs->run;
    run = MRun{};
    run.T = (int)T;
    run.NL = hs->s.NL;
    run.NB = hs->s.NB;
    run.x_dtype = ls[0].x_dtype;
    run.y_dtype = y_dtype;
    run.items1 = i1;
    run.items2 = i2;
    run.table = table_dev;
    run.lin1 = lin1;
    run.lin2 = lin2;
    hs->kcg_max = kcg_max;
    return LB_OK;
}

size_t mfma_group_state_bytes() { return sizeof(MGroupHost); }

int mfma_group_run(const void *host_state, hipStream_t st) {
    const MGroupHost *hs = (const MGroupHost *)host_state;
    MLin dummy{};
    return launch_shape(hs->s, hs->run, dummy, hs->kcg_max, st);
}

}  // namespace lb
