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
// (fp8 A x fp4 B, fp32 accumulate) contracts 128 weight bits of 16 weight rows
// against up to 16 (token, path, limb) activation rows per instruction.  Two
// limbs keep the relative error near 1e-3 (bf16 outputs), three near 2e-5
// (fp32 outputs).
//
// Operand roles: A = activation limbs (M rows: token slot x path x limb),
// B = signs (N columns: 16 weight rows).  The accumulator of lane l holds A
// rows 4*(l/16)..+3 of weight row l%16, so every limb and path of one token
// and one output row sits in one lane and the epilogue is a few in-lane adds.
//
// Data layout: packed planes (littlebit.h) put word (w, row) at w*ld + row, so
// one 16-byte load gives a lane four consecutive rows of one plane and a wave
// covers 64 rows x 4 planes (four 16-column MFMA instances share one A operand).
//
// Three launches per call or per group of linears (kernel boundaries are the
// only cross-workgroup synchronisation: a device-scope fence would write back
// the whole L2 of an XCD on gfx950):
//   stage 1: item = (linear, path, chunk of d_in, group of 256 latents).  The
//            workgroup issues its V-plane loads, turns g (.) x for its chunk
//            into fp8 limbs in LDS meanwhile, and writes partial latent sums.
//   latent:  item = (linear, path, group of 256 latents): adds the chunk
//            partials in chunk order, scales by l and writes the stage-2 A
//            operands (limbs of t) in MFMA lane order.
//   stage 2: item = (linear, block of output rows).  The workgroup copies the
//            A operands of its linear into LDS and each wave walks 64-row tiles,
//            streaming the U planes of both paths into one accumulator set.
#include <vector>

#include "lb_internal.h"

namespace lb {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;                 // weight rows per wave tile (4 MFMA instances of 16)
constexpr int kRG = kWaves * kTile;       // stage-1 latent rows per workgroup
constexpr int kOp = 64 * 32;              // bytes of one fp8 operand (64 lanes x 32)
constexpr int kOpS = kOp + 64;            // plus one scale byte per lane
constexpr int kLdsBudget = 64 * 1024;
constexpr int kMaxKcg = 16;               // K-groups per stage-1 chunk (loads in flight per wave)
constexpr int kBatch = 8;                 // stage-2 steps per load batch
constexpr int kTilesPerItem2 = 8;         // 64-row tiles per wave in one stage-2 item

// Activation-row layout of the A operands.  Stage 1 (one path): token n uses
// rows (n % TPM1)*S1 + q, S1 = 2 (two limbs) or 4 (three limbs).  Stage 2 (both
// paths): token n uses rows (n % TPM2)*S2 + p*NL + q, S2 = 4 or 8.  A token's
// rows fall in one group of four (one lane's accumulator) except for S2 = 8,
// whose two halves sit 16 lanes apart.
template <int NL> struct Rows {
    static constexpr int S1 = NL == 2 ? 2 : 4;
    static constexpr int TPM1 = 16 / S1;
    static constexpr int S2 = NL == 2 ? 4 : 8;
    static constexpr int TPM2 = 16 / S2;
};

// Per-linear schedule and workspace pointers (device-resident for groups).
struct MLin {
    const void *x;
    void *y;
    const uint32_t *v_bits, *u_bits;
    const uint16_t *g, *l, *h;
    int64_t ld_v, ld_u, d_in, d_out;
    int32_t r_p, P;
    int32_t kw_v, kw_u;   // planes of V (per path) and of U (per path)
    int32_t kcg;          // K-groups (128 inputs) per stage-1 chunk, <= kMaxKcg
    int32_t nchunks;      // stage-1 chunks along d_in
    int32_t nrg;          // 256-latent groups per path
    int32_t kg2;          // stage-2 K-groups per path
    int32_t rows2;        // output rows per stage-2 item
    int32_t n2;           // stage-2 items
    int64_t item1, itemF, item2;   // first item of this linear in each launch
    float *part;          // [nchunks][T][P*r_p]
    uint8_t *tb;          // [P][kg2][NB2] operands of kOpS bytes
};

struct MRun {
    int T, x_dtype, y_dtype;
    int ops2;                  // stage-2 operands (steps) the LDS holds at once
    int64_t items1, itemsF, items2;
    const MLin *table;         // null: the single linear passed by value
    const int32_t *lin1, *linF, *lin2;   // item -> linear, per launch
};

__device__ __forceinline__ float ldexp2(float v, int e) { return __builtin_amdgcn_ldexpf(v, e); }

// fp32 -> OCP e4m3 byte (round to nearest even; in range by construction)
__device__ __forceinline__ uint32_t to_fp8(float v) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xffu;
}
__device__ __forceinline__ float from_fp8(uint32_t b) {
    return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// Byte offset of (element e of a 128-element K-group, activation row c) in one
// fp8 operand.  The fp4 sign operand holds bit 4i+q of plane word g in MFMA slot
// s = 8q+i (fp4 lanes carry K = 32g+s); an fp8 operand holds K in lane group
// (K mod 64)/16 at byte (K mod 16) + 16*(K >= 64) (measured layout of the
// f8f6f4 instruction; the scale of K-block g sits in lane c + 16g).
__device__ __forceinline__ int op_offset(int e, int c) {
    const int g = e >> 5, bit = e & 31;
    const int s = ((bit & 3) << 3) | (bit >> 2);
    const int K = (g << 5) | s;
    const int gp = (K & 63) >> 4;
    const int sp = (K & 15) | ((K >> 6) << 4);
    return ((c + (gp << 4)) << 5) + sp;
}

// The NL limbs of v (element e of a K-group) into operand `op` at activation
// rows c0 .. c0+NL-1.  Called by whole waves: each 32-lane half handles one
// 32-element block (one plane word), whose largest magnitude sets the scales
// 2^(E-7-4q).  Lanes with ok == false take part in the reduction with v = 0
// and store nothing.
template <int NL>
__device__ __forceinline__ void emit_limbs(float v, int e, int c0, bool ok, uint8_t *op) {
    float m = fabsf(v);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const int E = (int)((__float_as_uint(m) >> 23) & 0xff) - 127;   // floor(log2 m); m == 0 -> -127
    const int off = op_offset(e, c0);
    float r = v;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
        const int eq = E - 7 - 4 * q;
        const uint32_t b = to_fp8(ldexp2(r, -eq));
        r -= ldexp2(from_fp8(b), eq);
        if (ok) {
            op[off + 32 * q] = (uint8_t)b;              // row c0+q is 32 bytes on
            if ((e & 31) == 0) {
                int sc = eq + 127;
                sc = sc < 0 ? 0 : (sc > 254 ? 254 : sc);
                op[kOp + c0 + q + ((e >> 5) << 4)] = (uint8_t)sc;
            }
        }
    }
}

// Zero the fp8 bytes and set scales to 1.0 for `count` operands at ops (LDS).
__device__ __forceinline__ void clear_ops(uint8_t *ops, int count) {
    uint32_t *w = (uint32_t *)ops;
    const int words = count * kOpS / 4;
    for (int i = threadIdx.x; i < words; i += kThreads) {
        const int off = (i * 4) % kOpS;
        w[i] = off >= kOp ? 0x7f7f7f7fu : 0u;
    }
}

// (x & mask) | one with mask = 0x88888888 in an SGPR and one = 0x22222222 in
// a VGPR: a single v_and_or_b32 (VOP3 on gfx950 takes no literal operand, so
// the compiler would otherwise split it into an AND and an OR).
struct Nib {
    uint32_t mask, one;
};

__device__ __forceinline__ uint32_t sign_nibbles(uint32_t x, const Nib &k) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(k.mask), "v"(k.one));
    return r;
}

// fp4 sign operand of one plane word: slot 8q+i <- bit 4i+q, as +-1.0.
__device__ __forceinline__ v8i unpack_word(uint32_t w, const Nib &one) {
    v8i a;
    a[0] = (int)sign_nibbles(w << 3, one);
    a[1] = (int)sign_nibbles(w << 2, one);
    a[2] = (int)sign_nibbles(w << 1, one);
    a[3] = (int)sign_nibbles(w, one);
    a[4] = a[5] = a[6] = a[7] = 0;
    return a;
}

// The two constants of sign_nibbles in registers, opaque to constant folding.
__device__ __forceinline__ Nib nibble_constants() {
    Nib k;
    asm volatile("s_mov_b32 %0, 0x88888888" : "=s"(k.mask));
    asm volatile("v_mov_b32 %0, 0x22222222" : "=v"(k.one));
    return k;
}
__device__ __forceinline__ v8i load_op(const uint8_t *op) {
    const int4 *p = (const int4 *)(op + (threadIdx.x & 63) * 32);
    const int4 lo = p[0], hi = p[1];
    v8i b;
    b[0] = lo.x; b[1] = lo.y; b[2] = lo.z; b[3] = lo.w;
    b[4] = hi.x; b[5] = hi.y; b[6] = hi.z; b[7] = hi.w;
    return b;
}

// acc += act (fp8, scale sa per lane) x signs (fp4, scale 1.0)
__device__ __forceinline__ v4f mfma(const v8i &act, const v8i &sg, v4f c, int sa) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(act, sg, c, 0, 4, 0, sa, 0, 127);
}

// Buffer descriptor of `bytes` bytes at p (raw, stride 0; gfx9-family dword 3).
// Loads past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
    const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, n, 0x00020000);
}

// Four consecutive rows of one plane: a 16-byte nontemporal load at byte
// offset voff of the descriptor (zeros when out of range).
__device__ __forceinline__ v4u load_rows(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 2);
}

// The linear of a work item, as a wave-uniform value (matrix instructions
// ignore the exec mask, so every branch around them must be uniform).
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

// Store 4 consecutive outputs y[e0 .. e0+4) (only those with row < d_out).
__device__ __forceinline__ void store4(void *y, int dtype, int64_t e0, int64_t row, int64_t d_out,
                                      const float (&v)[4]) {
    if (row + 4 <= d_out) {
        if (dtype == LB_BF16) {
            uint16_t *p = (uint16_t *)y + e0;
            if (((uintptr_t)p & 7) == 0) {
                v2u w;
                w[0] = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                w[1] = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                *(v2u *)p = w;
                return;
            }
        } else {
            float *p = (float *)y + e0;
            if (((uintptr_t)p & 15) == 0) {
                *(v4f *)p = v4f{v[0], v[1], v[2], v[3]};
                return;
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (row + q < d_out) store_act(y, dtype, e0 + q, v[q]);
}

// ---------------------------------------------------------------------------
// stage 1: partial latent sums u = sign(V_p)^T (g_p (.) x) over one chunk
// ---------------------------------------------------------------------------

template <int NL, int NB1>
__global__ __launch_bounds__(kThreads) void k_stage1(MRun run, MLin single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using R = Rows<NL>;
    const MLin L = pick(run, single, run.lin1);
    const int64_t local = (int64_t)blockIdx.x - L.item1;
    const int rg = (int)(local % L.nrg);
    const int c = (int)((local / L.nrg) % L.nchunks);
    const int p = (int)(local / ((int64_t)L.nrg * L.nchunks));
    const int T = run.T;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r16 = lane & 15, gq = lane >> 4;
    const Nib one = nibble_constants();

    // ---- the V-plane loads go out first; the limb work below hides them ----
    const int row0 = rg * kRG + wave * kTile;
    const int row = row0 + 4 * r16;
    const bool active = row0 < L.r_p;                            // wave-uniform
    // planes of this path only: planes past d_in read as zeros (their inputs are zero too)
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(L.v_bits + (int64_t)p * L.kw_v * L.ld_v, (int64_t)L.kw_v * L.ld_v * 4);
    const int plane0 = c * L.kcg * 4;
    const uint32_t vo = (uint32_t)(((int64_t)(plane0 + gq) * L.ld_v + row) * 4);
    const uint32_t vstep = (uint32_t)(4 * L.ld_v * 4);                 // one K-group of planes
    v4u w[kMaxKcg];
#pragma unroll
    for (int j = 0; j < kMaxKcg; ++j)
        w[j] = (active && j < L.kcg) ? load_rows(rv, vo + j * vstep) : v4u{0u, 0u, 0u, 0u};

    // ---- A operands: fp8 limbs of g_p (.) x over this chunk -----------------
    clear_ops(smem, L.kcg * NB1);
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
            uint8_t *op = smem + ((e >> 7) * NB1 + n / R::TPM1) * kOpS;
            emit_limbs<NL>(v, e & 127, (n % R::TPM1) * R::S1, ok, op);
        }
    }
    __syncthreads();
    if (!active) return;

    v4f acc[4][NB1];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int b = 0; b < NB1; ++b) acc[m][b] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxKcg; ++j) {
        if (j >= L.kcg) continue;                               // uniform; keeps w[] in registers
        const uint8_t *ops = smem + j * NB1 * kOpS;
        v8i ao[NB1];
        int sa[NB1];
#pragma unroll
        for (int b = 0; b < NB1; ++b) {
            ao[b] = load_op(ops + b * kOpS);
            sa[b] = ops[b * kOpS + kOp + lane];
        }
        const uint32_t ws[4] = {w[j][0], w[j][1], w[j][2], w[j][3]};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const v8i sg = unpack_word(ws[m], one);
#pragma unroll
            for (int b = 0; b < NB1; ++b) acc[m][b] = mfma(ao[b], sg, acc[m][b], sa[b]);
        }
    }

    // ---- partial latent sums: lane (gq, r16) holds latents row0+4*r16+m -------
    const int64_t Rtot = (int64_t)L.P * L.r_p;
    const int k0 = row0 + 4 * r16;
#pragma unroll
    for (int b = 0; b < NB1; ++b) {
#pragma unroll
        for (int s = 0; s < 4 / R::S1; ++s) {         // tokens in this lane's row group
            const int n = b * R::TPM1 + gq * (4 / R::S1) + s;
            float u[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                float sum = 0.0f;
#pragma unroll
                for (int q = 0; q < NL; ++q) sum += acc[m][b][s * R::S1 + q];
                u[m] = sum;
            }
            if (n < T && k0 < L.r_p)
                store4(L.part, LB_F32, ((int64_t)c * T + n) * Rtot + (int64_t)p * L.r_p + k0, k0,
                       L.r_p, u);
        }
    }
}

// ---------------------------------------------------------------------------
// latents: t = l (.) sum over chunks, as the stage-2 A operands
// ---------------------------------------------------------------------------

template <int NL, int NB2>
__global__ __launch_bounds__(kThreads) void k_latent(MRun run, MLin single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using R = Rows<NL>;
    const MLin L = pick(run, single, run.linF);
    const int64_t local = (int64_t)blockIdx.x - L.itemF;
    const int rg = (int)(local % L.nrg);
    const int p = (int)(local / L.nrg);
    const int T = run.T;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int kg_first = rg * 2;                                  // 256 latents = 2 K-groups
    const int kg_count = (int)imin(2, L.kg2 - kg_first);
    clear_ops(smem, kg_count * NB2);
    __syncthreads();
    const int64_t Rtot = (int64_t)L.P * L.r_p;
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
            float sum = 0.0f;
            for (int cc = 0; cc < L.nchunks; ++cc)
                sum += L.part[((int64_t)cc * T + n) * Rtot + (int64_t)p * L.r_p + k];
            v = f16_to_f32(lp[k]) * sum;
        }
        uint8_t *op = smem + ((e >> 7) * NB2 + n / R::TPM2) * kOpS;
        emit_limbs<NL>(v, e & 127, (n % R::TPM2) * R::S2 + p * NL, ok, op);
    }
    __syncthreads();
    const int4 *src = (const int4 *)smem;
    int4 *dst = (int4 *)(L.tb + ((int64_t)p * L.kg2 + kg_first) * NB2 * kOpS);
    const int vecs = kg_count * NB2 * kOpS / 16;
    for (int i = threadIdx.x; i < vecs; i += kThreads) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// stage 2: y = sum_p h_p (.) (sign(U_p) t_p)
// ---------------------------------------------------------------------------

// Each wave walks 64-row tiles; the U-plane loads of the next batch go out
// before the current batch is multiplied, and h for the tile's rows is fetched
// before its last batch.
template <int NL, int NB2>
__global__ __launch_bounds__(kThreads) void k_stage2(MRun run, MLin single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using R = Rows<NL>;
    const MLin L = pick(run, single, run.lin2);
    const int64_t local = (int64_t)blockIdx.x - L.item2;
    const int T = run.T;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r16 = lane & 15, gq = lane >> 4;
    const Nib one = nibble_constants();

    const int steps = L.P * L.kg2;                 // (path, K-group) pairs, path-major
    const int ops = run.ops2;                      // steps the LDS holds (a multiple of kBatch when < steps)
    const bool fits = steps <= ops;
    const int nbat = (int)cdiv(steps, kBatch);     // batches per tile
    const int64_t row_begin = local * L.rows2;
    const int tiles = (int)imin(L.rows2 / kRG, cdiv(L.d_out - row_begin, kRG));
    const int units = tiles * nbat;

    if (fits) {
        const int4 *src = (const int4 *)L.tb;
        int4 *dst = (int4 *)smem;
        const int vecs = steps * NB2 * kOpS / 16;
        for (int i = threadIdx.x; i < vecs; i += kThreads) dst[i] = src[i];
    }

    // all U planes of the linear; rows and planes past the end read as zeros
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(L.u_bits, (int64_t)L.P * L.kw_u * L.ld_u * 4);
    const uint32_t uo = (uint32_t)(((int64_t)gq * L.ld_u + wave * kTile + 4 * r16) * 4);
    auto issue = [&](v4u (&w)[kBatch], int u) {
        const int t = u / nbat, b = u % nbat;
        const int64_t rowt = row_begin + (int64_t)t * kRG;                 // uniform
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int st = b * kBatch + j;
            const int pp = st / L.kg2, kg = st % L.kg2;
            const uint32_t so = (uint32_t)((((int64_t)pp * L.kw_u + 4 * kg) * L.ld_u + rowt) * 4);
            // a path's last K-group may reach into the next path's planes: those
            // pair with zero activations
            w[j] = st < steps ? load_rows(ru, uo + so) : v4u{0u, 0u, 0u, 0u};
        }
    };

    v4f acc[4][NB2];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int b = 0; b < NB2; ++b) acc[m][b] = v4f{0.f, 0.f, 0.f, 0.f};

    v4u wc[kBatch];
    issue(wc, 0);
    for (int u = 0; u < units; ++u) {
        const int t = u / nbat, bt = u % nbat;
        const int64_t row = row_begin + (int64_t)t * kRG + wave * kTile + 4 * r16;   // this lane's 4 rows
        const bool last = bt == nbat - 1;
        // h of this lane's 4 rows, both paths, before the last batch of the tile
        float hv[2][4];
        if (last) {
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const uint16_t *hp = L.h + (int64_t)pp * L.d_out + row;
                if (pp < L.P && row + 4 <= L.d_out && ((uintptr_t)hp & 7) == 0) {
                    const v2u hw = *(const v2u *)hp;
                    hv[pp][0] = f16_to_f32((uint16_t)(hw[0] & 0xffffu));
                    hv[pp][1] = f16_to_f32((uint16_t)(hw[0] >> 16));
                    hv[pp][2] = f16_to_f32((uint16_t)(hw[1] & 0xffffu));
                    hv[pp][3] = f16_to_f32((uint16_t)(hw[1] >> 16));
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        hv[pp][q] = (pp < L.P && row + q < L.d_out) ? f16_to_f32(hp[q]) : 0.0f;
                }
            }
        }
        v4u wn[kBatch];
        if (u + 1 < units) issue(wn, u + 1);
        if (!fits && (bt * kBatch) % ops == 0) {   // next chunk of A operands
            const int s0 = bt * kBatch;
            const int ns = (int)imin(ops, steps - s0);
            __syncthreads();
            const int4 *src = (const int4 *)(L.tb + (int64_t)s0 * NB2 * kOpS);
            int4 *dst = (int4 *)smem;
            const int vecs = ns * NB2 * kOpS / 16;
            for (int i = threadIdx.x; i < vecs; i += kThreads) dst[i] = src[i];
        }
        if (u == 0 || !fits) __syncthreads();
        const int lds0 = fits ? 0 : ((bt * kBatch) / ops) * ops;    // first step held in LDS
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int st = bt * kBatch + j;
            if (st >= steps) continue;                          // uniform
            const uint8_t *opp = smem + (st - lds0) * NB2 * kOpS;
            v8i ao[NB2];
            int sa[NB2];
#pragma unroll
            for (int b = 0; b < NB2; ++b) {
                ao[b] = load_op(opp + b * kOpS);
                sa[b] = opp[b * kOpS + kOp + lane];
            }
            const uint32_t ws[4] = {wc[j][0], wc[j][1], wc[j][2], wc[j][3]};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const v8i sg = unpack_word(ws[m], one);
#pragma unroll
                for (int b = 0; b < NB2; ++b) acc[m][b] = mfma(ao[b], sg, acc[m][b], sa[b]);
            }
        }
        if (last) {
            // y = sum_p h_p z_p: lane (gq, r16) holds activation rows 4gq..4gq+3
            // of weight rows row+m; S2 = 4 puts one token's p0/p1 limbs there,
            // S2 = 8 splits them over lane groups gq and gq^1.
#pragma unroll
            for (int b = 0; b < NB2; ++b) {
                float y4[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const v4f a = acc[m][b];
                    // both paths add their limbs in the same order (limb 0 first)
                    if (NL == 2) {
                        y4[m] = hv[0][m] * (a[0] + a[1]) + hv[1][m] * (a[2] + a[3]);
                    } else {
                        // even lane group: p0 limbs 0..2 and p1 limb 0; odd: p1 limbs 1, 2
                        const float o0 = __shfl_xor(a[0], 16, 64), o1 = __shfl_xor(a[1], 16, 64);
                        const float z0 = (a[0] + a[1]) + a[2];
                        const float z1 = (a[3] + o0) + o1;
                        y4[m] = hv[0][m] * z0 + hv[1][m] * z1;
                    }
                }
                const int n = b * R::TPM2 + (NL == 2 ? gq : gq / 2);
                const bool writer = n < T && (NL == 2 || (gq & 1) == 0);
                if (writer) store4(L.y, run.y_dtype, (int64_t)n * L.d_out + row, row, L.d_out, y4);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int b = 0; b < NB2; ++b) acc[m][b] = v4f{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) wc[j] = wn[j];
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

struct Shape {
    int NL, NB1, NB2;
};

// Limbs from the output dtype; activation-row blocks from the token count.
bool shape_for(int64_t T, int y_dtype, Shape *s) {
    if (T < 1) return false;
    s->NL = y_dtype == LB_F32 ? 3 : 2;
    const int tpm1 = s->NL == 2 ? 8 : 4, tpm2 = s->NL == 2 ? 4 : 2;
    const int64_t nb1 = cdiv(T, tpm1), nb2 = cdiv(T, tpm2);
    // instantiated (NB1, NB2) pairs: (1,1) (1,2) (2,4) (4,8)
    if (nb2 <= 1) { s->NB1 = 1; s->NB2 = 1; }
    else if (nb2 <= 2 && nb1 <= 1) { s->NB1 = 1; s->NB2 = 2; }
    else if (nb2 <= 4 && nb1 <= 2) { s->NB1 = 2; s->NB2 = 4; }
    else if (nb2 <= 8 && nb1 <= 4) { s->NB1 = 4; s->NB2 = 8; }
    else return false;
    return true;
}

size_t rup256(size_t n) { return (n + 255) & ~(size_t)255; }

int kcg_cap(const Shape &s) { return (int)imin(kMaxKcg, kLdsBudget / (s.NB1 * kOpS)); }

// Steps the stage-2 LDS holds: all steps of the largest linear when they fit,
// else a multiple of the batch (at least one batch, which may exceed 64 KB).
int ops2_for(const Shape &s, int steps_max) {
    int cap = kLdsBudget / (s.NB2 * kOpS);
    if (cap < kBatch) cap = kBatch;
    return steps_max <= cap ? steps_max : (cap / kBatch) * kBatch;
}

// Fill the schedule fields of m and return the workspace bytes it needs.
size_t plan_linear(const Linear &a, const Shape &s, bool many, MLin *m) {
    *m = MLin{};
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
    int kcg = kcg_cap(s);
    const int64_t kgv = cdiv(m->kw_v, 4);
    if (!many)   // a lone linear: smaller chunks until the chip has work
        while (kcg > 1 && a.P * m->nrg * cdiv(kgv, kcg) < 512) kcg = (kcg + 1) / 2;
    if (kcg > kgv) kcg = (int)kgv;
    m->kcg = kcg;
    m->nchunks = (int32_t)cdiv(kgv, kcg);
    m->kg2 = (int32_t)cdiv(m->kw_u, 4);
    int tiles = kTilesPerItem2;
    if (!many)   // a lone linear: fewer tiles per item until the chip has work
        while (tiles > 1 && cdiv(a.d_out, (int64_t)kRG * tiles) < 512) tiles /= 2;
    m->rows2 = kRG * tiles;
    m->n2 = (int32_t)cdiv(a.d_out, m->rows2);
    const size_t part = rup256((size_t)m->nchunks * a.T * a.P * a.r_p * 4);
    const size_t tb = rup256((size_t)a.P * m->kg2 * s.NB2 * kOpS);
    return part + tb;
}

void bind_ws(MLin *m, const Linear &a, uint8_t *ws) {
    const size_t part = rup256((size_t)m->nchunks * a.T * a.P * a.r_p * 4);
    m->part = (float *)ws;
    m->tb = ws + part;
}

int64_t items1_of(const MLin &m) { return (int64_t)m.P * m.nchunks * m.nrg; }
int64_t itemsF_of(const MLin &m) { return (int64_t)m.P * m.nrg; }

// stage_mask: bit 0 = stage 1 and the latent pass, bit 1 = stage 2.
template <int NL, int NB1, int NB2>
int launch_all(const MRun &run, const MLin &single, int kcg_max, hipStream_t st, int stage_mask) {
    if (stage_mask & 1) {
        const size_t l1 = (size_t)kcg_max * NB1 * kOpS;
        k_stage1<NL, NB1><<<(unsigned)run.items1, kThreads, l1, st>>>(run, single);
        if (int rc = last_launch_status()) return rc;
        k_latent<NL, NB2><<<(unsigned)run.itemsF, kThreads, (size_t)2 * NB2 * kOpS, st>>>(run, single);
        if (int rc = last_launch_status()) return rc;
    }
    if (stage_mask & 2) {
        const size_t l2 = (size_t)run.ops2 * NB2 * kOpS;
        if (run.ops2 < 1 || l2 > 160 * 1024) return LB_EUNSUPPORTED;
        if (l2 > 64 * 1024) {
            static bool raised = false;    // once per instantiation (idempotent if raced)
            if (!raised) {
                // the largest request this instantiation makes: one batch
                const int most = (int)imax((int64_t)l2, (int64_t)kBatch * NB2 * kOpS);
                if (hipFuncSetAttribute((const void *)k_stage2<NL, NB2>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, most) != hipSuccess)
                    return hip_status(hipGetLastError());
                raised = true;
            }
        }
        k_stage2<NL, NB2><<<(unsigned)run.items2, kThreads, l2, st>>>(run, single);
        if (int rc = last_launch_status()) return rc;
    }
    return LB_OK;
}

int launch_shape(const Shape &s, const MRun &run, const MLin &single, int kcg_max, hipStream_t st,
                 int stage_mask = 3) {
    const int key = s.NL * 1000 + s.NB1 * 10 + s.NB2;
    switch (key) {
        case 2011: return launch_all<2, 1, 1>(run, single, kcg_max, st, stage_mask);
        case 2012: return launch_all<2, 1, 2>(run, single, kcg_max, st, stage_mask);
        case 2024: return launch_all<2, 2, 4>(run, single, kcg_max, st, stage_mask);
        case 2048: return launch_all<2, 4, 8>(run, single, kcg_max, st, stage_mask);
        case 3011: return launch_all<3, 1, 1>(run, single, kcg_max, st, stage_mask);
        case 3012: return launch_all<3, 1, 2>(run, single, kcg_max, st, stage_mask);
        case 3024: return launch_all<3, 2, 4>(run, single, kcg_max, st, stage_mask);
        case 3048: return launch_all<3, 4, 8>(run, single, kcg_max, st, stage_mask);
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
        MLin m;
        const size_t b = plan_linear(a, s, false, &m);
        if (b > need) need = b;
    }
    return need;
}

int mfma_decode_forward(const Linear &a, void *ws, hipStream_t st) {
    Shape s;
    if (!shape_for(a.T, a.y_dtype, &s)) return LB_EUNSUPPORTED;
    MLin m;
    plan_linear(a, s, false, &m);
    bind_ws(&m, a, (uint8_t *)ws);
    MRun run{};
    run.T = (int)a.T;
    run.x_dtype = a.x_dtype;
    run.y_dtype = a.y_dtype;
    run.ops2 = ops2_for(s, a.P * m.kg2);
    run.items1 = items1_of(m);
    run.itemsF = itemsF_of(m);
    run.items2 = m.n2;
    run.table = nullptr;
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
    int64_t i1 = 0, iF = 0, i2 = 0;
    for (int j = 0; j < n; ++j) {
        MLin m;
        need += plan_linear(ls[j], s, true, &m);
        i1 += items1_of(m);
        iF += itemsF_of(m);
        i2 += m.n2;
    }
    need += rup256((size_t)i1 * 4) + rup256((size_t)iF * 4) + rup256((size_t)i2 * 4);
    return need;
}

int mfma_group_prepare(const Linear *ls, int n, int64_t T, int y_dtype, void *ws, size_t ws_bytes,
                       void *host_state, hipStream_t st) {
    (void)st;
    MGroupHost *hs = (MGroupHost *)host_state;
    if (!shape_for(T, y_dtype, &hs->s)) return LB_EUNSUPPORTED;
    if (ws_bytes < mfma_group_workspace_bytes(ls, n, T, y_dtype)) return LB_EWORKSPACE;
    uint8_t *w = (uint8_t *)ws;
    MLin *table_dev = (MLin *)(w + 256);
    uint8_t *cur = w + 256 + rup256(sizeof(MLin) * n);
    std::vector<MLin> tab((size_t)n);
    int64_t i1 = 0, iF = 0, i2 = 0;
    int kcg_max = 1, steps_max = 1;
    for (int j = 0; j < n; ++j) {
        MLin &m = tab[(size_t)j];
        const size_t b = plan_linear(ls[j], hs->s, true, &m);
        bind_ws(&m, ls[j], cur);
        cur += b;
        m.item1 = i1;
        m.itemF = iF;
        m.item2 = i2;
        i1 += items1_of(m);
        iF += itemsF_of(m);
        i2 += m.n2;
        if (m.kcg > kcg_max) kcg_max = m.kcg;
        if (m.P * m.kg2 > steps_max) steps_max = m.P * m.kg2;
    }
    int32_t *lin1 = (int32_t *)cur;
    int32_t *linF = (int32_t *)(cur + rup256((size_t)i1 * 4));
    int32_t *lin2 = (int32_t *)(cur + rup256((size_t)i1 * 4) + rup256((size_t)iF * 4));
    std::vector<int32_t> h1((size_t)i1), hF((size_t)iF), h2((size_t)i2);
    for (int j = 0; j < n; ++j) {
        const MLin &m = tab[(size_t)j];
        for (int64_t k = 0; k < items1_of(m); ++k) h1[(size_t)(m.item1 + k)] = j;
        for (int64_t k = 0; k < itemsF_of(m); ++k) hF[(size_t)(m.itemF + k)] = j;
        for (int64_t k = 0; k < m.n2; ++k) h2[(size_t)(m.item2 + k)] = j;
    }
    if (hipMemcpy(table_dev, tab.data(), sizeof(MLin) * n, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(lin1, h1.data(), (size_t)i1 * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(linF, hF.data(), (size_t)iF * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(lin2, h2.data(), (size_t)i2 * 4, hipMemcpyHostToDevice) != hipSuccess)
        return hip_status(hipGetLastError());
    MRun &run = hs->run;
    run = MRun{};
    run.T = (int)T;
    run.x_dtype = ls[0].x_dtype;
    run.y_dtype = y_dtype;
    run.ops2 = ops2_for(hs->s, steps_max);
    run.items1 = i1;
    run.itemsF = iF;
    run.items2 = i2;
    run.table = table_dev;
    run.lin1 = lin1;
    run.linF = linF;
    run.lin2 = lin2;
    hs->kcg_max = kcg_max;
    return LB_OK;
}

size_t mfma_group_state_bytes() { return sizeof(MGroupHost); }

int mfma_group_run(const void *host_state, hipStream_t st, int stage_mask) {
    const MGroupHost *hs = (const MGroupHost *)host_state;
    MLin dummy{};
    return launch_shape(hs->s, hs->run, dummy, hs->kcg_max, st, stage_mask);
}

}  // namespace lb
