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
// Activation operands are kept "compact" in global memory: only the rows in use
// (a 144-byte record each: 128 fp8 bytes in lane-group order, 4 scales), and
// expanded into the MFMA lane layout in LDS by the kernel that consumes them.
//
// Four launches per call or per group of linears (kernel boundaries are the
// only cross-workgroup synchronisation: a device-scope fence would write back
// the whole L2 of an XCD on gfx950):
//   prep:    item = (linear, path, range of d_in): fp8 limbs of g (.) x.
//   stage 1: item = (linear, path, chunk of d_in, group of 256 latents): loads
//            its operands (before the plane loads, since loads complete in
//            order), streams the V planes and writes partial latent sums.
//   latent:  item = (linear, two stage-2 K-groups): adds the chunk partials
//            in chunk order, scales by l and writes the stage-2 operands
//            (limbs of t).  Stage-2 K-groups run over the U planes of both
//            paths back to back, so no plane is read twice.
//   stage 2: item = (linear, block of output rows): each wave walks 64-row
//            tiles, streaming the U planes of both paths into one accumulator set.
#include <atomic>
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "lb_internal.h"
#include "lb_f8.h"

namespace lb {


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
constexpr int kTilesPerItem2 = 8;         // 64-row tiles per wave in one stage-2 item, at most
constexpr int kSteps2 = 40;               // (tile, K-group) steps a stage-2 item aims for, per 4 activation rows
constexpr int kPreVec = 8;                // operand vectors a thread loads before the plane loads
constexpr int kWin2 = 8;                  // stage 2 (streaming form): plane loads in flight per wave
constexpr int kWin1 = 8;                  // stage 1 (fused form): plane loads in flight per wave
constexpr int kEarly1 = 2;                // of which issued before the limb work inside the one-launch pass
constexpr int kTB = 3;                   // stage 1 (fused form): tokens whose inputs load together
constexpr int kMaxKcf = 32;               // K-groups per fused stage-1 chunk (two 8-input pieces per thread)
constexpr uint32_t kOOB = 0x7ffffff0u;    // a buffer offset past every range: reads as zero
// Cache policy of a buffer access at device scope (sc1): coherent across the
// XCDs' L2 caches, as agent-scope atomics are.
constexpr int kDeviceScope = 16;
constexpr int kHRows = kRG * kTilesPerItem2;   // output rows of one stage-2 item, at most
constexpr int kYStage = 16 * 1024;        // LDS for k_stage2r's collected outputs, at most

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
    const void *x2;       // SwiGLU input: the linear reads silu(x) (.) x2 (both bf16), or null
    const float *xs;      // per-token input scale [T] (an RMSNorm's 1/rms), or null
    const void *resid;    // residual [T][d_out] in y's dtype, added to the output, or null
    void *y;
    const uint32_t *v_bits, *u_bits;
    const uint16_t *g, *l, *h;
    int64_t ld_v, ld_u, d_in, d_out;
    int32_t r_p, P;
    int32_t kw_v, kw_u;   // planes of V (per path) and of U (per path)
    int32_t kgv;          // K-groups of V per path
    int32_t kcg;          // K-groups (128 inputs) per stage-1 chunk, <= kMaxKcg (fused: <= kMaxKcf)
    int32_t nchunks;      // stage-1 chunks along d_in
    int32_t kcp;          // K-groups per prep item
    int32_t nprep;        // prep items per path
    int32_t nrg;          // latent groups per path: 256 latents (unfused), F tiles (fused)
    int32_t kgs;          // stage-2 K-groups over the planes of all paths (path-major)
    int32_t rows2;        // output rows per stage-2 item
    int32_t n2;           // stage-2 items
    int32_t R1, R2;       // activation rows in use (compact records per operand)
    int32_t xvec;         // fused stage 1: x and g read as 16-byte pieces (d_in % 8 == 0, aligned)
    int32_t xm_dh, xm_grp;   // fused stage 1: the input map of Linear (xm_dh = 0: none)
    int64_t item0, item1, itemF, item2;   // first item of this linear in each launch
    int64_t fin0;         // the one-launch pass: first (path, latent group) counter of this linear
    float *part;          // [nchunks][T][P*r_p]
    uint8_t *pa;          // stage-1 operands, compact: [P][kgv][NB1][R1][kRec] (unused by the fused form)
    uint8_t *tb;          // stage-2 operands, compact: [kgs][NB2][R2][kRec]
};

// items of a linear in each launch
__host__ __device__ inline int64_t items0_of(const MLin &m) { return (int64_t)m.P * m.nprep; }
__host__ __device__ inline int64_t items1_of(const MLin &m) { return (int64_t)m.P * m.nchunks * m.nrg; }
__host__ __device__ inline int64_t itemsF_of(const MLin &m) { return ((int64_t)m.kgs + 1) / 2; }
// latent groups of a linear (the one-launch pass counts each one's chunks)
__host__ __device__ inline int64_t groups_of(const MLin &m) { return (int64_t)m.P * m.nrg; }

struct MRun {
    int T, x_dtype, y_dtype;
    int ops2;                  // stage-2 operands (steps) the LDS holds at once
    int dma2;                  // stage 2 runs k_stage2r (all operands and h fit the LDS)
    int flush1;                // fused stage 1: latent tiles per item (F)
    int tsplit;                // fused stage 1: waves split the item's tiles (1) or its K-groups (0)
    int ystage;                // k_stage2r collects the item's outputs in LDS, stored after its stream
    int yst;                   // bytes per collected output: y's size, or 4 when a residual is added
    int64_t items0, items1, itemsF, items2;
    int64_t base0, base1, baseF, base2;   // item of workgroup 0 in each launch (0: all items)
    const MLin *table;         // null: the single linear passed by value
    const int32_t *lin0, *lin1, *linF, *lin2;   // item -> linear, per launch
    const int32_t *ord1, *ord2;  // workgroup -> item for stage 1 / stage 2 (largest first; null: identity)
    // the one-launch pass (k_pass)
    const int32_t *ordP1;          // workgroup -> stage-1 item
    const int32_t *tabP2;          // (workgroup - items1) -> (linear, first 256-row tile << 8 | tiles)
    int64_t items2P;               // stage-2 workgroups of k_pass
    uint32_t *arrive;              // per (linear, path, latent group): its stage-1 items counted in
    uint32_t *sync;                // per linear: latent groups stored (low 16 bits), events (high 16 bits)
    uint32_t spin_limit;           // polls a stage-2 wave makes before it gives up
    uint32_t want_extra;           // 0; 1 asks for one latent group more than exists (fault-report test)
    int pass;                      // 1: a full run is one k_pass launch
    // groups: the workspace stamp written at set-up and the tag it must equal
    // (null for a single linear, which keeps nothing in its workspace)
    const uint64_t *stamp;
    uint64_t tag;
    // the latent API (single linears): k_latent also writes the latents t
    // [T][P*r_p] (t_mode 1), or takes them from t instead of the partial sums
    // (t_mode 2); t_dtype LB_F32 or LB_BF16
    void *t_io;
    int t_dtype;
    int t_mode;
    // inline groups: the linears themselves (no device tables; table null)
    int xmap;                  // some linear of the launch reads x through an input map (xm_dh)
    int ninl;
    MLin inl[kMaxInline];
};

// Compact operands -> LDS operand layout.  Each operand holds R records of
// kRec bytes; record r goes to rows r of lane groups 0..3 and its four scales
// to lanes r + 16g.  One 16-byte vector per call; vector i of the source.
__device__ __forceinline__ void expand_vec(uint8_t *dst_ops, int i, int R, const v4u v) {
    const int o = i * 16;
    const int opi = o / (R * kRec);
    const int w = o - opi * R * kRec;
    const int r = w / kRec;
    const int b = w - r * kRec;
    uint8_t *op = dst_ops + opi * kOpS;
    if (b < 128) {
        *(v4u *)(op + ((r + ((b >> 5) << 4)) << 5) + (b & 31)) = v;
    } else if (b == 128) {
        const uint32_t sc = v[0];
#pragma unroll
        for (int g = 0; g < 4; ++g) op[kOp + r + 16 * g] = (uint8_t)(sc >> (8 * g));
    }
}

__device__ __forceinline__ v8i load_op(const uint8_t *op) {
    const int4 *p = (const int4 *)(op + (threadIdx.x & 63) * 32);
    const int4 lo = p[0], hi = p[1];
    v8i b;
    b[0] = lo.x; b[1] = lo.y; b[2] = lo.z; b[3] = lo.w;
    b[4] = hi.x; b[5] = hi.y; b[6] = hi.z; b[7] = hi.w;
    return b;
}

__device__ __forceinline__ v4f mfma(const v8i &act, const v8i &sg, v4f c, int sa) { return mfma_f8f4(act, sg, c, sa); }

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
// Launch kinds, for the inline lookup: which item offset of MLin numbers them.
enum { kKindPrep = 0, kKindStage1 = 1, kKindLatent = 2, kKindStage2 = 3 };

__device__ __forceinline__ int64_t item_start(const MLin &m, int kind) {
    return kind == kKindPrep ? m.item0 : kind == kKindStage1 ? m.item1 : kind == kKindLatent ? m.itemF : m.item2;
}

// Element i of a table the launch only reads (orders, linear maps, linear
// tables: written before the launch) at a uniform index, through the
// constant address space, so the compiler reads it with scalar loads.
template <typename T>
__device__ __forceinline__ T table_at(const T *p, int64_t i) {
    static_assert(sizeof(T) % 4 == 0, "tables are read as 32-bit words");
    typedef const __attribute__((address_space(4))) uint32_t cword;
    cword *q = (cword *)(p + i);
    uint32_t w[sizeof(T) / 4];
#pragma unroll
    for (int k = 0; k < (int)(sizeof(T) / 4); ++k) w[k] = q[k];
    T r;
    __builtin_memcpy(&r, w, sizeof(T));
    return r;
}

// SCALAR: the table entry through scalar loads (the standalone kernels; in
// the one-launch pass the whole entry in scalar registers would spill them).
template <int KIND, bool SCALAR = false>
__device__ __forceinline__ MLin pick(const MRun &run, const MLin &single, const int32_t *map, int64_t item) {
    MLin m;
    if (run.table) {
        m = SCALAR ? table_at(run.table, (int64_t)table_at(map, item)) : run.table[map[item]];
    } else if (run.ninl) {
        // inline groups: the last linear starting at or before item (constant
        // indices only: a variable index into the kernel arguments would copy
        // them to scratch memory)
        m = run.inl[0];
        static_assert(kMaxInline == 3, "inline lookup");
        if (run.ninl > 1 && item >= item_start(run.inl[1], KIND)) m = run.inl[1];
        if (run.ninl > 2 && item >= item_start(run.inl[2], KIND)) m = run.inl[2];
    } else {
        m = single;
    }
    static_assert(sizeof(MLin) % 4 == 0, "MLin is copied as 32-bit words");
    int w[sizeof(MLin) / 4];
    __builtin_memcpy(w, &m, sizeof(MLin));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(MLin) / 4); ++i) w[i] = __builtin_amdgcn_readfirstlane(w[i]);
    __builtin_memcpy(&m, w, sizeof(MLin));
    return m;
}

// Index of the inline linear whose KIND items hold `item` (constant indices).
template <int KIND>
__device__ __forceinline__ int inline_index(const MRun &run, int64_t item) {
    int j = 0;
    if (run.ninl > 1 && item >= item_start(run.inl[1], KIND)) j = 1;
    if (run.ninl > 2 && item >= item_start(run.inl[2], KIND)) j = 2;
    return j;
}

// Linear j of the run as a wave-uniform value.
__device__ __forceinline__ MLin pick_linear(const MRun &run, const MLin &single, int j) {
    MLin m = single;
    if (run.table) {
        m = run.table[j];
    } else if (run.ninl) {                 // constant indices, as in pick
        m = run.inl[0];
        if (j == 1) m = run.inl[1];
        if (j == 2) m = run.inl[2];
    }
    int w[sizeof(MLin) / 4];
    __builtin_memcpy(w, &m, sizeof(MLin));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(MLin) / 4); ++i) w[i] = __builtin_amdgcn_readfirstlane(w[i]);
    __builtin_memcpy(&m, w, sizeof(MLin));
    return m;
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// The item a workgroup runs: launches of a group start their largest items
// first (ord), so the last workgroups to start are short ones.
template <bool SCALAR = false>
__device__ __forceinline__ int64_t item_of(const int32_t *ord, int64_t base) {
    const int64_t w = (int64_t)blockIdx.x + base;
    if (!ord) return w;
    return SCALAR ? (int64_t)table_at(ord, w) : (int64_t)__builtin_amdgcn_readfirstlane(ord[w]);
}

// silu(z) = z / (1 + exp(-z)); -0 for very negative z, no NaN for finite z
__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values as a bf16 pair (hardware conversion, round to nearest even).
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Outputs through a buffer descriptor.  A flat store is counted with the LDS
// operations as well, and after one the compiler can only wait for every load
// in flight; buffer stores keep the plane-load window counted precisely.
struct OutBuf {
    __amdgpu_buffer_rsrc_t r;
    int dtype;
    bool vec;       // rows come in whole, aligned groups of four: one vector store per lane
};

__device__ __forceinline__ OutBuf out_buf(void *y, int dtype, int64_t elems, int64_t d_out) {
    OutBuf o;
    const int eb = dtype == LB_BF16 ? 2 : 4;
    o.r = make_rsrc(y, elems * eb);
    o.dtype = dtype;
    o.vec = (d_out & 3) == 0 && ((uintptr_t)y & 15) == 0;
    return o;
}

// y[e0 .. e0+4) = v for the rows row .. row+3 that are < d_out (ok: this lane writes).
__device__ __forceinline__ void store4(const OutBuf &o, int64_t e0, int64_t row, int64_t d_out,
                                      const float (&v)[4], bool ok) {
    if (o.dtype == LB_BF16) {
        if (o.vec) {
            v2u w;
            w[0] = bf16_pair(v[0], v[1]);
            w[1] = bf16_pair(v[2], v[3]);
            __builtin_amdgcn_raw_buffer_store_b64(w, o.r, ok && row < d_out ? (uint32_t)(e0 * 2) : kOOB, 0, 0);
        } else {
#pragma unroll
            for (int q = 0; q < 4; q += 2) {
                const uint32_t w = bf16_pair(v[q], v[q + 1]);
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w & 0xffffu), o.r,
                                                      ok && row + q < d_out ? (uint32_t)((e0 + q) * 2) : kOOB, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w >> 16), o.r,
                                                      ok && row + q + 1 < d_out ? (uint32_t)((e0 + q + 1) * 2) : kOOB, 0, 0);
            }
        }
    } else {
        if (o.vec) {
            const v4u w = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
            __builtin_amdgcn_raw_buffer_store_b128(w, o.r, ok && row < d_out ? (uint32_t)(e0 * 4) : kOOB, 0, 0);
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[q]), o.r,
                                                      ok && row + q < d_out ? (uint32_t)((e0 + q) * 4) : kOOB, 0, 0);
        }
    }
}

// Compact operands [nops][R records] of src -> LDS operands at dst.  The first
// kPreVec vectors of each thread were loaded into pre[] before the caller's
// plane loads; any remainder is copied here.
template <int AUX = 0>
__device__ __forceinline__ void expand_ops(uint8_t *dst, const uint8_t *src, int nops, int R,
                                           const v4u (&pre)[kPreVec]) {
    const int vecs = nops * R * kRec / 16;
#pragma unroll
    for (int j = 0; j < kPreVec; ++j) {
        const int i = j * kThreads + (int)threadIdx.x;
        if (i < vecs) expand_vec(dst, i, R, pre[j]);
    }
    if (vecs <= kPreVec * kThreads) return;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, (int64_t)vecs * 16);
    for (int i = kPreVec * kThreads + (int)threadIdx.x; i < vecs; i += kThreads)
        expand_vec(dst, i, R, __builtin_amdgcn_raw_buffer_load_b128(r, i * 16, 0, AUX));
}

// Buffer loads (not flat ones: the compiler cannot count flat loads among the
// vector-memory operations in flight and would wait for all of them), issued
// unconditionally; vectors past the end read as zeros.
template <int AUX = 0>
__device__ __forceinline__ void preload_ops(const uint8_t *src, int nops, int R, v4u (&pre)[kPreVec]) {
    const int vecs = nops * R * kRec / 16;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, (int64_t)vecs * 16);
#pragma unroll
    for (int j = 0; j < kPreVec; ++j)
        pre[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (j * kThreads + (int)threadIdx.x) * 16, 0, AUX);
}

// Compact operands [nops][R records] of src -> the same bytes at dst (k_stage2r
// keeps the records as they are).  The first kPreVec vectors of each thread
// were loaded into pre[] before the caller's plane loads; any remainder is
// copied here.
template <int AUX = 0>
__device__ __forceinline__ void copy_ops(uint8_t *dst, const uint8_t *src, int nops, int R,
                                         const v4u (&pre)[kPreVec]) {
    const int vecs = nops * R * kRec / 16;
#pragma unroll
    for (int j = 0; j < kPreVec; ++j) {
        const int i = j * kThreads + (int)threadIdx.x;
        if (i < vecs) *(v4u *)(dst + i * 16) = pre[j];
    }
    if (vecs <= kPreVec * kThreads) return;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src, (int64_t)vecs * 16);
    for (int i = kPreVec * kThreads + (int)threadIdx.x; i < vecs; i += kThreads)
        *(v4u *)(dst + i * 16) = __builtin_amdgcn_raw_buffer_load_b128(r, i * 16, 0, AUX);
}

// LDS of k_stage2r's operands: `steps` K-groups of NB2 compact operands of R2
// records, then one zero record (read by the lanes of rows no token fills).
__host__ __device__ inline size_t ops2r_bytes(int steps, int NB2, int R2) {
    return ((size_t)steps * NB2 * R2 + 1) * kRec;
}

constexpr uint32_t kSpinLimit = 1u << 20;
constexpr uint32_t kSpinLimitTest = 64;   // under LB_GROUP_FAULT_TEST
constexpr int kFlagStride = 64;           // words between two linears' counters (own 256-byte lines)

}  // namespace

// The fault word of each device: kernels OR LB_FAULT_* bits into it, and
// lb_device_faults reads and clears it.  Library-owned, so a kernel can report
// even when the workspace it was given is not (or no longer) the group's.
__device__ uint32_t g_lb_faults;
__device__ uint32_t g_lb_faults_out;      // where lb_device_faults exchanges it to

namespace {

__device__ __forceinline__ void report_fault(uint32_t bit) {
    __hip_atomic_fetch_or(&g_lb_faults, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Whether a group's workspace no longer carries the stamp the group was set up
// with (the memory was reused or overwritten since).  Its tables are then not
// to be trusted: the workgroup reports it and does nothing.  Uniform.
__device__ __forceinline__ bool stale_ws(const MRun &run) {
    if (!run.stamp) return false;
    if (*run.stamp == run.tag) return false;
    if (threadIdx.x == 0) report_fault(LB_FAULT_STALE_WORKSPACE);
    return true;
}

// The wave polls the low 16 bits of *w (device scope) until they read `want`
// or `limit` polls have gone by; false (after reporting the fault) if it gave
// up.  Nothing after the poll may move above it: the operand loads that follow
// are device-scope loads issued after the poll's value has been compared.
__device__ __forceinline__ bool wait_count(const uint32_t *w, uint32_t want, uint32_t limit) {
    uint32_t n = 0;
    bool ok;
    while (!(ok = ((uint32_t)__builtin_amdgcn_readfirstlane(
                       __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) & 0xffffu) == want) &&
           ++n < limit)
        __builtin_amdgcn_s_sleep(2);
    asm volatile("" ::: "memory");
    if (!ok && (threadIdx.x & 63) == 0) report_fault(LB_FAULT_HANDOFF_TIMEOUT);
    return ok;
}

// One event of a linear's run in its sync word (`add` = 0x10001 for a latent
// group whose operands are stored, 0x10000 for a stage-2 workgroup past its
// wait).  A run has `events` of them; the one that completes the count is the
// run's last access to the word and sets it back to zero, so every run starts
// from zero and no run number is needed.
__device__ __forceinline__ void sync_event(uint32_t *w, uint32_t add, uint32_t events) {
    const uint32_t old = __hip_atomic_fetch_add(w, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((old >> 16) + 1u == events) __hip_atomic_store(w, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// prep: fp8 limbs of g_p (.) x as compact stage-1 operands
// ---------------------------------------------------------------------------

template <int NL, int NB1>
__global__ __launch_bounds__(kThreads) void k_prep(MRun run, MLin single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    if (stale_ws(run)) return;
    using R = Rows<NL>;
    const int64_t item = (int64_t)blockIdx.x + run.base0;
    const MLin L = pick<kKindPrep, true>(run, single, run.lin0, item);
    const int64_t local = item - L.item0;
    const int c = (int)(local % L.nprep);
    const int p = (int)(local / L.nprep);
    const int T = run.T;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int kg0 = c * L.kcp;
    const int nkg = (int)imin(L.kcp, L.kgv - kg0);
    const int opb = L.R1 * kRec;                          // bytes of one compact operand

    // half h of wave w takes 32-element blocks 2w+h, 2w+h+8, ...: its block
    // within a K-group, and so its byte offset in a record, never change
    const int h = lane >> 5, el = lane & 31;
    const int bq = (2 * wave + h) & 3;
    const int off_e = rec_offset(bq * 32 + el);
    const int blocks = nkg * 4;
    const int64_t i0 = (int64_t)kg0 * 128;
    const uint16_t *gp = L.g + (int64_t)p * L.d_in;
    constexpr int kPre = 8;
    for (int n = 0; n < T; ++n) {
        const int c0 = (n % R::TPM1) * R::S1;
        uint8_t *opn = smem + (n / R::TPM1) * opb + c0 * kRec;
        for (int b0 = 2 * wave; b0 < blocks; b0 += 8 * kPre) {
            // all loads first, from clamped (always valid) indices; the
            // products of elements past the chunk or past d_in are masked after
            float v[kPre];
            uint16_t gv[kPre];
            float xv[kPre];
            if (run.x_dtype == LB_BF16) {                        // uniform: one branch for all loads
                const uint16_t *xp = (const uint16_t *)L.x + (int64_t)n * L.d_in;
                const uint16_t *x2p = L.x2 ? (const uint16_t *)L.x2 + (int64_t)n * L.d_in : xp;
                uint16_t xb[kPre], x2b[kPre];
#pragma unroll
                for (int j = 0; j < kPre; ++j) {
                    const int64_t i = imin(i0 + (b0 + 8 * j + h) * 32 + el, L.d_in - 1);
                    gv[j] = gp[i];
                    xb[j] = xp[i];
                    x2b[j] = x2p[i];
                }
                if (L.x2) {                                       // SwiGLU input (uniform)
#pragma unroll
                    for (int j = 0; j < kPre; ++j) xv[j] = silu(bf16_to_f32(xb[j])) * bf16_to_f32(x2b[j]);
                } else {
#pragma unroll
                    for (int j = 0; j < kPre; ++j) xv[j] = bf16_to_f32(xb[j]);
                }
            } else {
                const float *xp = (const float *)L.x + (int64_t)n * L.d_in;
#pragma unroll
                for (int j = 0; j < kPre; ++j) {
                    const int64_t i = imin(i0 + (b0 + 8 * j + h) * 32 + el, L.d_in - 1);
                    gv[j] = gp[i];
                    xv[j] = xp[i];
                }
            }
            if (L.xs) {                                           // uniform
                const float sc = L.xs[n];
#pragma unroll
                for (int j = 0; j < kPre; ++j) xv[j] *= sc;
            }
#pragma unroll
            for (int j = 0; j < kPre; ++j) {
                const int blk = b0 + 8 * j + h;
                const int64_t i = i0 + blk * 32 + el;
                v[j] = (blk < blocks && i < L.d_in) ? f16_to_f32(gv[j]) * xv[j] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < kPre; ++j) {
                const int bw = b0 + 8 * j;                          // wave-uniform
                if (bw >= blocks) break;
                const int blk = bw + h;
                uint8_t *op = opn + (blk >> 2) * NB1 * opb;
                emit_limbs<NL>(v[j], op + off_e, op + 128 + bq, blk < blocks, el == 0);
            }
        }
    }
    __syncthreads();
    // operands of tokens < T only; records of unused rows are never read
    const int4 *src = (const int4 *)smem;
    int4 *dst = (int4 *)(L.pa + ((int64_t)p * L.kgv + kg0) * NB1 * opb);
    const int vecs = nkg * NB1 * opb / 16;
    for (int i = threadIdx.x; i < vecs; i += kThreads) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// stage 1: partial latent sums u = sign(V_p)^T (g_p (.) x) over one chunk
// ---------------------------------------------------------------------------

template <int NL, int NB1>
__global__ __launch_bounds__(kThreads) void k_stage1(MRun run, MLin single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    if (stale_ws(run)) return;
    using R = Rows<NL>;
    const int64_t item = item_of<true>(run.ord1, run.base1);
    const MLin L = pick<kKindStage1, true>(run, single, run.lin1, item);
    const int64_t local = item - L.item1;
    const int rg = (int)(local % L.nrg);
    const int c = (int)((local / L.nrg) % L.nchunks);
    const int p = (int)(local / ((int64_t)L.nrg * L.nchunks));
    const int T = run.T;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r16 = lane & 15, gq = lane >> 4;
    const Nib nib = nibble_constants();

    // operands first: loads complete in issue order, so the LDS fill below
    // then waits for these only, not for the plane loads
    const int kg0 = c * L.kcg;
    const int nkg = (int)imin(L.kcg, L.kgv - kg0);
    const uint8_t *opsrc = L.pa + ((int64_t)p * L.kgv + kg0) * NB1 * L.R1 * kRec;
    v4u pre[kPreVec];
    preload_ops(opsrc, nkg * NB1, L.R1, pre);

    // ---- V-plane loads of this wave's 64-latent tile ------------------------
    const int row0 = rg * kRG + wave * kTile;
    const int row = row0 + 4 * r16;
    const bool active = row0 < L.r_p;                            // wave-uniform
    // planes of this path only: planes past d_in read as zeros (their inputs are zero too)
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(L.v_bits + (int64_t)p * L.kw_v * L.ld_v, (int64_t)L.kw_v * L.ld_v * 4);
    const uint32_t vo = (uint32_t)(((int64_t)(kg0 * 4 + gq) * L.ld_v + row) * 4);
    const uint32_t vstep = (uint32_t)(4 * L.ld_v * 4);                 // one K-group of planes
    v4u w[kMaxKcg];
#pragma unroll
    for (int j = 0; j < kMaxKcg; ++j)
        w[j] = (active && j < nkg) ? load_rows(rv, vo + j * vstep) : v4u{0u, 0u, 0u, 0u};

    // Rows of tokens >= T stay unwritten: an MFMA row only feeds its own
    // accumulator row, which the epilogue never reads.
    expand_ops(smem, opsrc, nkg * NB1, L.R1, pre);
    __syncthreads();
    if (!active) return;

    v4f acc[4][NB1];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int b = 0; b < NB1; ++b) acc[m][b] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxKcg; ++j) {
        if (j >= nkg) continue;                                 // uniform; keeps w[] in registers
        const uint8_t *ops = smem + j * NB1 * kOpS;
        v8i ao[NB1];
        int sa[NB1];
#pragma unroll
        for (int b = 0; b < NB1; ++b) {
            ao[b] = load_op(ops + b * kOpS);
            sa[b] = ops[b * kOpS + kOp + lane];
        }
        v8i sgq[4];
        unpack_quad(w[j], nib, sgq);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const v8i sg = sgq[m];
#pragma unroll
            for (int b = 0; b < NB1; ++b) acc[m][b] = mfma(ao[b], sg, acc[m][b], sa[b]);
        }
    }

    // ---- partial latent sums: lane (gq, r16) holds latents row0+4*r16+m -------
    const int64_t Rtot = (int64_t)L.P * L.r_p;
    // whole aligned groups of 4 latents only when r_p is a multiple of 4:
    // otherwise the group crossing r_p would spill into the next path's latents
    const OutBuf ob = out_buf(L.part, LB_F32, (int64_t)L.nchunks * T * Rtot, L.r_p);
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
            store4(ob, ((int64_t)c * T + n) * Rtot + (int64_t)p * L.r_p + row, row, L.r_p, u, n < T);
        }
    }
}

// ---------------------------------------------------------------------------
// stage 1, fused form: all tokens in one activation-row block (T <= TPM1)
// ---------------------------------------------------------------------------

// LDS writes of this wave done, then every wave of the workgroup meets; loads
// in flight stay in flight (no vmcnt wait, unlike __syncthreads).
__device__ __forceinline__ void lds_meet() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// max over the four lanes of a quad (DPP quad permutations xor 1, xor 2)
__device__ __forceinline__ float quad_max(float m) {
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
    return m;
}

// fp32 products g (.) x of 8 consecutive inputs from their 16-byte pieces
__device__ __forceinline__ void gx8_bf16(const v4u &g, const v4u &x, float (&v)[8]) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t gw = g[t >> 1], xw = x[t >> 1];
        const float gf = f16_to_f32((uint16_t)((t & 1) ? gw >> 16 : gw & 0xffffu));
        v[t] = gf * __uint_as_float((t & 1) ? xw & 0xffff0000u : xw << 16);
    }
}
// The SwiGLU input: g (.) silu(xg) (.) xu of 8 consecutive inputs (bf16 xg, xu)
__device__ __forceinline__ void gx8_glu(const v4u &g, const v4u &xg, const v4u &xu, float (&v)[8]) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t gw = g[t >> 1], aw = xg[t >> 1], bw = xu[t >> 1];
        const float gf = f16_to_f32((uint16_t)((t & 1) ? gw >> 16 : gw & 0xffffu));
        const float a = __uint_as_float((t & 1) ? aw & 0xffff0000u : aw << 16);
        const float b = __uint_as_float((t & 1) ? bw & 0xffff0000u : bw << 16);
        v[t] = gf * (silu(a) * b);
    }
}
__device__ __forceinline__ void gx8_f32(const v4u &g, const v4u &x0, const v4u &x1, float (&v)[8]) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const uint32_t gw = g[t >> 1];
        const float gf = f16_to_f32((uint16_t)((t & 1) ? gw >> 16 : gw & 0xffffu));
        v[t] = gf * __uint_as_float(t < 4 ? x0[t] : x1[t - 4]);
    }
}

// The NL limbs of one 8-input piece into compact records (same arithmetic as
// emit_limbs; the 32-input block is the lane's quad).  Piece a (0..3) of block
// gb (0..3) of a K-group: inputs t and t + 4 land in adjacent record bytes, at
// 64(gb&1) + 16(gb>>1) + 2a + {0, 8, 32, 40}[t] (rec_offset for 8a+t, 8a+t+4).
// rec0 points at the record of limb 0; limb q is q*kRec further.
template <int NL>
__device__ __forceinline__ void emit_piece(const float (&v)[8], uint8_t *rec0, int gb, int a, bool ok) {
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) m = fmaxf(m, fabsf(v[t]));
    m = quad_max(m);
    const int E = (int)((__float_as_uint(m) >> 23) & 0xff) - 127;
    float r[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = v[t];
    const int base = ((gb & 1) << 6) + ((gb >> 1) << 4) + 2 * a;
#pragma unroll
    for (int q = 0; q < NL; ++q) {
        const int eq = E - 7 - 4 * q;
        uint8_t *d = rec0 + q * kRec;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t b = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexp2(r[t], -eq), ldexp2(r[t + 4], -eq), 0, false);
            if (ok) *(uint16_t *)(d + base + ((t >> 1) << 5) + ((t & 1) << 3)) = (uint16_t)b;
            if (q + 1 < NL) {
                r[t] -= ldexp2(__builtin_amdgcn_cvt_f32_fp8((int)b, 0), eq);
                r[t + 4] -= ldexp2(__builtin_amdgcn_cvt_f32_fp8((int)b, 1), eq);
            }
        }
        if (ok && a == 0) d[128 + gb] = (uint8_t)(eq < -127 ? 0 : (eq > 127 ? 254 : eq + 127));
    }
}

// Item = (linear, path, chunk of up to kMaxKcf K-groups of d_in).  The
// workgroup turns g_p (.) x over its chunk into compact limb records in LDS
// (g and token 0 of x are loaded first), then each wave streams its share of
// the item's (tile, K-group) pairs with kWin1 plane loads in flight (rotating
// register slots, as k_stage2r).  Two ways to share them (run.tsplit):
//   - K split: wave w takes K-groups [w*sub, (w+1)*sub) of the chunk across
//     every 64-latent tile of the item; at the end the four waves' partial
//     sums meet in LDS and are added in wave order.  It keeps all four waves
//     busy with any number of tiles, but the partials take [F][kWaves][T][64]
//     floats of LDS.
//   - tile split: wave w takes tiles w, w+4, ... of the item across every
//     K-group of the chunk, so each latent has one wave and the partials need
//     [F][T][64] floats: with more tokens an item still covers many tiles.
// Either way one partial per (chunk, token, latent), in a fixed summation
// order.
// COHERENT: the partial sums are read back inside the same launch by another
// workgroup (the one-launch pass), so they are stored at device scope.
template <int NL, bool COHERENT, bool XM = false>
__device__ __forceinline__ void stage1f_item(const MRun &run, const MLin &L, int64_t item, uint8_t *smem) {
    using R = Rows<NL>;
    const int64_t local = item - L.item1;
    const int c = (int)(local % L.nchunks);
    const int rg = (int)((local / L.nchunks) % L.nrg);
    const int p = (int)(local / ((int64_t)L.nchunks * L.nrg));
    const int T = run.T;
    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = wave_id();
    const int r16 = lane & 15, gq = lane >> 4;
    const Nib nib = nibble_constants();
    const int kg0 = c * L.kcg;
    const int nkg = (int)imin(L.kcg, L.kgv - kg0);
    const int R1 = L.R1;
    uint8_t *recs = smem;                                               // [nkg][R1] records
    float *red = (float *)(smem + (size_t)L.kcg * R1 * kRec);          // [F][kWaves][T][64]

    // ---- g and token-0 x of this thread's pieces (8 inputs each) -------------
    constexpr int kPPT = kMaxKcf * 16 / kThreads;                      // pieces per thread
    const int npc = nkg * 16;
    const int64_t i_chunk = (int64_t)kg0 * 128;
    const bool xf32 = run.x_dtype == LB_F32;
    const int xb = xf32 ? 4 : 2;
    const bool vec = L.xvec != 0;
    const bool glu = L.x2 != nullptr;                                  // SwiGLU input (bf16 x only)
    const __amdgpu_buffer_rsrc_t rgs = make_rsrc(L.g + (int64_t)p * L.d_in, L.d_in * 2);
    // the input map (uniform): channel i of the linear's input is channel
    // xoff(i) of a row of x, rows dsrc apart
    // (instantiated apart (XM), so the plain form keeps its registers)
    const int64_t dsrc = XM ? L.d_in / L.xm_grp : L.d_in;
    auto xoff = [&](int64_t i) -> int64_t {
        if constexpr (!XM) return i;
        const uint32_t h = (uint32_t)i / (uint32_t)L.xm_dh;
        return (int64_t)(h / (uint32_t)L.xm_grp) * L.xm_dh + ((uint32_t)i - h * (uint32_t)L.xm_dh);
    };
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(L.x, (int64_t)T * dsrc * xb);
    // second piece of each input: the high half of fp32 x, or the up input x2
    const __amdgpu_buffer_rsrc_t rx2 = make_rsrc(glu ? L.x2 : L.x, (int64_t)T * dsrc * xb);
    auto second = [&](bool ok, int64_t e) -> uint32_t {         // byte offset of element e's second piece
        return ok && (xf32 || glu) ? (uint32_t)(xf32 ? e * 4 + 16 : e * 2) : kOOB;
    };
    v4u gr[kPPT], xr[kPPT][2];
#pragma unroll
    for (int j = 0; j < kPPT; ++j) {
        const int pc = tid + j * kThreads;
        const int64_t i = i_chunk + (int64_t)pc * 8;
        const bool ok = vec && pc < npc && i < L.d_in;
        const int64_t xi = xoff(i);
        gr[j] = __builtin_amdgcn_raw_buffer_load_b128(rgs, ok ? (uint32_t)(i * 2) : kOOB, 0, 0);
        xr[j][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? (uint32_t)(xi * xb) : kOOB, 0, 0);
        xr[j][1] = __builtin_amdgcn_raw_buffer_load_b128(rx2, second(ok, xi), 0, 0);
    }

    // ---- first plane loads ----------------------------------------------------
    const bool ts = run.tsplit != 0;
    const int sub = (L.kcg + kWaves - 1) / kWaves;
    const int ka = ts ? 0 : wave * sub;                                // chunk-local K-group
    const int nk = ts ? nkg : (int)imax(0, imin(sub, nkg - ka));
    const int tile0 = rg * run.flush1;                                 // first 64-latent tile of the item
    const int ntile = (int)imin(run.flush1, cdiv(L.r_p, kTile) - tile0);
    // this wave's tiles of the item: tf, tf + tstep, ... (wt of them)
    const int tf = ts ? wave : 0, tstep = ts ? kWaves : 1;
    const int wt = ts ? (ntile > wave ? (int)cdiv(ntile - wave, kWaves) : 0) : ntile;
    const int total = wt * nk;
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(L.v_bits + (int64_t)p * L.kw_v * L.ld_v, (int64_t)L.kw_v * L.ld_v * 4);
    const uint32_t vo =
        (uint32_t)(((int64_t)((kg0 + ka) * 4 + gq) * L.ld_v + (tile0 + tf) * kTile + 4 * r16) * 4);
    const uint32_t group4 = (uint32_t)(4 * L.ld_v * 4);
    // next (tile, K-group) to load; selects only, so every load is issued
    // on every path and the compiler can count them
    const int ltiles = nk > 0 ? wt : 0;
    int lt = 0, lk = 0;
    auto next_off = [&]() -> uint32_t {
        const bool live = lt < ltiles && (tile0 + tf + lt * tstep) * kTile + 4 * r16 < L.r_p;
        const uint32_t o = live ? vo + (uint32_t)(lt * tstep * kTile * 4) + (uint32_t)lk * group4 : kOOB;
        const bool wrap = lk + 1 == nk;
        lt = wrap ? lt + 1 : lt;
        lk = wrap ? 0 : lk + 1;
        return o;
    };
    // The standalone kernel issues its first plane loads now, so their latency
    // overlaps the limb work below.  Inside the one-launch pass only kEarly1
    // go out now and the rest after it: all of them held through the limb work
    // would take 32 more registers, and the pass, which holds stage 2 as well,
    // would fit one workgroup less per CU.
    constexpr int early = COHERENT ? kEarly1 : kWin1;
    v4u slot[kWin1];
#pragma unroll
    for (int k = 0; k < early; ++k) slot[k] = load_rows(rv, next_off());

    // ---- limbs of g (.) x into the records ------------------------------------
    // piece pc: K-group pc/16 of the chunk, block (pc/4)%4, quarter pc%4; a
    // quad of lanes holds one 32-input block
    auto rec_of = [&](int pc, int n) { return recs + ((size_t)(pc >> 4) * R1 + n * R::S1) * kRec; };
    if (vec) {
#pragma unroll
        for (int j = 0; j < kPPT; ++j) {                        // token 0 from the preloads
            const int pc = tid + j * kThreads;
            float v[8];
            if (xf32) gx8_f32(gr[j], xr[j][0], xr[j][1], v);
            else if (glu) gx8_glu(gr[j], xr[j][0], xr[j][1], v);
            else gx8_bf16(gr[j], xr[j][0], v);
            if (L.xs) {                                         // uniform
                const float sc = L.xs[0];
#pragma unroll
                for (int t = 0; t < 8; ++t) v[t] *= sc;
            }
            emit_piece<NL>(v, rec_of(pc, 0), (pc >> 2) & 3, pc & 3, pc < npc);
        }
        // the other tokens kTB at a time, all of a round's loads in flight
        // together (one load latency per round, not one per token)
        constexpr int TB = COHERENT ? 1 : kTB;   // the pass: T <= 2, registers kept for stage 2
        for (int n0 = 1; n0 < T; n0 += TB) {
            v4u xa[TB][kPPT][2];
#pragma unroll
            for (int u = 0; u < TB; ++u)
#pragma unroll
                for (int j = 0; j < kPPT; ++j) {
                    const int pc = tid + j * kThreads;
                    const int64_t i = i_chunk + (int64_t)pc * 8;
                    const bool in = n0 + u < T && pc < npc && i < L.d_in;
                    const int64_t e = (int64_t)(n0 + u) * dsrc + xoff(i);
                    xa[u][j][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? (uint32_t)(e * xb) : kOOB, 0, 0);
                    xa[u][j][1] = __builtin_amdgcn_raw_buffer_load_b128(rx2, second(in, e), 0, 0);
                }
#pragma unroll
            for (int u = 0; u < TB; ++u) {
                const int n = n0 + u;
                if (n >= T) break;                                  // uniform
#pragma unroll
                for (int j = 0; j < kPPT; ++j) {
                    const int pc = tid + j * kThreads;
                    float v[8];
                    if (xf32) gx8_f32(gr[j], xa[u][j][0], xa[u][j][1], v);
                    else if (glu) gx8_glu(gr[j], xa[u][j][0], xa[u][j][1], v);
                    else gx8_bf16(gr[j], xa[u][j][0], v);
                    if (L.xs) {                                     // uniform
                        const float sc = L.xs[n];
#pragma unroll
                        for (int t = 0; t < 8; ++t) v[t] *= sc;
                    }
                    emit_piece<NL>(v, rec_of(pc, n), (pc >> 2) & 3, pc & 3, pc < npc);
                }
            }
        }
    } else {                                                    // ragged or unaligned: input by input
        for (int n = 0; n < T; ++n) {
#pragma unroll
            for (int j = 0; j < kPPT; ++j) {
                const int pc = tid + j * kThreads;
                const int64_t i = i_chunk + (int64_t)pc * 8;
                float v[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const bool in = pc < npc && i + t < L.d_in;
                    const uint32_t go = in ? (uint32_t)((i + t) * 2) : kOOB;
                    const uint32_t xo = in ? (uint32_t)(((int64_t)n * dsrc + xoff(i + t)) * xb) : kOOB;
                    const float gf = f16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rgs, go, 0, 0));
                    float xf = xf32 ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx, xo, 0, 0))
                                    : bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rx, xo, 0, 0));
                    if (glu) xf = silu(xf) * bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rx2, xo, 0, 0));
                    v[t] = gf * xf;
                    if (L.xs) v[t] *= L.xs[n];
                }
                emit_piece<NL>(v, rec_of(pc, n), (pc >> 2) & 3, pc & 3, pc < npc);
            }
        }
    }
    lds_meet();

    // ---- stream ------------------------------------------------------------
#pragma unroll
    for (int k = early; k < kWin1; ++k) slot[k] = load_rows(rv, next_off());
    v4f acc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
    const int rr = r16 < R1 ? r16 : R1 - 1;       // rows past R1 repeat the last one (never read out)
    const int64_t Rtot = (int64_t)L.P * L.r_p;
    // partial sums through a buffer descriptor: a flat store would be counted
    // with the LDS operations too, and every later wait would become a full one
    const __amdgpu_buffer_rsrc_t rpart = make_rsrc(L.part, (int64_t)L.nchunks * T * Rtot * 4);
    // The wave's t-th tile done: its partials go to their LDS slot, with no wait.
    auto tile_end = [&](int t) {
        float *mine = red + ((size_t)(ts ? tf + t * tstep : t * kWaves + wave) * T) * 64;
#pragma unroll
        for (int s = 0; s < 4 / R::S1; ++s) {
            const int n = gq * (4 / R::S1) + s;
            v4f u;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                float sum = 0.0f;
#pragma unroll
                for (int q = 0; q < NL; ++q) sum += acc[m][s * R::S1 + q];
                u[m] = sum;
            }
            if (n < T) *(v4f *)(mine + n * 64 + 4 * r16) = u;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
    };
    int pk = 0, pt = 0;
    // this lane's operand quarter and scale in the record of row rr; records of
    // successive K-groups are R1 * kRec bytes apart (a scalar step)
    const uint8_t *rec_a = recs + (size_t)rr * kRec + gq * 32;
    const uint8_t *rec_s = recs + (size_t)rr * kRec + 128 + gq;
    const int rec_step = R1 * kRec;
    auto process = [&](const v4u &w) {
        const int ro = (ka + pk) * rec_step;
        const v8i ao = load_op_at(rec_a + ro);
        const int sa = rec_s[ro];
        v8i sgq[4];
        unpack_quad(w, nib, sgq);
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[m] = mfma(ao, sgq[m], acc[m], sa);
        if (++pk == nk) {
            tile_end(pt);
            pk = 0;
            ++pt;
        }
    };
    for (int e0 = 0; e0 < total; e0 += kWin1) {
#pragma unroll
        for (int k = 0; k < kWin1; ++k) {
            if (e0 + k < total) process(slot[k]);                 // uniform
            slot[k] = load_rows(rv, next_off());
        }
    }
    if (nk == 0 && !ts)
        for (int t = 0; t < ntile; ++t) tile_end(t);                  // zeros

    // every wave's partials in LDS: add them in wave order (K split), write
    // row-contiguous
    lds_meet();
    const int per = T * 64;                                           // floats of one wave's tile
    for (int f = tid; f < ntile * per; f += kThreads) {
        const int k = f / per, rem = f - k * per;
        const int n = rem >> 6, row = (tile0 + k) * kTile + (rem & 63);
        const float *q = red + (size_t)k * (ts ? 1 : kWaves) * per + rem;
        const float sum = ts ? q[0] : ((q[0] + q[per]) + q[2 * per]) + q[3 * per];
        const uint32_t po = (uint32_t)((((int64_t)c * T + n) * Rtot + (int64_t)p * L.r_p + row) * 4);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), rpart, row < L.r_p ? po : kOOB, 0,
                                              COHERENT ? kDeviceScope : 0);
    }
}

template <int NL, bool XM = false>
__global__ __launch_bounds__(kThreads) void k_stage1f(MRun run, MLin single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    if (stale_ws(run)) return;
    const int64_t item = item_of<true>(run.ord1, run.base1);
    stage1f_item<NL, false, XM>(run, pick<kKindStage1, true>(run, single, run.lin1, item), item, smem);
}

// ---------------------------------------------------------------------------
// latents: t = l (.) sum over chunks, as compact stage-2 operands
// ---------------------------------------------------------------------------

// K-groups kg_first .. kg_first+kg_count-1 of a linear's stage-2 operands.
// Lanes map to (unit = token x plane of 32 latents, latent); each lane
// gathers the chunk partials of up to kLU units at once.  A latent sums its
// partials slice by slice: the kLC chunks of a slice are loaded together (all
// in flight: unconditional buffer loads, chunks past the end read as zeros)
// and added in chunk order from zero, and the slice sums in slice order from
// zero.
constexpr int kLU = 4, kLC = 8;   // units per lane, chunks per slice
template <int NL, int NB2>
__device__ __forceinline__ void latent_item(const MRun &run, const MLin &L, int kg_first, int kg_count,
                                            uint8_t *smem) {
    using R = Rows<NL>;
    const int T = run.T;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int opb = L.R2 * kRec;
    const int opsz = kg_count * NB2 * opb;                        // bytes of the staged operands
    // every row of these operands that no (token, path, limb) fills reads as zero
    {
        uint32_t *w = (uint32_t *)smem;
        for (int i = threadIdx.x; i < opsz / 4; i += kThreads) w[i] = 0u;
    }
    __syncthreads();
    const int64_t Rtot = (int64_t)L.P * L.r_p;
    const int blocks = kg_count * 4;                              // planes, one path each
    const int units = T * blocks;
    const int64_t cs = (int64_t)T * Rtot;                         // floats per chunk
    const int ns = (int)cdiv(L.nchunks, kLC);                     // slices
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(L.part, (int64_t)L.nchunks * cs * 4);
    constexpr int step = 2 * kWaves;                              // wave halves of the workgroup
    for (int ub = 2 * wave; ub < units; ub += step * kLU) {      // uniform per wave
        uint32_t base[kLU];
        bool live[kLU];
#pragma unroll
        for (int q = 0; q < kLU; ++q) {
            const int u = ub + q * step + (lane >> 5);
            const bool ok = u < units;
            const int n = ok ? u / blocks : 0;
            const int pl = kg_first * 4 + (ok ? u % blocks : 0);  // plane over both paths
            const int p = pl / L.kw_u;                            // uniform per wave half
            const int k = (pl - p * L.kw_u) * 32 + (lane & 31);   // latent of path p
            live[q] = ok && p < L.P && k < L.r_p;
            base[q] = live[q] ? (uint32_t)(((int64_t)n * Rtot + (int64_t)p * L.r_p + k) * 4) : 0u;
        }
        float sum[kLU];
#pragma unroll
        for (int q = 0; q < kLU; ++q) sum[q] = 0.0f;
        for (int sl = 0; sl < (run.t_mode == 2 ? 0 : ns); ++sl) {   // uniform
            float a[kLU][kLC];
#pragma unroll
            for (int q = 0; q < kLU; ++q)
#pragma unroll
                for (int t = 0; t < kLC; ++t) {
                    const int c = sl * kLC + t;
                    a[q][t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        rp, live[q] && c < L.nchunks ? base[q] + (uint32_t)((int64_t)c * cs * 4) : kOOB, 0, 0));
                }
#pragma unroll
            for (int q = 0; q < kLU; ++q) {
                float x = 0.0f;
#pragma unroll
                for (int t = 0; t < kLC; ++t) x += a[q][t];
                sum[q] += x;
            }
        }
#pragma unroll
        for (int q = 0; q < kLU; ++q) {
            const int u = ub + q * step + (lane >> 5);
            const bool ok = u < units;
            const int n = ok ? u / blocks : 0;
            const int blk = ok ? u % blocks : 0;
            const int e = blk * 32 + (lane & 31);                 // element in the K-group range
            const int pl = kg_first * 4 + blk;
            const int p = pl / L.kw_u;
            const int k = (pl - p * L.kw_u) * 32 + (lane & 31);
            float v;
            if (run.t_mode == 2) {                                // latents given (uniform)
                const int64_t ti = (int64_t)n * Rtot + (int64_t)p * L.r_p + k;
                v = !live[q] ? 0.0f
                    : run.t_dtype == LB_F32 ? ((const float *)run.t_io)[ti]
                                            : bf16_to_f32(((const uint16_t *)run.t_io)[ti]);
            } else {
                v = live[q] ? f16_to_f32(L.l[(int64_t)p * L.r_p + k]) * sum[q] : 0.0f;
                if (run.t_mode == 1 && live[q]) {                 // latents out, as computed
                    const int64_t ti = (int64_t)n * Rtot + (int64_t)p * L.r_p + k;
                    if (run.t_dtype == LB_F32) ((float *)run.t_io)[ti] = v;
                    else ((uint16_t *)run.t_io)[ti] = f32_to_bf16(v);
                }
            }
            const int row = (n % R::TPM2) * R::S2 + (p < L.P ? p : 0) * NL;
            uint8_t *op = smem + ((e >> 7) * NB2 + n / R::TPM2) * opb + row * kRec;
            emit_limbs<NL>(v, op + rec_offset(e & 127), op + 128 + ((e & 127) >> 5), ok && p < L.P,
                           (e & 31) == 0);
        }
    }
    __syncthreads();
    const v4u *src = (const v4u *)smem;
    const int vecs = opsz / 16;
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(L.tb + (int64_t)kg_first * NB2 * opb, (int64_t)vecs * 16);
    for (int i = threadIdx.x; i < vecs; i += kThreads)
        __builtin_amdgcn_raw_buffer_store_b128(src[i], rt, i * 16, 0, 0);
}

// The one-launch pass: the latents of one stage-1 latent group (path p,
// 64-latent tiles [rg*F, (rg+1)*F), F = run.flush1) for every token, summed
// as latent_item sums them.  Each (token, 32-latent plane) is staged in LDS as
// NL records, of which only the plane's 32 bytes and its scale byte are
// stored: the stage-2 records' other planes belong to other groups, and rows
// no (token, path, limb) fills stay as the workspace set-up left them (zero).
// The partial sums come from other workgroups of the launch and the operands
// go to others, so both are accessed at device scope.
template <int NL, int NB2>
__device__ __forceinline__ void latent_rows(const MRun &run, const MLin &L, int p, int rg, uint8_t *smem) {
    using R = Rows<NL>;
    const int T = run.T;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int pl0 = rg * run.flush1 * 2;                          // first plane of the group (path p)
    const int npl = (int)imin(run.flush1 * 2, L.kw_u - pl0);
    const int units = T * npl;                                    // (token, plane), token-major
    const int64_t Rtot = (int64_t)L.P * L.r_p;
    const int64_t cs = (int64_t)T * Rtot;                         // floats per chunk
    const int ns = (int)cdiv(L.nchunks, kLC);                     // slices
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(L.part, (int64_t)L.nchunks * cs * 4);
    constexpr int step = 2 * kWaves;                              // wave halves of the workgroup
    for (int ub = 2 * wave; ub < units; ub += step * kLU) {      // uniform per wave
        uint32_t base[kLU];
        bool live[kLU];
#pragma unroll
        for (int q = 0; q < kLU; ++q) {
            const int u = ub + q * step + (lane >> 5);
            const bool ok = u < units;
            const int n = ok ? u / npl : 0;
            const int k = (pl0 + (ok ? u % npl : 0)) * 32 + (lane & 31);   // latent of path p
            live[q] = ok && k < L.r_p;
            base[q] = live[q] ? (uint32_t)(((int64_t)n * Rtot + (int64_t)p * L.r_p + k) * 4) : 0u;
        }
        float sum[kLU];
#pragma unroll
        for (int q = 0; q < kLU; ++q) sum[q] = 0.0f;
        for (int sl = 0; sl < ns; ++sl) {                         // uniform
            float a[kLU][kLC];
#pragma unroll
            for (int q = 0; q < kLU; ++q)
#pragma unroll
                for (int t = 0; t < kLC; ++t) {
                    const int c = sl * kLC + t;
                    a[q][t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        rp, live[q] && c < L.nchunks ? base[q] + (uint32_t)((int64_t)c * cs * 4) : kOOB, 0,
                        kDeviceScope));
                }
#pragma unroll
            for (int q = 0; q < kLU; ++q) {
                float x = 0.0f;
#pragma unroll
                for (int t = 0; t < kLC; ++t) x += a[q][t];
                sum[q] += x;
            }
        }
#pragma unroll
        for (int q = 0; q < kLU; ++q) {
            const int u = ub + q * step + (lane >> 5);
            const bool ok = u < units;
            const int pl = pl0 + (ok ? u % npl : 0);
            const int k = pl * 32 + (lane & 31);
            const float v = live[q] ? f16_to_f32(L.l[(int64_t)p * L.r_p + k]) * sum[q] : 0.0f;
            const int e = ((p * L.kw_u + pl) & 3) * 32 + (lane & 31);   // element in the K-group
            uint8_t *rec = smem + (size_t)(ok ? u : 0) * NL * kRec;
            emit_limbs<NL>(v, rec + rec_offset(e), rec + 128 + (e >> 5), ok, (e & 31) == 0);
        }
    }
    __syncthreads();
    // (unit, limb, 16-byte half) -> its place in the stage-2 records
    const int opb = L.R2 * kRec;
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(L.tb, (int64_t)L.kgs * NB2 * opb);
    for (int i = threadIdx.x; i < units * NL * 2; i += kThreads) {
        const int u = i / (NL * 2), q = (i >> 1) % NL, h = i & 1;
        const int n = u / npl, gp = p * L.kw_u + pl0 + u % npl;  // plane over both paths
        const int row = (n % R::TPM2) * R::S2 + p * NL + q;
        // block b of a record: bytes [16 * (b >> 1) + 64 * (b & 1), +16) and 32 further (rec_offset)
        const int blk = ((gp & 3) >> 1) * 16 + ((gp & 3) & 1) * 64 + h * 32;
        const uint32_t dst = (uint32_t)((((gp >> 2) * NB2 + n / R::TPM2) * L.R2 + row) * kRec + blk);
        const v4u w = *(const v4u *)(smem + (size_t)(u * NL + q) * kRec + blk);
        __builtin_amdgcn_raw_buffer_store_b128(w, rt, dst, 0, kDeviceScope);
    }
    for (int i = threadIdx.x; i < units * NL; i += kThreads) {
        const int u = i / NL, q = i % NL;
        const int n = u / npl, gp = p * L.kw_u + pl0 + u % npl;
        const int row = (n % R::TPM2) * R::S2 + p * NL + q;
        const uint32_t dst = (uint32_t)((((gp >> 2) * NB2 + n / R::TPM2) * L.R2 + row) * kRec + 128 + (gp & 3));
        __builtin_amdgcn_raw_buffer_store_b8(smem[(size_t)(u * NL + q) * kRec + 128 + (gp & 3)], rt, dst, 0,
                                             kDeviceScope);
    }
}

template <int NL, int NB2>
__global__ __launch_bounds__(kThreads) void k_latent(MRun run, MLin single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    if (stale_ws(run)) return;
    const int64_t item = (int64_t)blockIdx.x + run.baseF;
    const MLin L = pick<kKindLatent, true>(run, single, run.linF, item);
    const int kg_first = (int)(item - L.itemF) * 2;               // 2 K-groups = 8 planes per item
    latent_item<NL, NB2>(run, L, kg_first, (int)imin(2, L.kgs - kg_first), smem);
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
    if (stale_ws(run)) return;
    using R = Rows<NL>;
    const int64_t item = item_of<true>(run.ord2, run.base2);
    const MLin L = pick<kKindStage2, true>(run, single, run.lin2, item);
    const int64_t local = item - L.item2;
    const int T = run.T;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r16 = lane & 15, gq = lane >> 4;
    const Nib nib = nibble_constants();

    // K-groups run over the U planes of all paths back to back, so a group may
    // hold the last planes of path 0 and the first of path 1: each path's
    // activation rows are zero outside its own planes
    const int steps = L.kgs;
    const int ops = run.ops2;                      // steps the LDS holds (a multiple of kBatch when < steps)
    const bool fits = steps <= ops;
    const int nbat = (int)cdiv(steps, kBatch);     // batches per tile
    const int64_t row_begin = local * L.rows2;
    const int tiles = (int)imin(L.rows2 / kRG, cdiv(L.d_out - row_begin, kRG));
    const int units = tiles * nbat;
    const int opb = L.R2 * kRec;
    const OutBuf ob = out_buf(L.y, run.y_dtype, (int64_t)T * L.d_out, L.d_out);

    // operands first (loads complete in issue order)
    v4u pre[kPreVec];
    if (fits) preload_ops(L.tb, steps * NB2, L.R2, pre);

    // all U planes of the linear; rows and planes past the end read as zeros
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(L.u_bits, (int64_t)L.P * L.kw_u * L.ld_u * 4);
    const uint32_t uo = (uint32_t)(((int64_t)gq * L.ld_u + wave * kTile + 4 * r16) * 4);
    const uint32_t group4 = (uint32_t)(4 * L.ld_u * 4);            // bytes of one K-group of planes
    auto issue = [&](v4u (&w)[kBatch], int t, int b) {
        const uint32_t base = uo + (uint32_t)((row_begin + (int64_t)t * kRG) * 4) +
                              (uint32_t)(b * kBatch) * group4;
#pragma unroll
        for (int j = 0; j < kBatch; ++j)
            w[j] = b * kBatch + j < steps ? load_rows(ru, base + j * group4) : v4u{0u, 0u, 0u, 0u};
    };

    v4f acc[4][NB2];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int b = 0; b < NB2; ++b) acc[m][b] = v4f{0.f, 0.f, 0.f, 0.f};

    v4u wc[kBatch];
    issue(wc, 0, 0);
    if (fits) expand_ops(smem, L.tb, steps * NB2, L.R2, pre);
    int t = 0, bt = 0;                              // unit in flight
    for (int u = 0; u < units; ++u) {
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
        const int tn = last ? t + 1 : t, bn = last ? 0 : bt + 1;
        if (u + 1 < units) issue(wn, tn, bn);
        if (!fits && (bt * kBatch) % ops == 0) {   // next chunk of operands
            const int s0 = bt * kBatch;
            const int ns = (int)imin(ops, steps - s0);
            __syncthreads();
            const uint8_t *src = L.tb + (int64_t)s0 * NB2 * opb;
            const int vecs = ns * NB2 * opb / 16;
            for (int i = threadIdx.x; i < vecs; i += kThreads)
                expand_vec(smem, i, L.R2, ((const v4u *)src)[i]);
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
            v8i sgq[4];
            unpack_quad(wc[j], nib, sgq);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const v8i sg = sgq[m];
#pragma unroll
                for (int b = 0; b < NB2; ++b) acc[m][b] = mfma(ao[b], sg, acc[m][b], sa[b]);
            }
        }
        if (last) {
            // y = sum_p h_p z_p: lane (gq, r16) holds activation rows 4gq..4gq+3
            // of weight rows row+m; S2 = 4 puts one token's p0/p1 limbs there,
            // S2 = 8 splits them over lane groups gq and gq^1.  Both paths add
            // their limbs in the same order (limb 0 first).
#pragma unroll
            for (int b = 0; b < NB2; ++b) {
                float y4[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const v4f a = acc[m][b];
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
                if (L.resid && writer) {                        // (uniform pointer) the residual
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        if (row + m < L.d_out) y4[m] += load_act(L.resid, run.y_dtype, (int64_t)n * L.d_out + row + m);
                }
                store4(ob, (int64_t)n * L.d_out + row, row, L.d_out, y4, writer);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int b = 0; b < NB2; ++b) acc[m][b] = v4f{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) wc[j] = wn[j];
        t = tn;
        bt = bn;
    }
}

// Stage 2, streaming form: each wave walks its (tile, K-group) sequence with
// kWin2 plane loads in flight in a rotating set of registers: slot k is
// consumed and immediately reloaded with the element kWin2 further on, so no
// register is copied and no wait other than the one for the oldest load is
// needed.  Loads are unconditional (offsets past the range read zeros).  The
// operands of all steps (the compact records as the workspace holds them, plus
// a zero record for the rows no token fills) and h of the item's rows sit in
// LDS for the whole item.
// COHERENT: the operands were written earlier in the same launch (the
// one-launch pass); the low half of the linear's `sync` word counts its latent
// groups whose operands are stored.  Each wave loads it (device scope) as its
// first load, then h and its first plane loads; the check waits for the
// counter load alone (loads complete in issue order for the counter), and only
// then do the operand loads go out, at device scope.  Once all four waves are
// past the check, the workgroup counts itself in the high half (see k_pass).
template <int NL, int NB2, bool COHERENT>
__device__ __forceinline__ void stage2r_item(const MRun &run, const MLin &L, int64_t row_begin, int tiles,
                                             uint8_t *smem, uint32_t *sync) {
    using R = Rows<NL>;
    const int T = run.T;
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int r16 = lane & 15, gq = lane >> 4;
    const Nib nib = nibble_constants();

    const int steps = L.kgs;                       // K-groups over both paths' planes
    const int total = tiles * steps;               // this wave's stream (uniform)
    const OutBuf ob = out_buf(L.y, run.y_dtype, (int64_t)T * L.d_out, L.d_out);
    const int R2 = L.R2;
    uint8_t *ops = smem;                                          // [steps][NB2][R2] records
    uint8_t *zrec = ops + (size_t)steps * NB2 * R2 * kRec;        // the zero record
    uint16_t *hs = (uint16_t *)(smem + ops2r_bytes(run.ops2, NB2, R2));   // [2][kHRows] fp16 h
    // [T][kHRows] outputs of the item (bf16 or fp32): stores inside the stream
    // would share the in-order counter with the plane loads, so every later
    // wait would also wait for their acknowledgements
    uint8_t *ys = (uint8_t *)(hs + 2 * kHRows);
    const int yb = run.y_dtype == LB_BF16 ? 2 : 4;
    const int ysb = run.yst;                                      // bytes per collected output

    // operands and h first, as buffer loads (counted precisely, so the LDS
    // fill below waits for these only, not for the plane loads behind them)
    uint32_t flag = 0;
    if constexpr (COHERENT)
        flag = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(sync, 4), 0, 0, kDeviceScope);
    v4u pre[kPreVec];
    if constexpr (!COHERENT) preload_ops(L.tb, steps * NB2, L.R2, pre);
    // h of the item's rows: thread t holds 8 consecutive fp16 of path t / (kThreads/2)
    const int hp = (int)threadIdx.x / (kThreads / 2), hr = ((int)threadIdx.x % (kThreads / 2)) * 8;
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(L.h, (int64_t)L.P * L.d_out * 2);
    // 16-byte pieces when every row group of 8 starts 16-byte aligned and none straddles d_out
    const bool hvec = (L.d_out & 7) == 0 && ((uintptr_t)L.h & 15) == 0;
    v4u hq[kHRows / (kThreads / 2) / 8];
    const int64_t row_end = imin(L.d_out, row_begin + (int64_t)tiles * kRG);   // rows of the item
#pragma unroll
    for (int k = 0; k < kHRows / (kThreads / 2) / 8; ++k) {
        const int64_t row = row_begin + hr + k * (kThreads / 2) * 8;
        const bool ok = hvec && hp < L.P && row + 8 <= row_end;
        hq[k] = __builtin_amdgcn_raw_buffer_load_b128(rh, ok ? (uint32_t)(((int64_t)hp * L.d_out + row) * 2) : kOOB, 0, 0);
    }

    // lane (gq, r16) loads rows row+4r16 .. +3 of plane 4s + gq of tile i
    const __amdgpu_buffer_rsrc_t ru = make_rsrc(L.u_bits, (int64_t)L.P * L.kw_u * L.ld_u * 4);
    const uint32_t uo = (uint32_t)(((int64_t)gq * L.ld_u + row_begin + wave * kTile + 4 * r16) * 4);
    const uint32_t group4 = (uint32_t)(4 * L.ld_u * 4);
    // rows past d_out are not loaded (padding words of the planes)
    const int64_t lane_row = row_begin + wave * kTile + 4 * r16;
    auto off_of = [&](int e) -> uint32_t {
        const int i = e / steps, st = e - i * steps;
        return e < total && lane_row + (int64_t)i * kRG < L.d_out ? uo + (uint32_t)(i * kRG * 4) + (uint32_t)st * group4
                                                                 : kOOB;
    };
    v4u slot[kWin2];
#pragma unroll
    for (int k = 0; k < kWin2; ++k) slot[k] = load_rows(ru, off_of(k));
    if constexpr (COHERENT) {
        const uint32_t want = (uint32_t)(L.P * L.nrg) + run.want_extra;   // every latent group of the linear
        if (((uint32_t)__builtin_amdgcn_readfirstlane(flag) & 0xffffu) != want)
            wait_count(sync, want, run.spin_limit);
        preload_ops<kDeviceScope>(L.tb, steps * NB2, L.R2, pre);
    }

    // operands of every step and h of the item's rows into LDS, shared by the 4 waves
    copy_ops<COHERENT ? kDeviceScope : 0>(ops, L.tb, steps * NB2, R2, pre);
    if (threadIdx.x < kRec / 16) *(v4u *)(zrec + threadIdx.x * 16) = v4u{0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < kHRows / (kThreads / 2) / 8; ++k) {
        const int rl = hr + k * (kThreads / 2) * 8;
        *(v4u *)(hs + hp * kHRows + rl) = hq[k];
    }
    if (!hvec) {                  // rows the 16-byte loads did not cover: one by one
        __syncthreads();
        for (int i = threadIdx.x; i < 2 * kHRows; i += kThreads) {
            const int pp = i / kHRows, rl = i - pp * kHRows;
            const int64_t row = row_begin + rl;
            hs[i] = (pp < L.P && row < L.d_out) ? L.h[(int64_t)pp * L.d_out + row] : (uint16_t)0;
        }
    }
    __syncthreads();
    if constexpr (COHERENT) {
        // every wave is past its check: count this workgroup as an event of
        // the linear; the run's last event clears the word for the next run
        if (threadIdx.x == 0) sync_event(sync, 0x10000u, (uint32_t)(L.P * L.nrg + L.n2));
    }

    v4f acc[4][NB2];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int b = 0; b < NB2; ++b) acc[m][b] = v4f{0.f, 0.f, 0.f, 0.f};
    // lane (gq, r16) reads quarter gq of record r16 of each operand and its
    // scale; rows no token fills read the zero record
    const bool rlive = r16 < R2;
    const uint8_t *dl = (rlive ? ops + r16 * kRec : zrec) + gq * 32;
    const uint8_t *sl = (rlive ? ops + r16 * kRec : zrec) + 128 + gq;
    const int sb = rlive ? R2 * kRec : 0;                         // next token block
    const int ss = sb * NB2;                                      // next step
    int i = 0, st = 0, so = 0;
    auto process = [&](const v4u &w) {
        v8i ao[NB2];
        int sa[NB2];
#pragma unroll
        for (int b = 0; b < NB2; ++b) {
            ao[b] = load_op_at(dl + so + b * sb);
            sa[b] = sl[so + b * sb];
        }
        so += ss;
        v8i sgq[4];
        unpack_quad(w, nib, sgq);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const v8i sg = sgq[m];
#pragma unroll
            for (int b = 0; b < NB2; ++b) acc[m][b] = mfma(ao[b], sg, acc[m][b], sa[b]);
        }
        if (++st == steps) {
            // y = sum_p h_p z_p for this lane's 4 rows of tile i (as k_stage2)
            const int rl = i * kRG + wave * kTile + 4 * r16;      // row within the item
            const int64_t row = row_begin + rl;
            float hv[2][4];
#pragma unroll
            for (int pp = 0; pp < 2; ++pp) {
                const v2u hw = *(const v2u *)(hs + pp * kHRows + rl);
                hv[pp][0] = f16_to_f32((uint16_t)(hw[0] & 0xffffu));
                hv[pp][1] = f16_to_f32((uint16_t)(hw[0] >> 16));
                hv[pp][2] = f16_to_f32((uint16_t)(hw[1] & 0xffffu));
                hv[pp][3] = f16_to_f32((uint16_t)(hw[1] >> 16));
            }
#pragma unroll
            for (int b = 0; b < NB2; ++b) {
                float y4[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const v4f a = acc[m][b];
                    if (NL == 2) {
                        y4[m] = hv[0][m] * (a[0] + a[1]) + hv[1][m] * (a[2] + a[3]);
                    } else {
                        const float o0 = __shfl_xor(a[0], 16, 64), o1 = __shfl_xor(a[1], 16, 64);
                        const float z0 = (a[0] + a[1]) + a[2];
                        const float z1 = (a[3] + o0) + o1;
                        y4[m] = hv[0][m] * z0 + hv[1][m] * z1;
                    }
                }
                const int n = b * R::TPM2 + (NL == 2 ? gq : gq / 2);
                const bool writer = n < T && (NL == 2 || (gq & 1) == 0);
                if (run.ystage) {                               // uniform
                    if (writer) {
                        uint8_t *yp = ys + ((size_t)n * kHRows + rl) * ysb;
                        if (ysb == 2)
                            *(v2u *)yp = v2u{bf16_pair(y4[0], y4[1]), bf16_pair(y4[2], y4[3])};
                        else
                            *(v4f *)yp = v4f{y4[0], y4[1], y4[2], y4[3]};
                    }
                } else {
                    if (L.resid && writer) {                    // (uniform pointer) the residual, unrounded sum
#pragma unroll
                        for (int m = 0; m < 4; ++m)
                            if (row + m < L.d_out) y4[m] += load_act(L.resid, run.y_dtype, (int64_t)n * L.d_out + row + m);
                    }
                    store4(ob, (int64_t)n * L.d_out + row, row, L.d_out, y4, writer);
                }
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int b = 0; b < NB2; ++b) acc[m][b] = v4f{0.f, 0.f, 0.f, 0.f};
            st = 0;
            so = 0;
            ++i;
        }
    };
    for (int e0 = 0; e0 < total; e0 += kWin2) {
#pragma unroll
        for (int k = 0; k < kWin2; ++k) {
            if (e0 + k < total) process(slot[k]);                 // uniform
            slot[k] = load_rows(ru, off_of(e0 + k + kWin2));
        }
    }
    if (run.ystage) {
        // the item's outputs leave as one contiguous burst per token row
        // (16-byte chunks, all threads together), not as scattered pieces
        // between other workgroups' plane reads
        __syncthreads();
        const int64_t rows = imin((int64_t)tiles * kRG, L.d_out - row_begin);
        const int per = 16 / yb;                                   // outputs per chunk
        const bool chunky = ob.vec && (L.d_out % per) == 0 && ((uintptr_t)L.y & 15) == 0;
        const int cpr = (int)cdiv(rows, per);                      // chunks per token row
        // a residual (same dtype and layout as y) is added to the unrounded
        // fp32 outputs, which are then collected at 4 bytes each
        const __amdgpu_buffer_rsrc_t rres = make_rsrc(L.resid, (int64_t)T * L.d_out * yb);
        for (int c = threadIdx.x; c < T * cpr; c += kThreads) {
            const int n = c / cpr, k = c - n * cpr;
            const int64_t r0 = (int64_t)k * per;                   // row within the item
            const int64_t e0 = (int64_t)n * L.d_out + row_begin + r0;
            v4u w;
            if (ysb == yb && !L.resid) {                           // uniform
                w = *(const v4u *)(ys + ((size_t)n * kHRows + r0) * yb);
            } else {
                // fp32 collected; add the residual, then y's dtype
                float f[8];
#pragma unroll
                for (int q = 0; q < 8; q += 4) {
                    if (q >= per) break;
                    const v4f a = *(const v4f *)(ys + ((size_t)n * kHRows + r0 + q) * 4);
                    f[q] = a[0];
                    f[q + 1] = a[1];
                    f[q + 2] = a[2];
                    f[q + 3] = a[3];
                }
                if (L.resid) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        if (q >= per) break;
                        const bool ok = r0 + q < rows;
                        const uint32_t ro = ok ? (uint32_t)((e0 + q) * yb) : kOOB;
                        f[q] += yb == 2 ? bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rres, ro, 0, 0))
                                        : __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rres, ro, 0, 0));
                    }
                }
                if (yb == 2)
                    w = v4u{bf16_pair(f[0], f[1]), bf16_pair(f[2], f[3]), bf16_pair(f[4], f[5]), bf16_pair(f[6], f[7])};
                else
                    w = v4u{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
            }
            if (chunky) {
                __builtin_amdgcn_raw_buffer_store_b128(w, ob.r, r0 + per <= rows ? (uint32_t)(e0 * yb) : kOOB, 0, 0);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    if (q >= per) break;
                    const bool ok = r0 + q < rows;
                    if (yb == 2)
                        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(w[q >> 1] >> (16 * (q & 1))), ob.r,
                                                              ok ? (uint32_t)((e0 + q) * 2) : kOOB, 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(w[q], ob.r, ok ? (uint32_t)((e0 + q) * 4) : kOOB, 0, 0);
                }
            }
        }
    }
}

template <int NL, int NB2>
__global__ __launch_bounds__(kThreads) void k_stage2r(MRun run, MLin single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    if (stale_ws(run)) return;
    const int64_t item = item_of<true>(run.ord2, run.base2);
    const MLin L = pick<kKindStage2, true>(run, single, run.lin2, item);
    const int64_t row_begin = (item - L.item2) * L.rows2;
    const int tiles = (int)imin(L.rows2 / kRG, cdiv(L.d_out - row_begin, kRG));
    stage2r_item<NL, NB2, false>(run, L, row_begin, tiles, smem, nullptr);
}

// ---------------------------------------------------------------------------
// the one-launch pass: stage 1, latents and stage 2 of a group in one grid
// ---------------------------------------------------------------------------

// Workgroups [0, items1) run stage-1 items, the rest stage-2 items.  A linear's
// stage-2 items need its latents, so the hand-off goes through counters,
// inside the launch:
//   - a stage-1 workgroup stores its partial sums at device scope, waits until
//     they are complete, and counts itself in the counter of its latent group
//     (linear, path, tiles [rg*F, (rg+1)*F)), whose chunks are its nchunks
//     items;
//   - the workgroup that completes that count (the group's last chunk in this
//     run) sets the counter back to zero, sums the group's partials into its
//     planes of the stage-2 operands (the latent step, spread over the
//     linear's P * nrg groups), stores them at device scope and counts the
//     group in the linear's sync word;
//   - a stage-2 workgroup waits until every group of its linear is counted in
//     before it loads the operands, then counts itself in the same word.
// The sync word of a linear holds the stored groups in its low half and all
// events (groups stored, stage-2 workgroups past their wait) in its high half;
// the run's last event sets it back to zero.  So every counter is zero when a
// run starts and again when it has ended, and a run needs nothing from the
// host but its tables: a captured launch replays like a fresh one.
// Device-scope accesses bypass the non-coherent caches of the other XCDs, so
// no cache-wide write-back or invalidation is needed.  Workgroups start in
// index order, so when a stage-2 workgroup runs, every stage-1 workgroup has
// started already; those never wait, so every wait ends.  The wait is also
// bounded (spin_limit polls): a wave that gives up reports
// LB_FAULT_HANDOFF_TIMEOUT in the fault word (its outputs are wrong) and the
// launch still ends; the counters still return to zero.
template <int NL, int NB2, bool XM = false>
__global__ __launch_bounds__(kThreads) void k_pass(MRun run, MLin single) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ uint32_t s_count;
    if (stale_ws(run)) return;
    const int64_t b = blockIdx.x;
    if (b < run.items1) {
        // groups: the stage-1 order from the workspace; inline runs: item order
        const int64_t item = run.ordP1 ? (int64_t)__builtin_amdgcn_readfirstlane(run.ordP1[b]) : b;
        const int j = run.table ? __builtin_amdgcn_readfirstlane(run.lin1[item])
                                : run.ninl ? inline_index<kKindStage1>(run, item) : 0;
        const MLin L = pick<kKindStage1>(run, single, run.lin1, item);
        stage1f_item<NL, true, XM>(run, L, item, smem);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // this wave's partial sums are stored
        __syncthreads();
        const int f = (int)((item - L.item1) / L.nchunks);          // latent group: path * nrg + rg
        uint32_t *arr = run.arrive + (L.fin0 + f) * kFlagStride;
        if (threadIdx.x == 0)
            s_count = __hip_atomic_fetch_add(arr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (s_count + 1u == (uint32_t)L.nchunks) {           // uniform: the group's last chunk
            if (threadIdx.x == 0) __hip_atomic_store(arr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            latent_rows<NL, NB2>(run, L, f / L.nrg, f % L.nrg, smem);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's operand bytes are stored
            __syncthreads();
            if (threadIdx.x == 0)
                sync_event(run.sync + j * kFlagStride, 0x10001u, (uint32_t)(L.P * L.nrg + L.n2));
        }
    } else {
        // (linear, first 256-row tile << 8 | tiles) of this workgroup: from the
        // workspace table (groups), or the inline linears' stage-2 items in order
        int j, g;
        if (run.tabP2) {
            const int32_t *e = run.tabP2 + 2 * (b - run.items1);
            j = __builtin_amdgcn_readfirstlane(e[0]);
            g = __builtin_amdgcn_readfirstlane(e[1]);
        } else {
            const int64_t e = b - run.items1;
            j = run.ninl ? inline_index<kKindStage2>(run, e) : 0;
            const MLin m = pick_linear(run, single, j);
            const int64_t local = e - m.item2;
            const int per = (int)(m.rows2 / kRG);
            const int tiles = (int)imin(per, cdiv(m.d_out - local * m.rows2, kRG));
            g = (int)((local * per) << 8) | tiles;
        }
        stage2r_item<NL, NB2, true>(run, pick_linear(run, single, j), (int64_t)(g >> 8) * kRG, g & 255, smem,
                                    run.sync + j * kFlagStride);
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

int rows1(const Shape &s, int64_t T) { return (int)imin(16, T * (s.NL == 2 ? 2 : 4)); }
int rows2(const Shape &s, int64_t T) { return (int)imin(16, T * (s.NL == 2 ? 4 : 8)); }
int kcg_cap(const Shape &s) { return (int)imin(kMaxKcg, kLdsBudget / (s.NB1 * kOpS)); }

// Stage 1 runs fused (k_stage1f) when the tokens fill one activation-row block.
bool fused1(const Shape &s) { return s.NB1 == 1; }
constexpr int64_t kFusedBytes = 192 * 1024;    // V-plane bytes per fused stage-1 item, about
// Fused form: an item covers at most F latent tiles, as many as the LDS of its
// cross-wave sums ([F][kWaves][T][64] floats) holds within kRedBudget.
constexpr size_t kRedBudget = 24 * 1024;
int flush1_for(int64_t T, int ts) {
    return (int)imax(1, (int64_t)kRedBudget / ((ts ? 1 : kWaves) * T * 64 * 4));
}
size_t red1_bytes(int64_t T, int F, int ts) { return (size_t)F * (ts ? 1 : kWaves) * T * 64 * 4; }
// The fused stage 1 splits an item's tiles among the waves when every linear
// has at least one 64-latent tile per wave, else its K-groups.
bool tsplit_for(const Linear *ls, int n) {
    for (int j = 0; j < n; ++j)
        if (cdiv(ls[j].r_p, kTile) < kWaves) return false;
    return n > 0;
}

// Steps the stage-2 LDS holds: all steps of the largest linear when they fit,
// else a multiple of the batch (at least one batch, which may exceed 64 KB).
// Whether stage 2 can run k_stage2r: every step's operands and h of an item
// fit the LDS of one CU (two workgroups' worth when possible).
// k_stage2r collects an item's outputs in LDS when they fit kYStage.
int ystage_for(int64_t T, int yst) { return (size_t)T * kHRows * yst <= (size_t)kYStage ? 1 : 0; }

// Bytes per collected stage-2 output: y's size, or 4 when any linear of the
// launch adds a residual (it is added to the unrounded sum).
int yst_for(const Linear *ls, int n, int y_dtype) {
    for (int j = 0; j < n; ++j)
        if (ls[j].resid) return 4;
    return y_dtype == LB_BF16 ? 2 : 4;
}

bool dma2_for(const Shape &s, int64_t T, int steps_max) {
    return ops2r_bytes(steps_max, s.NB2, rows2(s, T)) + 2 * kHRows * 2 <= 88 * 1024;
}

int ops2_for(const Shape &s, int steps_max) {
    int cap = kLdsBudget / (s.NB2 * kOpS);
    if (cap < kBatch) cap = kBatch;
    return steps_max <= cap ? steps_max : (cap / kBatch) * kBatch;
}

// Fill the schedule fields of m and return the workspace bytes it needs.
// Grain of a group's items: the fused stage-1 chunk target (bytes of V planes)
// and the 256-row tiles of a stage-2 item.
struct Grain {
    int64_t fused_bytes = kFusedBytes;
    int tiles2 = kTilesPerItem2;
    int tsplit = 0;       // fused stage 1 splits tiles among the waves (tsplit_for)
    int f_cap = 1 << 20;  // fused stage 1: 64-latent tiles per item, at most
};

size_t plan_linear(const Linear &a, const Shape &s, bool many, MLin *m, Grain gr = Grain{}) {
    *m = MLin{};
    m->x = a.x;
    m->x2 = a.x2;
    m->xs = a.xs;
    m->resid = a.resid;
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
    m->kgv = (int32_t)cdiv(m->kw_v, 4);
    m->nrg = (int32_t)cdiv(a.r_p, kRG);
    m->R1 = rows1(s, a.T);
    m->R2 = rows2(s, a.T);
    if (fused1(s)) {
        // chunks of about kFusedBytes of V planes (all latents of the path),
        // LDS-bounded, spread evenly over d_in
        const int64_t per_kg = (int64_t)a.r_p * 16;
        int64_t kc = imax(1, imin(kMaxKcf, gr.fused_bytes / per_kg));
        kc = imin(kc, (int64_t)((kLdsBudget - kRedBudget) / (m->R1 * kRec)));
        if (!many)   // a lone linear: smaller chunks until the chip has work
            while (kc > 4 && a.P * cdiv(m->kgv, kc) < 256) kc = (kc + 1) / 2;
        const int64_t nch = cdiv(m->kgv, kc);
        m->kcg = (int32_t)cdiv(m->kgv, nch);
        m->nchunks = (int32_t)cdiv(m->kgv, m->kcg);
        m->nrg = (int32_t)cdiv(cdiv(a.r_p, kTile), imin(flush1_for(a.T, gr.tsplit), gr.f_cap));
        m->kcp = 0;
        m->nprep = 0;
        m->xvec = (a.d_in % 8 == 0 && ((uintptr_t)a.x & 15) == 0 && ((uintptr_t)a.x2 & 15) == 0 &&
                   ((uintptr_t)a.g & 15) == 0 && a.xm_dh % 8 == 0) ? 1 : 0;
        m->xm_dh = a.xm_dh;
        m->xm_grp = a.xm_dh ? a.xm_grp : 1;
    } else {
        int kcg = kcg_cap(s);
        if (!many)   // a lone linear: smaller chunks until the chip has work
            while (kcg > 1 && a.P * m->nrg * cdiv(m->kgv, kcg) < 512) kcg = (kcg + 1) / 2;
        if (kcg > m->kgv) kcg = m->kgv;
        m->kcg = kcg;
        m->nchunks = (int32_t)cdiv(m->kgv, kcg);
        // prep items: up to 16 K-groups, LDS-bounded
        int kcp = (int)imin(16, kLdsBudget / (s.NB1 * m->R1 * kRec));
        if (kcp < 1) kcp = 1;
        if (kcp > m->kgv) kcp = m->kgv;
        m->kcp = kcp;
        m->nprep = (int32_t)cdiv(m->kgv, kcp);
    }
    m->kgs = (int32_t)cdiv((int64_t)a.P * m->kw_u, 4);
    // long K (many K-groups per tile): fewer tiles per item, so that an item
    // streams about kSteps2 (tile, K-group) steps per 4 activation rows and the
    // last items of a launch end close together.  (Every item first loads all
    // of its linear's operands, R2 rows per K-group, so with more rows it
    // keeps more tiles.)
    int tiles = (int)imax(1, imin(gr.tiles2, kSteps2 * m->R2 / (4 * m->kgs)));
    if (!many)   // a lone linear: fewer tiles per item until the chip has work
        while (tiles > 1 && cdiv(a.d_out, (int64_t)kRG * tiles) < 512) tiles /= 2;
    m->rows2 = kRG * tiles;
    m->n2 = (int32_t)cdiv(a.d_out, m->rows2);
    const size_t part = rup256((size_t)m->nchunks * a.T * a.P * a.r_p * 4);
    const size_t pa = fused1(s) ? 0 : rup256((size_t)a.P * m->kgv * s.NB1 * m->R1 * kRec);
    const size_t tb = rup256((size_t)m->kgs * s.NB2 * m->R2 * kRec);
    return part + pa + tb;
}

void bind_ws(MLin *m, const Linear &a, const Shape &s, uint8_t *ws) {
    const size_t part = rup256((size_t)m->nchunks * a.T * a.P * a.r_p * 4);
    const size_t pa = fused1(s) ? 0 : rup256((size_t)a.P * m->kgv * s.NB1 * m->R1 * kRec);
    m->part = (float *)ws;
    m->pa = fused1(s) ? nullptr : ws + part;
    m->tb = ws + part + pa;
}


// LDS of each kernel, given the largest per-linear figures of a launch.
struct Lds {
    size_t prep, s1, lat, s2;
};

// stage_mask: bit 0 = prep, stage 1 and the latent pass; bit 1 = stage 2;
// bit 2 = the latent pass alone (from given latents).
template <int NL, int NB1, int NB2>
int launch_all(const MRun &run, const MLin &single, const Lds &lds, hipStream_t st, int stage_mask) {
    // launches with no items (a chunk of a group may have none of a kind) are skipped
    if ((stage_mask & 1) && NB1 == 1) {
        if (run.items1 > 0) {
            if (run.xmap) {                // input maps: bf16 out only
                if constexpr (NL == 2) k_stage1f<NL, true><<<(unsigned)run.items1, kThreads, lds.s1, st>>>(run, single);
                else return LB_EUNSUPPORTED;
            } else {
                k_stage1f<NL><<<(unsigned)run.items1, kThreads, lds.s1, st>>>(run, single);
            }
            if (int rc = last_launch_status()) return rc;
        }
    } else if (stage_mask & 1) {
        if (run.items0 > 0) {
            k_prep<NL, NB1><<<(unsigned)run.items0, kThreads, lds.prep, st>>>(run, single);
            if (int rc = last_launch_status()) return rc;
        }
        if (run.items1 > 0) {
            k_stage1<NL, NB1><<<(unsigned)run.items1, kThreads, lds.s1, st>>>(run, single);
            if (int rc = last_launch_status()) return rc;
        }
    }
    if ((stage_mask & 5) && run.itemsF > 0) {
        k_latent<NL, NB2><<<(unsigned)run.itemsF, kThreads, lds.lat, st>>>(run, single);
        if (int rc = last_launch_status()) return rc;
    }
    if ((stage_mask & 2) && run.items2 <= 0) return LB_OK;
    if ((stage_mask & 2) && run.dma2) {
        const size_t l2 = ops2r_bytes(run.ops2, NB2, rows2(Shape{NL, NB1, NB2}, run.T)) + 2 * kHRows * 2 +
                          (run.ystage ? (size_t)run.T * kHRows * run.yst : 0);
        if (l2 > 160 * 1024) return LB_EUNSUPPORTED;
        static bool raised = false;        // once per instantiation (idempotent if raced)
        if (!raised) {
            if (hipFuncSetAttribute((const void *)k_stage2r<NL, NB2>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    160 * 1024) != hipSuccess)
                return hip_status(hipGetLastError());
            raised = true;
        }
        k_stage2r<NL, NB2><<<(unsigned)run.items2, kThreads, l2, st>>>(run, single);
        if (int rc = last_launch_status()) return rc;
    } else if (stage_mask & 2) {
        const size_t l2 = lds.s2;
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

int launch_shape(const Shape &s, const MRun &run, const MLin &single, const Lds &lds, hipStream_t st,
                 int stage_mask = 3) {
    const int key = s.NL * 1000 + s.NB1 * 10 + s.NB2;
    switch (key) {
        case 2011: return launch_all<2, 1, 1>(run, single, lds, st, stage_mask);
        case 2012: return launch_all<2, 1, 2>(run, single, lds, st, stage_mask);
        case 2024: return launch_all<2, 2, 4>(run, single, lds, st, stage_mask);
        case 2048: return launch_all<2, 4, 8>(run, single, lds, st, stage_mask);
        case 3011: return launch_all<3, 1, 1>(run, single, lds, st, stage_mask);
        case 3012: return launch_all<3, 1, 2>(run, single, lds, st, stage_mask);
        case 3024: return launch_all<3, 2, 4>(run, single, lds, st, stage_mask);
        case 3048: return launch_all<3, 4, 8>(run, single, lds, st, stage_mask);
    }
    return LB_EUNSUPPORTED;
}

void lds_add(Lds *l, const MLin &m, const Shape &s, int ops2, int64_t T, int F, int ts) {
    const size_t prep = (size_t)m.kcp * s.NB1 * m.R1 * kRec;
    const size_t s1 = fused1(s) ? (size_t)m.kcg * m.R1 * kRec + red1_bytes(T, F, ts) : (size_t)m.kcg * s.NB1 * kOpS;
    const size_t lat = (size_t)2 * s.NB2 * m.R2 * kRec;
    const size_t s2 = (size_t)ops2 * s.NB2 * kOpS;
    if (prep > l->prep) l->prep = prep;
    if (s1 > l->s1) l->s1 = s1;
    if (lat > l->lat) l->lat = lat;
    if (s2 > l->s2) l->s2 = s2;
}

}  // namespace

bool mfma_fused_stage1(int64_t T, int y_dtype) {
    Shape s;
    return shape_for(T, y_dtype, &s) && fused1(s);
}

bool mfma_decode_supported(int64_t T, int y_dtype) {
    Shape s;
    return shape_for(T, y_dtype, &s);
}

bool mfma_decode_shape_ok(const Linear &a) {
    // every buffer the kernels address through 32-bit offsets stays below 2 GiB
    const int64_t lim = 1ll << 31;
    const int64_t kgv = cdiv(a.kw_v(), 4), kgs = cdiv((int64_t)a.P * a.kw_u(), 4);
    return (int64_t)a.P * a.kw_v() * a.ld_v * 4 < lim && (int64_t)a.P * a.kw_u() * a.ld_u * 4 < lim &&
           a.T * a.d_in * 4 < lim && a.T * a.d_out * 4 < lim && (int64_t)a.P * a.d_out * 2 < lim &&
           kgv * a.T * a.P * a.r_p * 4 < lim && kgs * 8 * 16 * kRec < lim;
}

// The fault word's address on the current device, looked up once per device
// (threads that race on the first lookup store the same address).
uint32_t *fault_word_ptr() {
    static std::atomic<uint32_t *> ptr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    uint32_t *q = ptr[dev].load(std::memory_order_acquire);
    if (!q) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_lb_faults)) != hipSuccess) return nullptr;
        q = (uint32_t *)p;
        ptr[dev].store(q, std::memory_order_release);
    }
    return q;
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
        Linear c = a;                  // the one-launch form (mfma_decode_forward takes it when it applies)
        c.y_dtype = yd;
        need = std::max(need, mfma_inline_workspace_bytes(&c, 1));
    }
    return need;
}

namespace {
// A single linear's launch state on the decode kernels.
int single_setup(const Linear &a, void *ws, Shape *s, MLin *m, MRun *run, Lds *lds) {
    if (!shape_for(a.T, a.y_dtype, s)) return LB_EUNSUPPORTED;
    Grain gr;
    gr.tsplit = fused1(*s) && tsplit_for(&a, 1) ? 1 : 0;
    plan_linear(a, *s, false, m, gr);
    bind_ws(m, a, *s, (uint8_t *)ws);
    *run = MRun{};
    if (a.xm_dh && !(fused1(*s) && s->NL == 2)) return LB_EUNSUPPORTED;   // input maps: fused stage 1, bf16 out
    run->xmap = a.xm_dh ? 1 : 0;
    run->T = (int)a.T;
    run->x_dtype = a.x_dtype;
    run->y_dtype = a.y_dtype;
    run->dma2 = dma2_for(*s, a.T, m->kgs);
    run->yst = yst_for(&a, 1, a.y_dtype);
    run->ystage = ystage_for(a.T, run->yst);
    run->ops2 = run->dma2 ? m->kgs : ops2_for(*s, m->kgs);
    run->items0 = items0_of(*m);
    run->items1 = items1_of(*m);
    run->itemsF = itemsF_of(*m);
    run->items2 = m->n2;
    run->table = nullptr;
    *lds = Lds{};
    run->tsplit = gr.tsplit;
    run->flush1 = (int)imin(flush1_for(a.T, run->tsplit), cdiv(m->r_p, kTile));
    lds_add(lds, *m, *s, run->ops2, a.T, run->flush1, run->tsplit);
    return LB_OK;
}
}  // namespace

int mfma_decode_forward(const Linear &a, void *ws, hipStream_t st) {
    if (mfma_inline_pass(&a, 1)) return mfma_inline_forward(&a, 1, ws, st);   // one launch after a clear
    Shape s;
    MLin m;
    MRun run;
    Lds lds;
    if (int rc = single_setup(a, ws, &s, &m, &run, &lds)) return rc;
    return launch_shape(s, run, m, lds, st);
}

int mfma_decode_stage(const Linear &a, void *ws, int stage, void *t, int t_dtype, hipStream_t st) {
    Shape s;
    MLin m;
    MRun run;
    Lds lds;
    if (int rc = single_setup(a, ws, &s, &m, &run, &lds)) return rc;
    run.t_io = t;
    run.t_dtype = t_dtype;
    run.t_mode = stage == 1 ? 1 : 2;
    // stage 1: activation operands, first contractions, latents (also to t);
    // stage 2: the latent step from t, second contractions
    return launch_shape(s, run, m, lds, st, stage == 1 ? 1 : 6);
}

// ---- groups ------------------------------------------------------------------

struct MGroupHost {
    Shape s;
    MRun run;
    Lds lds;
    size_t lds_pass;     // dynamic LDS of k_pass
    int n;               // linears
};

// k_pass: stage-2 items of the linears whose stage-1 items start among the last
// kLateItems of the launch's stage-1 order go after all other stage-2 items
// (those are ready by the time they start), so few workgroups wait.
constexpr int64_t kLateItems = 1024;

// Items sized for large stacks leave a small group (one layer) with a few
// dozen workgroups; halve the grain while a launch has fewer than
// kMinGroupItems items (the stage-1 chunk down to a floor of K-groups, the
// stage-2 item down to one 256-row tile).
constexpr int64_t kMinGroupItems = 1024;

// The one-launch pass sums a latent group's chunk partials in one workgroup
// (the group's last chunk), a few loads per chunk in sequence: small groups
// keep chunks of at least kPassMinKcg K-groups there, where the three-launch
// form (which spreads that sum over many workgroups) goes down to 4.
constexpr int kPassMinKcg = 16;

// Token counts the one-launch pass serves: those that fill at most 8 of the
// 16 stage-2 activation rows (bf16 out: T <= 2, fp32 out: T = 1).  On the 32-,
// 40- and 80-layer stacks it measured 4 to 7 percent faster than the three
// launches at T = 1 and -1 to +6 percent at T = 2, but 12 to 26 percent
// slower at T = 4, where its workgroups hold stage 2's 16-row operands.
bool pass_tokens(const Shape &s, int64_t T) { return fused1(s) && rows2(s, T) <= 8; }

// Whether a group runs as one launch (k_pass): such a token count and a stage
// 2 whose operands fit the LDS (the K-groups, and so that test, do not depend
// on the grain).
bool pass_form(const Linear *ls, int n, const Shape &s) {
    if (!pass_tokens(s, ls[0].T)) return false;
    int steps_max = 1;
    for (int j = 0; j < n; ++j) {
        MLin m;
        plan_linear(ls[j], s, true, &m);
        steps_max = (int)imax(steps_max, m.kgs);
    }
    return dma2_for(s, ls[0].T, steps_max);
}

Grain group_grain(const Linear *ls, int n, const Shape &s) {
    Grain g;
    g.tsplit = fused1(s) && tsplit_for(ls, n) ? 1 : 0;
    const int kc_floor = pass_form(ls, n, s) ? kPassMinKcg : 4;
    for (int pass = 0; pass < 16; ++pass) {
        int64_t i1 = 0, i2 = 0, kc_min = kMaxKcf;
        for (int j = 0; j < n; ++j) {
            MLin m;
            plan_linear(ls[j], s, true, &m, g);
            i1 += items1_of(m);
            i2 += m.n2;
            kc_min = imin(kc_min, m.kcg);
        }
        bool changed = false;
        if (fused1(s) && i1 < kMinGroupItems && kc_min > kc_floor && g.fused_bytes > 4096) {
            g.fused_bytes /= 2;
            changed = true;
        } else if (fused1(s) && i1 < kMinGroupItems) {
            // then fewer latent tiles per item (down to one per wave)
            int64_t f = imin(g.f_cap, flush1_for(ls[0].T, g.tsplit)), tiles = 1;
            for (int j = 0; j < n; ++j) tiles = imax(tiles, cdiv(ls[j].r_p, kTile));
            f = imin(f, tiles);
            const int64_t fmin = g.tsplit ? kWaves : 1;
            if (f > fmin) {
                g.f_cap = (int)imax(fmin, f / 2);
                changed = true;
            }
        }
        if (i2 < kMinGroupItems && g.tiles2 > 1) {
            g.tiles2 /= 2;
            changed = true;
        }
        if (!changed) break;
    }
    return g;
}

// Workspace of a group, in this order: the 256-byte header (the stamp), the
// per-linear table, the item tables and dispatch orders, the counters (the
// "control" part, which a run reads but never writes except the counters,
// which it leaves at zero), then each linear's scratch (partial latents,
// operand records), which must start zero.
struct GroupLayout {
    int64_t i0 = 0, i1 = 0, iF = 0, i2 = 0, nf = 0;
    size_t table, lin0, lin1, linF, lin2, ord1, ord2, ordP1, tabP2, arrive, sync, ctrl_end, total;
};

GroupLayout group_layout(const Linear *ls, int n, const Shape &s, const Grain &gr, std::vector<MLin> *tab,
                         std::vector<size_t> *scratch) {
    GroupLayout g;
    size_t lin_bytes = 0;
    if (tab) tab->assign((size_t)n, MLin{});
    if (scratch) scratch->assign((size_t)n, 0);
    for (int j = 0; j < n; ++j) {
        MLin m;
        const size_t b = plan_linear(ls[j], s, true, &m, gr);
        m.item0 = g.i0;
        m.item1 = g.i1;
        m.itemF = g.iF;
        m.item2 = g.i2;
        m.fin0 = g.nf;
        g.i0 += items0_of(m);
        g.i1 += items1_of(m);
        g.iF += itemsF_of(m);
        g.i2 += m.n2;
        g.nf += groups_of(m);
        if (tab) (*tab)[(size_t)j] = m;
        if (scratch) (*scratch)[(size_t)j] = b;
        lin_bytes += b;
    }
    size_t at = 256;
    auto take = [&](size_t bytes) { const size_t o = at; at += rup256(bytes); return o; };
    g.table = take(sizeof(MLin) * n);
    g.lin0 = take((size_t)g.i0 * 4);
    g.lin1 = take((size_t)g.i1 * 4);
    g.linF = take((size_t)g.iF * 4);
    g.lin2 = take((size_t)g.i2 * 4);
    g.ord1 = take((size_t)g.i1 * 4);     // dispatch orders
    g.ord2 = take((size_t)g.i2 * 4);
    g.ordP1 = take((size_t)g.i1 * 4);    // k_pass: stage-1 order, stage-2 table
    g.tabP2 = take((size_t)g.i2 * 8);
    g.arrive = take((size_t)g.nf * kFlagStride * 4);   // per latent group
    g.sync = take((size_t)n * kFlagStride * 4);        // per linear
    g.ctrl_end = at;
    g.total = at + lin_bytes;
    return g;
}

size_t mfma_group_workspace_bytes(const Linear *ls, int n, int64_t T, int y_dtype) {
    Shape s;
    if (!shape_for(T, y_dtype, &s)) return 0;
    return group_layout(ls, n, s, group_grain(ls, n, s), nullptr, nullptr).total;
}

int mfma_group_plan(const Linear *ls, int n, int64_t T, int y_dtype, void *ws, size_t ws_bytes, uint64_t tag,
                    bool fault_test, void *host_state, GroupImage *img) {
    MGroupHost *hs = (MGroupHost *)host_state;
    *hs = MGroupHost{};
    if (!shape_for(T, y_dtype, &hs->s)) return LB_EUNSUPPORTED;
    const Grain gr = group_grain(ls, n, hs->s);
    std::vector<MLin> tab;
    std::vector<size_t> scratch;
    const GroupLayout G = group_layout(ls, n, hs->s, gr, &tab, &scratch);
    if (ws_bytes < G.total) return LB_EWORKSPACE;
    const int64_t i0 = G.i0, i1 = G.i1, iF = G.iF, i2 = G.i2;
    uint8_t *w = (uint8_t *)ws;
    std::vector<uint8_t> &im = img->bytes;
    im.assign(G.ctrl_end, 0);
    memcpy(im.data(), &tag, sizeof(tag));
    uint8_t *cur = w + G.ctrl_end;
    int steps_max = 1;
    for (int j = 0; j < n; ++j) {
        MLin &m = tab[(size_t)j];
        bind_ws(&m, ls[j], hs->s, cur);
        cur += scratch[(size_t)j];
        if (m.kgs > steps_max) steps_max = m.kgs;
    }
    img->zero_off = G.ctrl_end;
    img->zero_bytes = G.total - G.ctrl_end;
    MRun &run = hs->run;
    run = MRun{};
    run.dma2 = dma2_for(hs->s, T, steps_max);
    run.yst = yst_for(ls, n, y_dtype);
    run.ystage = ystage_for(T, run.yst);
    run.ops2 = run.dma2 ? steps_max : ops2_for(hs->s, steps_max);
    hs->lds = Lds{};
    int64_t ntile_max = 1;
    for (int j = 0; j < n; ++j) ntile_max = imax(ntile_max, cdiv(tab[(size_t)j].r_p, kTile));
    run.tsplit = gr.tsplit;
    run.flush1 = (int)imin(imin(flush1_for(T, run.tsplit), ntile_max), gr.f_cap);
    for (int j = 0; j < n; ++j) lds_add(&hs->lds, tab[(size_t)j], hs->s, run.ops2, T, run.flush1, run.tsplit);
    auto put = [&](size_t off, const void *src, size_t bytes) { if (bytes) memcpy(im.data() + off, src, bytes); };
    std::vector<int32_t> h0((size_t)i0), h1((size_t)i1), hF((size_t)iF), h2((size_t)i2);
    for (int j = 0; j < n; ++j) {
        const MLin &m = tab[(size_t)j];
        for (int64_t k = 0; k < items0_of(m); ++k) h0[(size_t)(m.item0 + k)] = j;
        for (int64_t k = 0; k < items1_of(m); ++k) h1[(size_t)(m.item1 + k)] = j;
        for (int64_t k = 0; k < itemsF_of(m); ++k) hF[(size_t)(m.itemF + k)] = j;
        for (int64_t k = 0; k < m.n2; ++k) h2[(size_t)(m.item2 + k)] = j;
    }
    put(G.table, tab.data(), sizeof(MLin) * n);
    put(G.lin0, h0.data(), (size_t)i0 * 4);
    put(G.lin1, h1.data(), (size_t)i1 * 4);
    put(G.linF, hF.data(), (size_t)iF * 4);
    put(G.lin2, h2.data(), (size_t)i2 * 4);
    // dispatch orders: largest items first (bytes of sign planes each streams;
    // ties keep item order), so a launch ends on short workgroups
    const bool fz = fused1(hs->s);
    std::vector<int64_t> c1((size_t)i1), c2((size_t)i2);
    for (int j = 0; j < n; ++j) {
        const MLin &m = tab[(size_t)j];
        for (int64_t k = 0; k < items1_of(m); ++k) {
            const int64_t c = k % m.nchunks;
            const int64_t rg = fz ? (k / m.nchunks) % m.nrg : k % m.nrg;
            const int64_t cc = fz ? c : (k / m.nrg) % m.nchunks;
            const int64_t nkg = imin(m.kcg, m.kgv - cc * m.kcg);
            const int64_t span = fz ? (int64_t)run.flush1 * kTile : kRG;
            const int64_t rows = imin(span, m.r_p - rg * span);
            c1[(size_t)(m.item1 + k)] = nkg * rows;
        }
        for (int64_t k = 0; k < m.n2; ++k) {
            const int64_t tiles = imin(m.rows2 / kRG, cdiv(m.d_out - k * m.rows2, kRG));
            c2[(size_t)(m.item2 + k)] = tiles * m.kgs;
        }
    }
    auto order = [](const std::vector<int64_t> &cost) {
        std::vector<int32_t> o(cost.size());
        for (size_t i = 0; i < o.size(); ++i) o[i] = (int32_t)i;
        std::stable_sort(o.begin(), o.end(), [&](int32_t a, int32_t b) { return cost[(size_t)a] > cost[(size_t)b]; });
        return o;
    };
    const std::vector<int32_t> o1 = order(c1), o2 = order(c2);
    put(G.ord1, o1.data(), (size_t)i1 * 4);
    put(G.ord2, o2.data(), (size_t)i2 * 4);
    // k_pass: stage-1 items linear by linear (a linear's latents are ready
    // early); stage-2 items of the early linears largest first, then those of
    // the late ones, largest first
    std::vector<int32_t> p1((size_t)i1), p2;
    for (size_t i = 0; i < p1.size(); ++i) p1[i] = (int32_t)i;
    std::vector<int32_t> early, late;
    for (size_t i = 0; i < o2.size(); ++i) {
        const MLin &m = tab[(size_t)h2[(size_t)o2[i]]];
        (m.item1 + items1_of(m) > i1 - kLateItems ? late : early).push_back(o2[i]);
    }
    p2 = early;
    p2.insert(p2.end(), late.begin(), late.end());
    // one entry per stage-2 workgroup: (linear, first 256-row tile << 8 |
    // tiles).  (Cutting the last items into smaller pieces, so that the
    // launch drains sooner, was slower: every piece pays the operand and flag
    // round trips of an item.)
    std::vector<int32_t> e2;
    e2.reserve((size_t)i2 * 2);
    for (size_t i = 0; i < p2.size(); ++i) {
        const int j = h2[(size_t)p2[i]];
        const MLin &m = tab[(size_t)j];
        const int64_t local = p2[i] - m.item2;
        const int tiles = (int)imin(m.rows2 / kRG, cdiv(m.d_out - local * m.rows2, kRG));
        e2.push_back(j);
        e2.push_back((int32_t)(((local * (m.rows2 / kRG)) << 8) | tiles));
    }
    run.items2P = (int64_t)e2.size() / 2;
    put(G.ordP1, p1.data(), (size_t)i1 * 4);
    put(G.tabP2, e2.data(), e2.size() * 4);
    hs->n = n;
    run.T = (int)T;
    run.x_dtype = ls[0].x_dtype;
    run.y_dtype = y_dtype;
    run.items0 = i0;
    run.items1 = i1;
    run.itemsF = iF;
    run.items2 = i2;
    run.table = (const MLin *)(w + G.table);
    run.lin0 = (const int32_t *)(w + G.lin0);
    run.lin1 = (const int32_t *)(w + G.lin1);
    run.linF = (const int32_t *)(w + G.linF);
    run.lin2 = (const int32_t *)(w + G.lin2);
    run.ord1 = (const int32_t *)(w + G.ord1);
    run.ord2 = (const int32_t *)(w + G.ord2);
    run.ordP1 = (const int32_t *)(w + G.ordP1);
    run.tabP2 = (const int32_t *)(w + G.tabP2);
    run.arrive = (uint32_t *)(w + G.arrive);
    run.sync = (uint32_t *)(w + G.sync);
    run.stamp = (const uint64_t *)w;
    run.tag = tag;
    run.spin_limit = fault_test ? kSpinLimitTest : kSpinLimit;
    run.want_extra = fault_test ? 1u : 0u;
    // one launch per run when stage 1 is the fused form and stage 2 k_stage2r,
    // and each linear's events fit the 16-bit halves of its sync word
    run.pass = pass_tokens(hs->s, T) && run.dma2 && i1 > 0 && i2 > 0 ? 1 : 0;
    for (int j = 0; j < n; ++j) {
        const MLin &m = tab[(size_t)j];
        if ((int64_t)m.P * m.nrg + m.n2 >= 0xffff) run.pass = 0;
    }
    hs->lds_pass = 0;
    if (run.pass) {
        const size_t l2 = ops2r_bytes(run.ops2, hs->s.NB2, rows2(hs->s, T)) + 2 * kHRows * 2 +
                          (run.ystage ? (size_t)T * kHRows * run.yst : 0);
        // a latent group's (token, plane) units staged as NL records each
        const size_t lat = (size_t)T * run.flush1 * 2 * hs->s.NL * kRec;
        hs->lds_pass = std::max(std::max(hs->lds.s1, lat), l2);
        if (hs->lds_pass > 160 * 1024 - 64) run.pass = 0;
    }
    return LB_OK;
}

size_t mfma_group_state_bytes() { return sizeof(MGroupHost); }

template <int NL, int NB2, bool XM = false>
int launch_pass(const MRun &run, size_t lds, hipStream_t st) {
    static bool raised = false;        // once per instantiation (idempotent if raced)
    if (!raised) {
        if (hipFuncSetAttribute((const void *)k_pass<NL, NB2, XM>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024 - 64) != hipSuccess)
            return hip_status(hipGetLastError());
        raised = true;
    }
    MLin dummy{};
    k_pass<NL, NB2, XM><<<(unsigned)(run.items1 + run.items2P), kThreads, lds, st>>>(run, dummy);
    return last_launch_status();
}

int mfma_group_run(const void *host_state, hipStream_t st, int stage_mask) {
    const MGroupHost *hs = (const MGroupHost *)host_state;
    const MRun &r = hs->run;
    // every launch of a group looks its items up in these tables
    if (!r.table || (r.items0 > 0 && !r.lin0) || (r.items1 > 0 && !r.lin1) || (r.itemsF > 0 && !r.linF) ||
        (r.items2 > 0 && !r.lin2))
        return LB_EINVAL;
    if (stage_mask == 3 && r.pass) {
        if (!r.ordP1 || !r.tabP2 || !r.arrive || !r.sync || r.items2P != r.items2) return LB_EINVAL;
        const int key = hs->s.NL * 10 + hs->s.NB2;
        switch (key) {
            case 21: return launch_pass<2, 1>(r, hs->lds_pass, st);
            case 22: return launch_pass<2, 2>(r, hs->lds_pass, st);
            case 31: return launch_pass<3, 1>(r, hs->lds_pass, st);
            case 32: return launch_pass<3, 2>(r, hs->lds_pass, st);
        }
        return LB_EUNSUPPORTED;
    }
    MLin dummy{};
    return launch_shape(hs->s, hs->run, dummy, hs->lds, st, stage_mask);
}

// ---- inline groups -----------------------------------------------------------

namespace {
// The schedule of up to kMaxInline linears in the kernel arguments; returns
// the workspace bytes (each linear's scratch, back to back, then, for the
// one-launch form, the latent-group and per-linear counters).  The one-launch
// form (k_pass) is taken under the same conditions as for a group; its
// workspace must be all zero when the launch starts (the caller clears it;
// the pass leaves the counters at zero, not the rest).
size_t inline_setup(const Linear *ls, int n, uint8_t *ws, Shape *s, MRun *run, Lds *lds, size_t *lds_pass) {
    *run = MRun{};
    *lds = Lds{};
    *lds_pass = 0;
    if (n < 1 || n > kMaxInline || !shape_for(ls[0].T, ls[0].y_dtype, s)) return 0;
    const Grain gr = group_grain(ls, n, *s);
    size_t off = 0;
    int64_t i0 = 0, i1 = 0, iF = 0, i2 = 0, nf = 0;
    int steps_max = 1;
    int64_t ntile_max = 1;
    for (int j = 0; j < n; ++j) {
        MLin &m = run->inl[j];
        const size_t b = plan_linear(ls[j], *s, true, &m, gr);
        if (ws) bind_ws(&m, ls[j], *s, ws + off);
        off += b;
        m.item0 = i0;
        m.item1 = i1;
        m.itemF = iF;
        m.item2 = i2;
        m.fin0 = nf;
        i0 += items0_of(m);
        i1 += items1_of(m);
        iF += itemsF_of(m);
        i2 += m.n2;
        nf += groups_of(m);
        steps_max = (int)imax(steps_max, m.kgs);
        ntile_max = imax(ntile_max, cdiv(m.r_p, kTile));
    }
    run->ninl = n;
    for (int j = 0; j < n; ++j)
        if (ls[j].xm_dh) run->xmap = 1;
    if (run->xmap && !(fused1(*s) && s->NL == 2)) return 0;    // input maps: fused stage 1, bf16 out
    run->T = (int)ls[0].T;
    run->x_dtype = ls[0].x_dtype;
    run->y_dtype = ls[0].y_dtype;
    run->dma2 = dma2_for(*s, ls[0].T, steps_max);
    run->yst = yst_for(ls, n, ls[0].y_dtype);
    run->ystage = ystage_for(ls[0].T, run->yst);
    run->ops2 = run->dma2 ? steps_max : ops2_for(*s, steps_max);
    run->items0 = i0;
    run->items1 = i1;
    run->itemsF = iF;
    run->items2 = i2;
    run->tsplit = gr.tsplit;
    run->flush1 = (int)imin(imin(flush1_for(ls[0].T, run->tsplit), ntile_max), gr.f_cap);
    for (int j = 0; j < n; ++j) lds_add(lds, run->inl[j], *s, run->ops2, ls[0].T, run->flush1, run->tsplit);
    // the one-launch form: as a group takes it (pass_form, the 16-bit event
    // halves, the LDS of one CU)
    const int64_t T = ls[0].T;
    bool pass = pass_tokens(*s, T) && run->dma2 && i1 > 0 && i2 > 0;
    for (int j = 0; j < n; ++j)
        if ((int64_t)run->inl[j].P * run->inl[j].nrg + run->inl[j].n2 >= 0xffff) pass = false;
    size_t lp = 0;
    if (pass) {
        const size_t l2 = ops2r_bytes(run->ops2, s->NB2, rows2(*s, T)) + 2 * kHRows * 2 +
                          (run->ystage ? (size_t)T * kHRows * run->yst : 0);
        const size_t lat = (size_t)T * run->flush1 * 2 * s->NL * kRec;
        lp = std::max(std::max(lds->s1, lat), l2);
        if (lp > 160 * 1024 - 64) pass = false;
    }
    if (pass) {
        const size_t ctrl = rup256(off), arrive = rup256((size_t)nf * kFlagStride * 4);
        if (ws) {
            run->arrive = (uint32_t *)(ws + ctrl);
            run->sync = (uint32_t *)(ws + ctrl + arrive);
        }
        run->pass = 1;
        run->items2P = i2;
        run->spin_limit = kSpinLimit;
        *lds_pass = lp;
        off = ctrl + arrive + rup256((size_t)n * kFlagStride * 4);
    }
    return off;
}

int launch_pass_shape(const Shape &s, const MRun &run, size_t lds, hipStream_t st) {
    if (run.xmap) return s.NL == 2 && s.NB2 == 1 ? launch_pass<2, 1, true>(run, lds, st) : LB_EUNSUPPORTED;
    switch (s.NL * 10 + s.NB2) {
        case 21: return launch_pass<2, 1>(run, lds, st);
        case 22: return launch_pass<2, 2>(run, lds, st);
        case 31: return launch_pass<3, 1>(run, lds, st);
        case 32: return launch_pass<3, 2>(run, lds, st);
    }
    return LB_EUNSUPPORTED;
}
}  // namespace

bool mfma_inline_pass(const Linear *ls, int n) {
    Shape s;
    MRun run;
    Lds lds;
    size_t lp;
    return inline_setup(ls, n, nullptr, &s, &run, &lds, &lp) > 0 && run.pass;
}

size_t mfma_inline_workspace_bytes(const Linear *ls, int n) {
    Shape s;
    MRun run;
    Lds lds;
    size_t lp;
    return inline_setup(ls, n, nullptr, &s, &run, &lds, &lp);
}

int mfma_inline_forward(const Linear *ls, int n, void *ws, hipStream_t st, bool zeroed) {
    Shape s;
    MRun run;
    Lds lds;
    size_t lp;
    const size_t bytes = inline_setup(ls, n, (uint8_t *)ws, &s, &run, &lds, &lp);
    if (bytes == 0) return LB_EUNSUPPORTED;
    if (run.pass) {
        if (!zeroed)
            if (int rc = fill_words(ws, bytes, 0u, st)) return rc;
        return launch_pass_shape(s, run, lp, st);
    }
    MLin dummy{};
    return launch_shape(s, run, dummy, lds, st);
}

// ---- the fault word ----------------------------------------------------------

namespace {
__global__ void k_take_faults(uint32_t *out) {
    *out = __hip_atomic_exchange(&g_lb_faults, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__global__ void k_fill_words(uint32_t *a, int64_t n, uint32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        a[i] = v;
}
}  // namespace

int take_faults(hipStream_t st, uint32_t *faults) {
    // one word per device for the exchanged value, found once per device
    static uint32_t *out_dev[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hip_status(hipGetLastError());
    if (!out_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_lb_faults_out)) != hipSuccess) return hip_status(hipGetLastError());
        out_dev[dev] = (uint32_t *)p;
    }
    k_take_faults<<<1, 1, 0, st>>>(out_dev[dev]);
    if (int rc = last_launch_status()) return rc;
    uint32_t v = 0;
    if (hipMemcpyAsync(&v, out_dev[dev], 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return hip_status(hipGetLastError());
    *faults = v;
    return LB_OK;
}

int fill_words(void *p, size_t bytes, uint32_t v, hipStream_t st) {
    const int64_t n = (int64_t)(bytes / 4);
    if (n <= 0) return LB_OK;
    k_fill_words<<<(unsigned)imin(2048, cdiv(n, 256)), 256, 0, st>>>((uint32_t *)p, n, v);
    return last_launch_status();
}

}  // namespace lb
