// lb_gemm.hip -- prefill path (many tokens) of the LittleBit forward on bf16 matrix cores.
//
// Proposition 1 (sesamedisk page, "What the method actually computes") over a
// block of T tokens is two skinny GEMMs with diagonal scalings between them:
//   stage 1:  u = X . (diag(g_p) sign(V_p))        M = T, N = latents of all paths, K = d_in
//             t = l (.) u, rounded to bf16         (the rank-r intermediate, workspace)
//   stage 2:  y = t . (sign(U_p)^T diag(h_p))      M = T, N = d_out, K = latents of all paths
// Both run as v_mfma_f32_32x32x16_bf16 with fp32 accumulation ("two smaller
// binary matmuls with FP16 element-wise scaling between them", same page, the
// compute paragraph; the scales enter rounded to bf16 here).
//
// Sign operand: multiplying by -1 is a sign flip (same page, the note after
// the proposition), so each operand pair is a bf16 scale pair (g per
// contraction element in stage 1, h per output column in stage 2) whose sign
// bits are flipped where the packed bit is 1.  While a K-tile is staged, each
// packed word is "unzipped" once (even bits to the low half, odd bits to the
// high half); a pair of adjacent elements is then one shift, one AND and one
// XOR away: ((X << c) & 0x80008000) ^ scale_pair.
//
// The product is computed transposed, D = S . A^T (signs as the first
// operand), so the accumulator quad of a lane holds 4 consecutive output
// columns of one token: one 8-byte store of bf16.
//
// Tiles: 256 tokens x 128 columns, K-tiles of 64 elements double-buffered in
// LDS (activations with a 16-byte XOR swizzle, unzipped sign words, scales),
// 4 waves of 128 x 64.  Stage 1 splits d_in into pieces of at most 8192 when
// it is longer; a reduce pass then adds the pieces in order.  A launch covers
// every linear of a group (a table maps work items to linears), and work items
// are renumbered so that each of the 8 XCDs (own L2) gets a contiguous range:
// neighbouring tiles share their activation rows.
#include <vector>

#include "lb_internal.h"

namespace lb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

namespace {

constexpr int kBM = 256;                     // tokens per tile
constexpr int kBK = 64;                      // contraction elements per K-tile (two packed words)
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowBytes = kBK * 2;           // one activation row of a K-tile (bf16)
constexpr int kABytes = kBM * kRowBytes;     // 32 KB
constexpr int kGWave = 2 * kBK * 2;          // a wave's bf16 g: [2 paths][kBK]

// Two tile shapes, by n-blocks (32 columns) per wave NBW; waves are 2 x 2:
//   NBW = 2: 256 x 128 tiles, 128 x 64 per wave, 2-slot ring (70 KB): two
//            workgroups per CU (stage 1: few, long tiles)
//   NBW = 4: 256 x 256 tiles, 128 x 128 per wave (accumulators in AGPRs),
//            4-slot ring (148 KB): one workgroup per CU, three K-tiles in flight
template <int NBW> struct Shape {
    static constexpr int BN = 64 * NBW;
    static constexpr int XWave = 2 * NBW * 32 * 4;     // a wave's sign words: [2 words][NBW*32]
    static constexpr int Slot = kABytes + kWaves * (XWave + kGWave);
    static constexpr int Stages = NBW == 4 ? 4 : 2;
    static constexpr int Lds = Stages * Slot;
};
constexpr int kNBW1 = 2, kNBW2 = 2;          // stage 1, stage 2
constexpr int kBN1 = Shape<kNBW1>::BN, kBN2 = Shape<kNBW2>::BN;
constexpr int kWG1 = 512;                    // stage-1 workgroups a launch aims for: two per
                                             // CU on 256 CUs, so no CU runs a second round
constexpr uint32_t kOOB = 0x7ffffff0u;       // a buffer offset past every range: reads as zero

// One linear of a prefill launch.
struct GLin {
    const void *x;        // [T][d_in] bf16 (fp32 inputs are converted first)
    void *y;
    const uint32_t *v_bits, *u_bits;
    const uint16_t *g, *l, *h;
    uint16_t *t;          // [T][ldt] bf16 latents; zero outside the P*r_p real ones
    uint16_t *gb;         // [P][d_in] g rounded to bf16          (written by k_prep)
    uint32_t *vz, *uz;    // V and U sign words, unzipped, planes of zld_v / zld_u words
    float *part;          // [nsplit][T][ldt] fp32 stage-1 pieces (nsplit > 1)
    int64_t ld_v, ld_u, d_in, d_out;
    int64_t zld_v, zld_u; // plane strides of vz / uz: r_p and d_out rounded up to 4
    int32_t r_p, P;
    int32_t kw;           // packed words per path along r_p (= U planes per path)
    int32_t kw_v;         // packed words along d_in (= V planes per path)
    int32_t ldt;          // latent row stride: P*kw*32 rounded up to kBK
    int32_t nsplit, ktps; // stage-1 pieces and K-tiles per piece
    int32_t nkt1, nkt2;   // K-tiles of stage 1 (d_in) and stage 2 (ldt)
    int32_t mt, nt1, nt2; // token tiles; column tiles of stage 1 (ldt) and stage 2 (d_out)
    int32_t nred;         // reduce items (nsplit > 1), 0 otherwise
    int32_t ngp;          // prep items
    int64_t itemG, item1, itemR, item2;
};

struct GRun {
    int T, y_dtype, pad0_, pad1_;
    int64_t itemsG, items1, itemsR, items2;
    const GLin *table;                       // null: the single linear passed by value
    const int32_t *linG, *lin1, *linR, *lin2;   // item -> linear, per launch
};

// Work item v of n for block b: each XCD (blocks b % 8) takes a contiguous range.
__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t n) {
    const int64_t x = b & 7, j = b >> 3;
    const int64_t per = n >> 3, rem = n & 7;
    return x * per + (x < rem ? x : rem) + j;
}

// The linear of work item v as a wave-uniform value (matrix instructions ignore
// the exec mask, so every branch around them must be uniform).
__device__ __forceinline__ GLin pick(const GRun &run, const GLin &single, const int32_t *map,
                                     int64_t v) {
    GLin m = run.table ? run.table[map[v]] : single;
    static_assert(sizeof(GLin) % 4 == 0, "GLin is copied as 32-bit words");
    int w[sizeof(GLin) / 4];
    __builtin_memcpy(w, &m, sizeof(GLin));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(GLin) / 4); ++i) w[i] = __builtin_amdgcn_readfirstlane(w[i]);
    __builtin_memcpy(&m, w, sizeof(GLin));
    return m;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
    const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, n, 0x00020000);
}

typedef __attribute__((address_space(3))) void lds_void;

// Global -> LDS without registers: lane i's `size` bytes land at dst + size*i
// (dst wave-uniform); offsets past the descriptor's range read as zero.
template <int SIZE>
__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t voff) {
    static_assert(SIZE == 4 || SIZE == 16, "LDS load size");
    if constexpr (SIZE == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, (int)voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 4, (int)voff, 0, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are outstanding,
// then meet the other waves: their loads before the wait are in LDS too.
template <int N>
__device__ __forceinline__ void wait_and_meet() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Even bits of x to the low half, odd bits to the high half (inverse perfect
// shuffle by four delta swaps).
__device__ __forceinline__ uint32_t unzip_bits(uint32_t x) {
    uint32_t t;
    t = (x ^ (x >> 1)) & 0x22222222u; x ^= t ^ (t << 1);
    t = (x ^ (x >> 2)) & 0x0C0C0C0Cu; x ^= t ^ (t << 2);
    t = (x ^ (x >> 4)) & 0x00F000F0u; x ^= t ^ (t << 4);
    t = (x ^ (x >> 8)) & 0x0000FF00u; x ^= t ^ (t << 8);
    return x;
}

// two fp32 -> two bf16 in one word (v_cvt_pk_bf16_f32: round to nearest even)
// 16-byte chunk position of chunk c in activation row r of a K-tile: rows
// 0..7 and rows 0..15 of one parity all use different positions, so an 8- or
// 16-lane phase of a 16-byte LDS read touches every bank once (32 or 64 banks).
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ __forceinline__ f32x16 mfma(const u32x4 &s, const u32x4 &a, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, s),
                                                   __builtin_bit_cast(bf16x8, a), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// the two GEMM stages
// ---------------------------------------------------------------------------

// STAGE 1: A = x (bf16), sign words of V, scales g; output t (bf16, l applied)
//          or fp32 pieces.
// STAGE 2: A = t (bf16), sign words of U, scales h; output y.
template <int STAGE, int NBW>
__global__ __launch_bounds__(kThreads, NBW == 4 ? 1 : 2) void k_gemm(GRun run, GLin single) {
    using SH = Shape<NBW>;
    constexpr int BN = SH::BN, XWave = SH::XWave, Slot = SH::Slot, Stages = SH::Stages;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int64_t items = STAGE == 1 ? run.items1 : run.items2;
    const int64_t v = xcd_order(blockIdx.x, items);
    const GLin L = pick(run, single, STAGE == 1 ? run.lin1 : run.lin2, v);
    const int64_t local = v - (STAGE == 1 ? L.item1 : L.item2);
    // item = (piece of d_in [stage 1], token tile, column tile)
    const int nt = STAGE == 1 ? L.nt1 : L.nt2;
    const int ni = (int)(local % nt);
    const int mi = (int)((local / nt) % L.mt);
    const int split = STAGE == 1 ? (int)(local / ((int64_t)nt * L.mt)) : 0;
    const int T = run.T;
    const int64_t m0 = (int64_t)mi * kBM;
    const int n0 = ni * BN;
    const int kt0 = STAGE == 1 ? split * L.ktps : 0;
    const int kt1 = STAGE == 1 ? (int)imin(L.nkt1, kt0 + L.ktps) : L.nkt2;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, l32 = lane & 31;
    const int wm = wave & 1, wn = wave >> 1;
    const int nw0 = n0 + wn * NBW * 32;                       // this wave's first column

    // ---- loads of one K-tile (per wave: 8 activation DMAs, NBW sign-word DMAs, 1 g DMA) ----
    // activations: wave w fills rows 64w .. 64w+63, 8 rows (1 KB) per DMA; lane i
    // lands in row r = r0 + i/8 at position i%8, which holds chunk (i%8) ^ swz(r)
    const int64_t K = STAGE == 1 ? L.d_in : L.ldt;
    const int rows = (int)imin(kBM, (int64_t)T - m0);
    const uint8_t *abase = STAGE == 1 ? (const uint8_t *)L.x : (const uint8_t *)L.t;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(abase + m0 * K * 2, (int64_t)rows * K * 2);
    // (rows r0 .. r0+7 with r0 = 64w + 8i: swz(r) = (i/8 % 8) ^ (i & 1))
    const int arow0 = wave * 64 + (lane >> 3);               // + 8i
    const int ach0 = (lane & 7) ^ ((lane >> 3) & 7);          // chunk for even i
    const int ach1 = ach0 ^ 1;                                // chunk for odd i
    const uint32_t aoffe = (uint32_t)(arow0 * K * 2) + (uint32_t)(ach0 * 16);
    const uint32_t aoffo = (uint32_t)(arow0 * K * 2) + (uint32_t)(ach1 * 16);
    const uint32_t astep = (uint32_t)(8 * K * 2);            // 8 rows
    // sign words: this wave's columns nw0 + 64c + lane, c < NBW/2, both words of the K-tile
    __amdgpu_buffer_rsrc_t rx;
    uint32_t xoff[NBW / 2], xstep;
    int xwords;
    if (STAGE == 1) {
        rx = make_rsrc(L.vz, (int64_t)L.P * L.kw_v * L.zld_v * 4);
#pragma unroll
        for (int c = 0; c < NBW / 2; ++c) {
            const int xn = nw0 + 64 * c + lane;
            const int qn = xn >> 5;
            const int p = qn / L.kw;
            const int k = (qn - p * L.kw) * 32 + (xn & 31);
            xoff[c] = (p < L.P && k < L.r_p) ? (uint32_t)(((int64_t)p * L.kw_v * L.zld_v + k) * 4) : kOOB;
        }
        xstep = (uint32_t)(L.zld_v * 4);
        xwords = L.kw_v;
    } else {
        rx = make_rsrc(L.uz, (int64_t)L.P * L.kw * L.zld_u * 4);
#pragma unroll
        for (int c = 0; c < NBW / 2; ++c) {
            const int xn = nw0 + 64 * c + lane;
            xoff[c] = xn < L.d_out ? (uint32_t)(xn * 4) : kOOB;
        }
        xstep = (uint32_t)(L.zld_u * 4);
        xwords = L.P * L.kw;
    }
    // g (stage 1, bf16): lane i -> path i/32, elements 2(i%32), +1 of the K-tile
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(L.gb, (int64_t)L.P * L.d_in * 2);
    const int gpath = lane >> 5, gel = 2 * (lane & 31);

    auto issue = [&](int kt, int slot) {
        uint8_t *S = smem + slot * Slot;
        const bool kine = kt * kBK + 8 * ach0 < K;            // chunk inside the row
        const bool kino = kt * kBK + 8 * ach1 < K;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool kin = (i & 1) ? kino : kine;
            const uint32_t off = ((i & 1) ? aoffo : aoffe) + i * astep + (uint32_t)(kt * kBK * 2);
            dma<16>(ra, S + (wave * 64 + 8 * i) * kRowBytes, kin ? off : kOOB);
        }
        uint8_t *X = S + kABytes + wave * (XWave + kGWave);
#pragma unroll
        for (int wd = 0; wd < 2; ++wd) {
            const int q = kt * 2 + wd;
#pragma unroll
            for (int c = 0; c < NBW / 2; ++c)
                dma<4>(rx, X + (wd * NBW * 32 + 64 * c) * 4,
                       (xoff[c] != kOOB && q < xwords) ? xoff[c] + (uint32_t)q * xstep : kOOB);
        }
        if (STAGE == 1) {
            const int64_t e = (int64_t)kt * kBK + gel;
            dma<4>(rg, X + XWave, e < L.d_in ? (uint32_t)((gpath * L.d_in + e) * 2) : kOOB);
        }
    };
    constexpr int kIssued = 8 + NBW + (STAGE == 1 ? 1 : 0);   // DMAs per K-tile per wave

    // ---- per-lane constants of the sign operands ----
    int gofs[NBW];           // stage 1: byte offset of this lane's g run (path of the column)
    uint32_t hpair[NBW][2];  // stage 2: bf16 h pair per n-block and path
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        const int n = nw0 + b * 32 + l32;
        if (STAGE == 1) {
            const int p = (n >> 5) / L.kw;
            gofs[b] = (p < L.P ? p : 0) * kBK * 2 + hh * 16;
        } else {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const float hv = (p < L.P && n < L.d_out) ? f16_to_f32(L.h[(int64_t)p * L.d_out + n]) : 0.0f;
                hpair[b][p] = bf16_pair(hv, hv);
            }
        }
    }
    const uint32_t xshift = 4u - 4u * (uint32_t)hh;

    // stage 1 without pieces: l for this lane's output columns (4 per accumulator
    // quad), loaded before the K loop.  r_p is a multiple of 16, so a run of 4
    // columns is all real latents or all padding.
    u32x2 lsc[NBW][4];
    uint32_t lok = 0;                                  // bit 4b+q4: run of real latents
    if (STAGE == 1 && L.nsplit == 1) {
        const uint16_t *lp[NBW][4];
#pragma unroll
        for (int b = 0; b < NBW; ++b)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int n = nw0 + b * 32 + 8 * q4 + 4 * hh;
                const int qn = n >> 5;
                const int p = qn / L.kw;
                const int k = (qn - p * L.kw) * 32 + (n & 31);
                const bool ok = n < L.ldt && p < L.P && k < L.r_p;
                lok |= (ok ? 1u : 0u) << (4 * b + q4);
                lp[b][q4] = L.l + (ok ? (int64_t)p * L.r_p + k : 0);
            }
        if (((uintptr_t)L.l & 7) == 0) {
#pragma unroll
            for (int b = 0; b < NBW; ++b)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) lsc[b][q4] = *(const u32x2 *)lp[b][q4];
        } else {
#pragma unroll
            for (int b = 0; b < NBW; ++b)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const uint16_t *q = lp[b][q4];
                    lsc[b][q4] = u32x2{(uint32_t)q[0] | ((uint32_t)q[1] << 16),
                                       (uint32_t)q[2] | ((uint32_t)q[3] << 16)};
                }
        }
    }

    f32x16 acc[NBW][4];
#pragma unroll
    for (int b = 0; b < NBW; ++b)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][mb][i] = 0.0f;

    // One K-tile = 4 steps of 16 elements (step st: word st/2, half st%2).
    auto compute = [&](int slot, int kt) {
        const uint8_t *A = smem + slot * Slot;
        const uint8_t *Xw = A + kABytes + wave * (XWave + kGWave);
        const uint8_t *G = Xw + XWave;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int w2 = st >> 1, s = st & 1;
            u32x4 act[4];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const int row = wm * 128 + mb * 32 + l32;
                const int chunk = 2 * st + hh;
                act[mb] = *(const u32x4 *)(A + row * kRowBytes + ((chunk ^ swz(row)) << 4));
            }
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                const uint32_t xs = ((const uint32_t *)Xw)[w2 * NBW * 32 + b * 32 + l32] << xshift;
                u32x4 sc;
                if (STAGE == 1) {
                    sc = *(const u32x4 *)(G + gofs[b] + (32 * w2 + 16 * s) * 2);
                } else {
                    const uint32_t hp = (kt * 2 + w2) >= L.kw ? hpair[b][1] : hpair[b][0];
                    sc = u32x4{hp, hp, hp, hp};
                }
                u32x4 sg;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    sg[jj] = sc[jj] ^ ((xs << (11 - 8 * s - jj)) & 0x80008000u);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) acc[b][mb] = mfma(sg, act[mb], acc[b][mb]);
            }
        }
    };

    // ---- K loop over a ring of Stages slots ----
    // At the top of iteration kt the tiles kt .. kt+Stages-2 have been issued;
    // after the wait and the barrier tile kt is in LDS for every wave and the
    // slot of tile kt-1 is free again, so tile kt+Stages-1 is issued into it.
#pragma unroll
    for (int j = 0; j < Stages - 1; ++j)
        if (kt0 + j < kt1) issue(kt0 + j, j);
    for (int kt = kt0; kt < kt1; ++kt) {
        const int slot = (kt - kt0) % Stages;
        if (kt + Stages - 2 < kt1) wait_and_meet<(Stages - 2) * kIssued>();
        else wait_and_meet<0>();
        if (kt + Stages - 1 < kt1) issue(kt + Stages - 1, (slot + Stages - 1) % Stages);
        compute(slot, kt);
    }

    // ---- epilogue ----
    // The lane holds columns n .. n+3 of token m per accumulator quad.  Each
    // wave stages 64 rows of its tile at a time in its own part of the (now
    // idle) ring and writes them back as whole 16-byte chunks of rows, through
    // a buffer descriptor over this token tile's rows: rows past T fall outside
    // the range and are dropped.
    const int64_t ld_out = STAGE == 1 ? L.ldt : L.d_out;
    const int64_t n_lim = STAGE == 1 ? L.ldt : L.d_out;       // columns that exist
    const int osz = STAGE == 1 ? (L.nsplit > 1 ? 4 : 2) : (run.y_dtype == LB_BF16 ? 2 : 4);
    const uint8_t *obase = STAGE == 1
        ? (L.nsplit > 1 ? (const uint8_t *)(L.part + (int64_t)split * T * L.ldt) : (const uint8_t *)L.t)
        : (const uint8_t *)L.y;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(obase + m0 * ld_out * osz, (int64_t)rows * ld_out * osz);
    constexpr int WC = NBW * 32;                               // columns of a wave
    const int rbytes = WC * osz + 16;                          // staged row (padded)
    uint8_t *stage = smem + wave * 64 * (WC * 4 + 16);         // room for the fp32 case
    // whole 16-byte chunks only when every row starts 16-byte aligned
    const bool chunky = ((ld_out * osz) % 16) == 0 && ((uintptr_t)obase % 16) == 0;
    wait_and_meet<0>();                                        // every wave is done with the ring
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        // accumulators -> LDS (l applied for stage-1 latents)
#pragma unroll
        for (int mh = 0; mh < 2; ++mh) {
            const int mb = 2 * half + mh;
            uint8_t *rowp = stage + (mh * 32 + l32) * rbytes;
#pragma unroll
            for (int b = 0; b < NBW; ++b)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x16 &a = acc[b][mb];
                    float o0 = a[4 * q4], o1 = a[4 * q4 + 1], o2 = a[4 * q4 + 2], o3 = a[4 * q4 + 3];
                    const int c = b * 32 + 8 * q4 + 4 * hh;          // column within the wave
                    if (STAGE == 1 && L.nsplit == 1) {
                        const u32x2 w = lsc[b][q4];
                        const bool ok = (lok >> (4 * b + q4)) & 1u;   // padding columns stay zero
                        o0 = ok ? f16_to_f32((uint16_t)(w[0] & 0xffffu)) * o0 : 0.0f;
                        o1 = ok ? f16_to_f32((uint16_t)(w[0] >> 16)) * o1 : 0.0f;
                        o2 = ok ? f16_to_f32((uint16_t)(w[1] & 0xffffu)) * o2 : 0.0f;
                        o3 = ok ? f16_to_f32((uint16_t)(w[1] >> 16)) * o3 : 0.0f;
                    }
                    if (osz == 2)
                        *(u32x2 *)(rowp + c * 2) = u32x2{bf16_pair(o0, o1), bf16_pair(o2, o3)};
                    else
                        *(f32x4 *)(rowp + c * 4) = f32x4{o0, o1, o2, o3};
                }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's LDS writes land
        // LDS -> global: 64 rows x WC columns in 16-byte chunks, lane order row-major
        const int cpr = WC * osz / 16;                         // chunks per row
        const int nchunks = 64 * cpr;
        for (int ci = lane; ci < nchunks; ci += 64) {
            const int r = ci / cpr, ch = ci - r * cpr;
            const int col = ch * (16 / osz);                   // first column of the chunk
            const int n = nw0 + col;
            const u32x4 val = *(const u32x4 *)(stage + r * rbytes + ch * 16);
            const uint32_t off =
                (uint32_t)(((wm * 128 + half * 64 + r) * ld_out + n) * osz);
            const int per = 16 / osz;
            if (chunky && n + per <= n_lim) {
                // non-temporal: the outputs stream out instead of filling the L2
                // that holds the activation rows other tiles still read
                __builtin_amdgcn_raw_buffer_store_b128(val, ro, (int)off, 0, 2);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (e >= per || n + e >= n_lim) break;
                    if (osz == 2)
                        __builtin_amdgcn_raw_buffer_store_b16(
                            (unsigned short)((val[e >> 1] >> (16 * (e & 1))) & 0xffffu), ro, (int)(off + 2 * e), 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b32(val[e], ro, (int)(off + 4 * e), 0, 0);
                }
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next half
    }
}

// Per-call operand preparation: g -> bf16 (round to nearest even) for the
// stage-1 sign operands, and every packed sign word of V and U unzipped (even
// bits to the low half, odd bits to the high half) for both stages.
constexpr int kPrep = 1024;       // words per item

__global__ __launch_bounds__(kThreads) void k_prep(GRun run, GLin single) {
    const int64_t v = blockIdx.x;
    const GLin L = pick(run, single, run.linG, v);
    const int64_t local = v - L.itemG;
    const int64_t ng = (int64_t)L.P * L.d_in / 2;                 // g pairs
    const int64_t nv = (int64_t)L.P * L.kw_v * L.zld_v;           // V words (compact)
    const int64_t nu = (int64_t)L.P * L.kw * L.zld_u;             // U words (compact)
    for (int i = threadIdx.x; i < kPrep; i += kThreads) {
        int64_t e = local * kPrep + i;
        if (e < ng) {
            const uint32_t w = ((const uint32_t *)L.g)[e];
            ((uint32_t *)L.gb)[e] = bf16_pair(f16_to_f32((uint16_t)(w & 0xffffu)), f16_to_f32((uint16_t)(w >> 16)));
            continue;
        }
        e -= ng;
        if (e < nv) {
            const int64_t pl = e / L.zld_v;
            L.vz[e] = unzip_bits(L.v_bits[pl * L.ld_v + (e - pl * L.zld_v)]);
            continue;
        }
        e -= nv;
        if (e < nu) {
            const int64_t pl = e / L.zld_u;
            L.uz[e] = unzip_bits(L.u_bits[pl * L.ld_u + (e - pl * L.zld_u)]);
        }
    }
}

// Stage-1 pieces -> t: the pieces are added in order, then scaled by l.
// Item = kRedGroups groups of 4 latents (one token row segment each).
constexpr int kRedGroups = 1024;

__global__ __launch_bounds__(kThreads) void k_reduce(GRun run, GLin single) {
    const int64_t v = blockIdx.x;
    const GLin L = pick(run, single, run.linR, v);
    const int64_t local = v - L.itemR;
    const int T = run.T;
    const int64_t groups = (int64_t)T * (L.ldt / 4);
    const int64_t stride = (int64_t)T * L.ldt;
    for (int i = threadIdx.x; i < kRedGroups; i += kThreads) {
        const int64_t gi = local * kRedGroups + i;
        if (gi >= groups) break;
        const int64_t m = gi / (L.ldt / 4);
        const int n = (int)(gi - m * (L.ldt / 4)) * 4;
        f32x4 s = *(const f32x4 *)(L.part + m * L.ldt + n);
        for (int sp = 1; sp < L.nsplit; ++sp) {
            const f32x4 a = *(const f32x4 *)(L.part + sp * stride + m * L.ldt + n);
            s[0] += a[0];
            s[1] += a[1];
            s[2] += a[2];
            s[3] += a[3];
        }
        const int qn = n >> 5;
        const int p = qn / L.kw;
        const int k = (qn - p * L.kw) * 32 + (n & 31);
        float tv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            tv[e] = (p < L.P && k + e < L.r_p) ? f16_to_f32(L.l[(int64_t)p * L.r_p + k + e]) * s[e] : 0.0f;
        *(u32x2 *)(L.t + m * L.ldt + n) = u32x2{bf16_pair(tv[0], tv[1]), bf16_pair(tv[2], tv[3])};
    }
}

// fp32 activations -> bf16 (round to nearest even), 4 per thread.
__global__ __launch_bounds__(kThreads) void k_to_bf16(const float *__restrict__ x, uint16_t *__restrict__ xb,
                                                      int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n4) return;
    const f32x4 v = ((const f32x4 *)x)[i];
    ((u32x2 *)xb)[i] = u32x2{bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3])};
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

size_t rup256(size_t n) { return (n + 255) & ~(size_t)255; }

// Shapes the GEMM kernels take: 16-byte activation rows (d_in % 8 == 0), a
// 16-byte aligned x and a 4-byte aligned g (both are read by 16- and 4-byte
// LDS loads).  Others run on the vector-ALU kernels.
bool gemm_shape_ok(const Linear &a) {
    if (a.d_in % 8 != 0) return false;
    if (a.x && ((uintptr_t)a.x % 16) != 0) return false;
    if (a.g && ((uintptr_t)a.g % 4) != 0) return false;
    if (a.T > (1ll << 24)) return false;
    // 32-bit buffer offsets over one 256-token tile of activations or latents,
    // and over the packed words of one linear
    if (a.d_in >= (1ll << 21) || a.r_p >= (1ll << 19) || a.d_out >= (1ll << 20)) return false;
    if ((int64_t)a.P * cdiv(a.d_in, 32) * rup(a.r_p, 4) * 4 >= (1ll << 31)) return false;
    if ((int64_t)a.P * cdiv(a.r_p, 32) * rup(a.d_out, 4) * 4 >= (1ll << 31)) return false;
    return true;
}

// Schedule fields of one linear; returns the workspace bytes it needs (the
// latents, the stage-1 pieces and, for fp32 inputs, their bf16 copy).
// Stage-1 pieces (d_in splits) per linear for a launch over ls[0..n): start
// at one piece per tile and, while the launch stays within kWG1 workgroups,
// split further the linear whose pieces are longest (every tile of a linear
// takes one more piece).  Writes splits[j].
void stage1_splits(const Linear *ls, int n, std::vector<int> &splits) {
    std::vector<int64_t> nkt((size_t)n), tiles((size_t)n);
    int64_t used = 0;
    for (int j = 0; j < n; ++j) {
        const Linear &a = ls[j];
        const int64_t ldt = rup((int64_t)a.P * cdiv(a.r_p, 32) * 32, kBK);
        nkt[(size_t)j] = cdiv(a.d_in, kBK);
        tiles[(size_t)j] = cdiv(ldt, kBN1) * cdiv(a.T, kBM);
        used += tiles[(size_t)j];
    }
    splits.assign((size_t)n, 1);
    for (;;) {
        int best = -1;
        int64_t len = 0;
        for (int j = 0; j < n; ++j) {
            const int64_t l = cdiv(nkt[(size_t)j], splits[(size_t)j]);
            if (l > len && splits[(size_t)j] < nkt[(size_t)j]) { len = l; best = j; }
        }
        if (best < 0 || len <= 8 || used + tiles[(size_t)best] > kWG1) break;
        used += tiles[(size_t)best];
        ++splits[(size_t)best];
    }
}

size_t plan(const Linear &a, GLin *m, int nsplit) {
    *m = GLin{};
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
    m->zld_v = rup(a.r_p, 4);
    m->zld_u = rup(a.d_out, 4);
    m->kw = (int32_t)cdiv(a.r_p, 32);
    m->kw_v = (int32_t)cdiv(a.d_in, 32);
    m->ldt = (int32_t)rup((int64_t)a.P * m->kw * 32, kBK);
    m->nkt1 = (int32_t)cdiv(a.d_in, kBK);
    m->nsplit = (int32_t)imax(1, nsplit);
    m->ktps = (int32_t)cdiv(m->nkt1, m->nsplit);
    m->nsplit = (int32_t)cdiv(m->nkt1, m->ktps);
    m->nkt2 = m->ldt / kBK;
    m->mt = (int32_t)cdiv(a.T, kBM);
    m->nt1 = (int32_t)cdiv(m->ldt, kBN1);
    m->nt2 = (int32_t)cdiv(a.d_out, kBN2);
    m->nred = m->nsplit > 1 ? (int32_t)cdiv(a.T * (m->ldt / 4), kRedGroups) : 0;
    const int64_t nv = (int64_t)a.P * m->kw_v * m->zld_v, nu = (int64_t)a.P * m->kw * m->zld_u;
    m->ngp = (int32_t)cdiv((int64_t)a.P * a.d_in / 2 + nv + nu, kPrep);
    const size_t tb = rup256((size_t)a.T * m->ldt * 2);
    const size_t pb = m->nsplit > 1 ? rup256((size_t)m->nsplit * a.T * m->ldt * 4) : 0;
    const size_t gbb = rup256((size_t)a.P * a.d_in * 2);
    const size_t vzb = rup256((size_t)nv * 4), uzb = rup256((size_t)nu * 4);
    const size_t xb = rup256((size_t)a.T * a.d_in * 2);
    return tb + pb + gbb + vzb + uzb + xb;
}

// Workspace pointers; returns the bf16 copy of x (used when x is fp32).
uint16_t *bind(GLin *m, const Linear &a, uint8_t *ws) {
    const size_t tb = rup256((size_t)a.T * m->ldt * 2);
    const size_t pb = m->nsplit > 1 ? rup256((size_t)m->nsplit * a.T * m->ldt * 4) : 0;
    const size_t gbb = rup256((size_t)a.P * a.d_in * 2);
    const int64_t nv = (int64_t)a.P * m->kw_v * m->zld_v, nu = (int64_t)a.P * m->kw * m->zld_u;
    const size_t vzb = rup256((size_t)nv * 4), uzb = rup256((size_t)nu * 4);
    m->t = (uint16_t *)ws;
    m->part = m->nsplit > 1 ? (float *)(ws + tb) : nullptr;
    m->gb = (uint16_t *)(ws + tb + pb);
    m->vz = (uint32_t *)(ws + tb + pb + gbb);
    m->uz = (uint32_t *)(ws + tb + pb + gbb + vzb);
    return (uint16_t *)(ws + tb + pb + gbb + vzb + uzb);
}

int64_t items1_of(const GLin &m) { return (int64_t)m.nsplit * m.nt1 * m.mt; }
int64_t items2_of(const GLin &m) { return (int64_t)m.nt2 * m.mt; }

template <typename K>
int raise_lds(K kern, int bytes) {
    // > 64 KB of dynamic LDS needs an explicit opt-in (once per kernel; idempotent)
    static bool done = false;
    if (!done) {
        if (hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) !=
            hipSuccess)
            return hip_status(hipGetLastError());
        done = true;
    }
    return LB_OK;
}

int launch_gemms(const GRun &run, const GLin &single, hipStream_t st) {
    int rc;
    if (run.itemsG > 0) {
        k_prep<<<(unsigned)run.itemsG, kThreads, 0, st>>>(run, single);
        if ((rc = last_launch_status())) return rc;
    }
    if (run.items1 > 0) {
        if ((rc = raise_lds(k_gemm<1, kNBW1>, Shape<kNBW1>::Lds))) return rc;
        k_gemm<1, kNBW1><<<(unsigned)run.items1, kThreads, Shape<kNBW1>::Lds, st>>>(run, single);
        if ((rc = last_launch_status())) return rc;
    }
    if (run.itemsR > 0) {
        k_reduce<<<(unsigned)run.itemsR, kThreads, 0, st>>>(run, single);
        if ((rc = last_launch_status())) return rc;
    }
    if (run.items2 > 0) {
        if ((rc = raise_lds(k_gemm<2, kNBW2>, Shape<kNBW2>::Lds))) return rc;
        k_gemm<2, kNBW2><<<(unsigned)run.items2, kThreads, Shape<kNBW2>::Lds, st>>>(run, single);
        if ((rc = last_launch_status())) return rc;
    }
    return LB_OK;
}

}  // namespace

size_t gemm_workspace_bytes(const Linear &a) {
    const size_t v = valu_workspace_bytes(a);
    if (!gemm_shape_ok(a)) return v;
    GLin m;
    std::vector<int> sp;
    stage1_splits(&a, 1, sp);
    const size_t g = plan(a, &m, sp[0]);
    return g > v ? g : v;     // a misaligned x at run time takes the vector-ALU kernels
}

int gemm_forward(const Linear &a, void *ws, hipStream_t st) {
    if (!gemm_shape_ok(a)) return valu_forward(a, ws, st);
    GLin m;
    std::vector<int> sp;
    stage1_splits(&a, 1, sp);
    plan(a, &m, sp[0]);
    uint16_t *xb = bind(&m, a, (uint8_t *)ws);
    if (a.x_dtype == LB_F32) {
        const int64_t n4 = a.T * a.d_in / 4;
        k_to_bf16<<<(unsigned)cdiv(n4, kThreads), kThreads, 0, st>>>((const float *)a.x, xb, n4);
        if (int rc = last_launch_status()) return rc;
        m.x = xb;
    }
    GRun run{};
    run.T = (int)a.T;
    run.y_dtype = a.y_dtype;
    run.itemsG = m.ngp;
    run.items1 = items1_of(m);
    run.itemsR = m.nred;
    run.items2 = items2_of(m);
    run.table = nullptr;
    return launch_gemms(run, m, st);
}

// ---- groups ------------------------------------------------------------------

struct GGroupHost {
    GRun run;      // the weight preparation (k_prep) ran at prepare time
};

// bf16 inputs only (fp32 groups run linear by linear)
bool gemm_group_supported(const Linear *ls, int n) {
    for (int j = 0; j < n; ++j)
        if (!gemm_shape_ok(ls[j]) || ls[j].x_dtype != LB_BF16) return false;
    return n > 0 && ls[0].T > 0;
}

size_t gemm_group_workspace_bytes(const Linear *ls, int n) {
    std::vector<int> sp;
    stage1_splits(ls, n, sp);
    size_t need = 256 + rup256(sizeof(GLin) * n);
    int64_t iG = 0, i1 = 0, iR = 0, i2 = 0;
    for (int j = 0; j < n; ++j) {
        GLin m;
        need += plan(ls[j], &m, sp[(size_t)j]);
        iG += m.ngp;
        i1 += items1_of(m);
        iR += m.nred;
        i2 += items2_of(m);
    }
    return need + rup256((size_t)iG * 4) + rup256((size_t)i1 * 4) + rup256((size_t)iR * 4) +
           rup256((size_t)i2 * 4);
}

size_t gemm_group_state_bytes() { return sizeof(GGroupHost); }

int gemm_group_prepare(const Linear *ls, int n, void *ws, size_t ws_bytes, void *host_state,
                       hipStream_t st) {
    GGroupHost *hs = (GGroupHost *)host_state;
    if (!gemm_group_supported(ls, n)) return LB_EUNSUPPORTED;
    if (ws_bytes < gemm_group_workspace_bytes(ls, n)) return LB_EWORKSPACE;
    uint8_t *w = (uint8_t *)ws;
    std::vector<int> sp;
    stage1_splits(ls, n, sp);
    GLin *table_dev = (GLin *)(w + 256);
    uint8_t *cur = w + 256 + rup256(sizeof(GLin) * n);
    std::vector<GLin> tab((size_t)n);
    int64_t iG = 0, i1 = 0, iR = 0, i2 = 0;
    for (int j = 0; j < n; ++j) {
        GLin &m = tab[(size_t)j];
        const size_t b = plan(ls[j], &m, sp[(size_t)j]);
        bind(&m, ls[j], cur);
        cur += b;
        m.itemG = iG;
        m.item1 = i1;
        m.itemR = iR;
        m.item2 = i2;
        iG += m.ngp;
        i1 += items1_of(m);
        iR += m.nred;
        i2 += items2_of(m);
    }
    int32_t *linG = (int32_t *)cur;
    int32_t *lin1 = (int32_t *)((uint8_t *)linG + rup256((size_t)iG * 4));
    int32_t *linR = (int32_t *)((uint8_t *)lin1 + rup256((size_t)i1 * 4));
    int32_t *lin2 = (int32_t *)((uint8_t *)linR + rup256((size_t)iR * 4));
    std::vector<int32_t> hG((size_t)iG), h1((size_t)i1), hR((size_t)iR), h2((size_t)i2);
    for (int j = 0; j < n; ++j) {
        const GLin &m = tab[(size_t)j];
        for (int64_t k = 0; k < m.ngp; ++k) hG[(size_t)(m.itemG + k)] = j;
        for (int64_t k = 0; k < items1_of(m); ++k) h1[(size_t)(m.item1 + k)] = j;
        for (int64_t k = 0; k < m.nred; ++k) hR[(size_t)(m.itemR + k)] = j;
        for (int64_t k = 0; k < items2_of(m); ++k) h2[(size_t)(m.item2 + k)] = j;
    }
    if (hipMemcpy(table_dev, tab.data(), sizeof(GLin) * n, hipMemcpyHostToDevice) != hipSuccess ||
        (iG && hipMemcpy(linG, hG.data(), (size_t)iG * 4, hipMemcpyHostToDevice) != hipSuccess) ||
        (i1 && hipMemcpy(lin1, h1.data(), (size_t)i1 * 4, hipMemcpyHostToDevice) != hipSuccess) ||
        (iR && hipMemcpy(linR, hR.data(), (size_t)iR * 4, hipMemcpyHostToDevice) != hipSuccess) ||
        (i2 && hipMemcpy(lin2, h2.data(), (size_t)i2 * 4, hipMemcpyHostToDevice) != hipSuccess))
        return hip_status(hipGetLastError());
    GRun &run = hs->run;
    run = GRun{};
    run.T = (int)ls[0].T;
    run.y_dtype = ls[0].y_dtype;
    run.itemsG = iG;
    run.items1 = i1;
    run.itemsR = iR;
    run.items2 = i2;
    run.table = table_dev;
    run.linG = linG;
    run.lin1 = lin1;
    run.linR = linR;
    run.lin2 = lin2;
    // the factors are captured with the group: convert g and unzip the sign
    // words once here (runs read the converted copies)
    GRun prep = run;
    prep.items1 = prep.itemsR = prep.items2 = 0;
    GLin dummy{};
    if (int rc = launch_gemms(prep, dummy, st)) return rc;
    run.itemsG = 0;
    return hip_status(hipStreamSynchronize(st));
}

int gemm_group_run(const void *host_state, hipStream_t st, int stage_mask) {
    const GGroupHost *hs = (const GGroupHost *)host_state;
    GRun run = hs->run;
    if (!(stage_mask & 1)) run.items1 = run.itemsR = 0;
    if (!(stage_mask & 2)) run.items2 = 0;
    GLin dummy{};
    return launch_gemms(run, dummy, st);
}

}  // namespace lb
