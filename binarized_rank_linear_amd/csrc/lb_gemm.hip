// lb_gemm.hip -- prefill path (many tokens) of the LittleBit forward on bf16 matrix cores.
//
// Proposition 1 (sesamedisk page, "What the method actually computes") over a
// block of T tokens is two skinny GEMMs with diagonal scalings between them:
//   stage 1:  u = X . (diag(g_p) sign(V_p))        M = T, N = latents of all paths, K = d_in
//             t = l (.) u, rounded to bf16         (the rank-r intermediate, workspace)
//   stage 2:  y = t . (sign(U_p)^T diag(h_p))      M = T, N = d_out, K = latents of all paths
// Both run as v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The same page
// (its compute paragraph) describes the layer as two binary products joined by
// elementwise fp16 scalings; here the scales enter rounded to bf16.
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
// Tiles: 256 tokens (stage 1) or 128 tokens (stage 2) x 128 columns, K-tiles
// of 64 elements double-buffered in LDS (activations with a 16-byte XOR
// swizzle, unzipped sign words, scales), 4 waves of 128 (64) x 64.  Stage 1 splits d_in into pieces of at most 8192 when
// it is longer; a reduce pass then adds the pieces in order.  A launch covers
// every linear of a group (a table maps work items to linears), and work items
// are renumbered so that each of the 8 XCDs (own L2) gets a contiguous range:
// neighbouring tiles share their activation rows.
#include <algorithm>
#include <cstring>
#include <functional>
#include <map>
#include <type_traits>
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

// Tokens per tile, by the launch's token count T:
//   T > 128: 256 in stage 1 (long K: the sign operand a wave builds serves 128
//            tokens), 128 in stage 2 (short K, the latents: smaller tiles let
//            three workgroups share a CU, whose tiles' epilogues and prologues
//            overlap each other's matrix work);
//   64 < T <= 128: 128 in both; 32 < T <= 64: 64 in both; T <= 32: 32 in
//            both (a tile is mostly padding otherwise: the matrix work
//            follows the tile, not T); these small tiles are 256 columns
//            wide, the others 128.
constexpr int kBM1 = 256, kBM2 = 128;
struct TileRows {
    int bm1, bm2, bn1, bn2;    // tokens per tile of each stage; output columns per tile
};
TileRows tile_rows(int64_t T) {
    if (T <= 32) return {32, 32, 256, 256};
    if (T <= 64) return {64, 64, 256, 256};
    if (T <= 128) return {128, 128, 128, 128};
    return {kBM1, kBM2, 128, 128};
}
// Columns per tile of a stage's kernel with BM token rows (as tile_rows plans).
constexpr int tile_cols(int stage, int bm) { return bm <= 64 ? 256 : 128; }
constexpr int kBK = 64;                      // contraction elements per K-tile (two packed words)
constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kRowBytes = kBK * 2;           // one activation row of a K-tile (bf16)
constexpr int kGWave = 2 * kBK * 2;          // a wave's bf16 g: [2 paths][kBK]

// Tile shapes by n-blocks (32 columns) per wave NBW, tokens per tile BM and
// wave rows WR (the 4 waves are WR x 4/WR):
//   NBW = 2, WR = 2: BM x 128 tiles, BM/2 x 64 per wave, 2-slot ring (70 KB
//            at BM = 256: two workgroups per CU; 38 KB at BM = 128: three)
//   NBW = 1, WR = 1: 32 x 128 tiles, 32 x 32 per wave: no two waves build the
//            same sign operand (the form for at most 32 tokens)
//   NBW = 4, WR = 2: 256 x 256 tiles, 128 x 128 per wave (accumulators in
//            AGPRs), 4-slot ring (148 KB): one workgroup per CU
template <int NBW, int BM, int WR = 2> struct Shape {
    static constexpr int BN = (4 / WR) * NBW * 32;
    static constexpr int ABytes = BM * kRowBytes;      // activation rows of a K-tile
    static constexpr int XS = (NBW < 2 ? 2 : NBW) * 32;   // sign-word slots per word and wave
    static constexpr int XWave = 2 * XS * 4;           // a wave's sign words: [2 words][XS]
    static constexpr int Slot = ABytes + kWaves * (XWave + kGWave);
    static constexpr int Stages = NBW == 4 ? 4 : 2;
    static constexpr int ER = BM >= 128 ? 64 : 32;     // epilogue rows per wave and round
    static constexpr int Staging = kWaves * ER * (NBW * 32 * 4 + 16);   // room for fp32 outputs
    static constexpr int Lds = Stages * Slot > Staging ? Stages * Slot : Staging;
    static constexpr int MinWG = NBW == 4 ? 1 : (BM == 256 ? 2 : (BM == 128 || NBW == 2 ? 3 : 4));   // workgroups per CU
};
constexpr int kNBW1 = 2;                     // stage 1 on 256-token tiles (2 x 2 waves)
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
    int32_t mt, nt1, nt2; // token tiles of stage 1; column tiles of stage 1 (ldt) and stage 2 (d_out)
    int32_t mt2;          // token tiles of stage 2
    int32_t nred;         // reduce items (nsplit > 1), 0 otherwise
    int32_t ngp;          // prep items
    int64_t itemG, item1, itemR, item2;
};

struct GRun {
    int T, y_dtype, pad0_, pad1_;
    int64_t itemsG, items1, itemsR, items2;
    const GLin *table;                       // null: the single linear passed by value
    const int32_t *linG, *lin1, *linR, *lin2;   // item -> linear, per launch
    // groups: the workspace stamp written at set-up, the tag it must equal and
    // the device's fault word (stamp null for a single linear)
    const uint64_t *stamp;
    uint64_t tag;
    uint32_t *faults;
    // groups: workgroup -> item for stage 1 / stage 2, longest items first in
    // blocks spread over the XCDs (null: xcd_order)
    const int32_t *ord1, *ord2;
};

// Whether a group's workspace no longer carries the stamp the group was set up
// with: its tables are then not to be trusted, so the workgroup reports
// LB_FAULT_STALE_WORKSPACE and does nothing.  Uniform.
__device__ __forceinline__ bool stale_ws(const GRun &run) {
    if (!run.stamp || *run.stamp == run.tag) return false;
    if (threadIdx.x == 0 && run.faults)
        __hip_atomic_fetch_or(run.faults, (uint32_t)LB_FAULT_STALE_WORKSPACE, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

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
template <int STAGE, int NBW, int BM, int WR>
__global__ __launch_bounds__(kThreads, (Shape<NBW, BM, WR>::MinWG)) void k_gemm(GRun run, GLin single) {
    using SH = Shape<NBW, BM, WR>;
    constexpr int BN = SH::BN, XWave = SH::XWave, XS = SH::XS, Slot = SH::Slot, Stages = SH::Stages;
    constexpr int XC = NBW < 2 ? 1 : NBW / 2;     // sign-word DMAs per word (64 lanes each)
    constexpr int kABytes = SH::ABytes;
    constexpr int MB = BM / (32 * WR);            // 32-token blocks per wave
    constexpr int ER = SH::ER;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    if (stale_ws(run)) return;
    const int64_t items = STAGE == 1 ? run.items1 : run.items2;
    const int32_t *ord = STAGE == 1 ? run.ord1 : run.ord2;
    const int64_t v = ord ? (int64_t)__builtin_amdgcn_readfirstlane(ord[blockIdx.x]) : xcd_order(blockIdx.x, items);
    const GLin L = pick(run, single, STAGE == 1 ? run.lin1 : run.lin2, v);
    // item = (piece of d_in [stage 1], token tile, column tile); a launch has
    // fewer than 2^31 items, so the decode runs in 32 bits
    const uint32_t local = (uint32_t)(v - (STAGE == 1 ? L.item1 : L.item2));
    const uint32_t nt = (uint32_t)(STAGE == 1 ? L.nt1 : L.nt2);
    const uint32_t mt = (uint32_t)(STAGE == 1 ? L.mt : L.mt2);
    const uint32_t lq = local / nt;
    const int ni = (int)(local - lq * nt);
    const uint32_t lq2 = lq / mt;
    const int mi = (int)(lq - lq2 * mt);
    const int split = STAGE == 1 ? (int)lq2 : 0;
    const int T = run.T;
    const int64_t m0 = (int64_t)mi * BM;
    const int n0 = ni * BN;
    const int kt0 = STAGE == 1 ? split * L.ktps : 0;
    const int kt1 = STAGE == 1 ? (int)imin(L.nkt1, kt0 + L.ktps) : L.nkt2;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, l32 = lane & 31;
    const int wm = WR == 2 ? (wave & 1) : 0, wn = WR == 2 ? (wave >> 1) : wave;
    const int nw0 = n0 + wn * NBW * 32;                       // this wave's first column

    // ---- loads of one K-tile (per wave: BM/32 activation DMAs, 2 XC sign-word DMAs, 1 g DMA) ----
    // activations: wave w fills rows (BM/4) w .. (BM/4) w + BM/4 - 1, 8 rows (1 KB)
    // per DMA; lane i lands in row r = r0 + i/8 at position i%8, which holds
    // chunk (i%8) ^ swz(r)
    const int64_t K = STAGE == 1 ? L.d_in : L.ldt;
    const int rows = (int)imin(BM, (int64_t)T - m0);
    const uint8_t *abase = STAGE == 1 ? (const uint8_t *)L.x : (const uint8_t *)L.t;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(abase + m0 * K * 2, (int64_t)rows * K * 2);
    // (rows r0 .. r0+7 with r0 = 64w + 8i: swz(r) = (i/8 % 8) ^ (i & 1))
    const int arow0 = wave * (BM / 4) + (lane >> 3);         // + 8i
    // (row >> 3) & 1 of DMA i's rows is (wave * BM / 32 + i) & 1: i's parity,
    // and the wave's own for 8-row waves (BM = 32)
    const int ach0 = (lane & 7) ^ ((lane >> 3) & 7) ^ ((wave * (BM / 32)) & 1);   // chunk for even i
    const int ach1 = ach0 ^ 1;                                // chunk for odd i
    const uint32_t aoffe = (uint32_t)(arow0 * K * 2) + (uint32_t)(ach0 * 16);
    const uint32_t aoffo = (uint32_t)(arow0 * K * 2) + (uint32_t)(ach1 * 16);
    const uint32_t astep = (uint32_t)(8 * K * 2);            // 8 rows
    // sign words: this wave's columns nw0 + 64c + lane, c < XC, both words of
    // the K-tile (with one n-block per wave, lanes 32..63 load nothing)
    __amdgpu_buffer_rsrc_t rx;
    uint32_t xoff[XC], xstep;
    const bool xlane = NBW >= 2 || lane < 32;
    int xwords;
    if (STAGE == 1) {
        rx = make_rsrc(L.vz, (int64_t)L.P * L.kw_v * L.zld_v * 4);
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const int xn = nw0 + 64 * c + lane;
            const int qn = xn >> 5;
            const int p = qn / L.kw;
            const int k = (qn - p * L.kw) * 32 + (xn & 31);
            xoff[c] = (xlane && p < L.P && k < L.r_p) ? (uint32_t)(((int64_t)p * L.kw_v * L.zld_v + k) * 4) : kOOB;
        }
        xstep = (uint32_t)(L.zld_v * 4);
        xwords = L.kw_v;
    } else {
        rx = make_rsrc(L.uz, (int64_t)L.P * L.kw * L.zld_u * 4);
#pragma unroll
        for (int c = 0; c < XC; ++c) {
            const int xn = nw0 + 64 * c + lane;
            xoff[c] = (xlane && xn < L.d_out) ? (uint32_t)(xn * 4) : kOOB;
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
        for (int i = 0; i < BM / 32; ++i) {
            const bool kin = (i & 1) ? kino : kine;
            const uint32_t off = ((i & 1) ? aoffo : aoffe) + i * astep + (uint32_t)(kt * kBK * 2);
            dma<16>(ra, S + (wave * (BM / 4) + 8 * i) * kRowBytes, kin ? off : kOOB);
        }
        uint8_t *X = S + kABytes + wave * (XWave + kGWave);
#pragma unroll
        for (int wd = 0; wd < 2; ++wd) {
            const int q = kt * 2 + wd;
#pragma unroll
            for (int c = 0; c < XC; ++c)
                dma<4>(rx, X + (wd * XS + 64 * c) * 4,
                       (xoff[c] != kOOB && q < xwords) ? xoff[c] + (uint32_t)q * xstep : kOOB);
        }
        if (STAGE == 1) {
            const int64_t e = (int64_t)kt * kBK + gel;
            dma<4>(rg, X + XWave, e < L.d_in ? (uint32_t)((gpath * L.d_in + e) * 2) : kOOB);
        }
    };
    constexpr int kIssued = BM / 32 + 2 * XC + (STAGE == 1 ? 1 : 0);   // DMAs per K-tile per wave

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
    // quad), loaded before the K loop.  A run of 4 columns whose first one is a
    // padding latent is all padding (bit of lok clear: zeros out); a run that
    // crosses r_p (r_p not a multiple of 4) takes l = 0 past it, so its padding
    // columns come out zero too.
    u32x2 lsc[NBW][4];
    uint32_t lok = 0;                                  // bit 4b+q4: run starts at a real latent
    if (STAGE == 1 && L.nsplit == 1) {
        int lk[NBW][4];                                // the run's first latent of its path, or -1
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
                lk[b][q4] = ok ? k : -1;
                lp[b][q4] = L.l + (ok ? (int64_t)p * L.r_p + k : 0);
            }
        if (((uintptr_t)L.l & 7) == 0 && (L.r_p & 3) == 0) {     // uniform: whole runs, 8-byte aligned
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
                    const int k = lk[b][q4];
                    uint32_t e[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) e[i] = (k >= 0 && k + i < L.r_p) ? (uint32_t)q[i] : 0u;
                    lsc[b][q4] = u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
                }
        }
    }

    f32x16 acc[NBW][MB];
#pragma unroll
    for (int b = 0; b < NBW; ++b)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[b][mb][i] = 0.0f;

    // One K-tile = 4 steps of 16 elements (step st: word st/2, half st%2).
    auto compute = [&](int slot, int kt) {
        const uint8_t *A = smem + slot * Slot;
        const uint8_t *Xw = A + kABytes + wave * (XWave + kGWave);
        const uint8_t *G = Xw + XWave;
        // operands of step st+1 are read from LDS before step st's matrix
        // instructions (two register sets), so their latency hides behind them
        u32x4 act[2][MB], scr[2][NBW];
        uint32_t xsr[2][NBW];
        auto fetch = [&](int st, int bi) {
            const int w2 = st >> 1, s = st & 1;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = wm * (BM / WR) + mb * 32 + l32;
                const int chunk = 2 * st + hh;
                act[bi][mb] = *(const u32x4 *)(A + row * kRowBytes + ((chunk ^ swz(row)) << 4));
            }
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                xsr[bi][b] = ((const uint32_t *)Xw)[w2 * XS + b * 32 + l32];
                if (STAGE == 1) scr[bi][b] = *(const u32x4 *)(G + gofs[b] + (32 * w2 + 16 * s) * 2);
            }
        };
        fetch(0, 0);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
            const int w2 = st >> 1, s = st & 1, bi = st & 1;
            if (st < 3) fetch(st + 1, bi ^ 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                const uint32_t xs = xsr[bi][b] << xshift;
                u32x4 sc;
                if (STAGE == 1) {
                    sc = scr[bi][b];
                } else {
                    const uint32_t hp = (kt * 2 + w2) >= L.kw ? hpair[b][1] : hpair[b][0];
                    sc = u32x4{hp, hp, hp, hp};
                }
                u32x4 sg;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    sg[jj] = sc[jj] ^ ((xs << (11 - 8 * s - jj)) & 0x80008000u);
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) acc[b][mb] = mfma(sg, act[bi][mb], acc[b][mb]);
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
    // wave stages ER rows of its tile at a time in its own part of the (now
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
    uint8_t *stage = smem + wave * ER * (WC * 4 + 16);         // room for the fp32 case
    static_assert(kWaves * ER * (WC * 4 + 16) <= SH::Lds, "epilogue staging fits the ring");
    // whole 16-byte chunks only when every row starts 16-byte aligned
    const bool chunky = ((ld_out * osz) % 16) == 0 && ((uintptr_t)obase % 16) == 0;
    // buffer offsets stay below 2^31 (the descriptor's range), so 32 bits hold them
    const uint32_t ld32 = (uint32_t)ld_out, nlim32 = (uint32_t)n_lim;
    wait_and_meet<0>();                                        // every wave is done with the ring
    auto epilogue = [&](auto osz_c) {
        constexpr int OSZ = decltype(osz_c)::value;
        constexpr int rbytes = WC * OSZ + 16;                  // staged row (padded)
#pragma unroll
        for (int half = 0; half < MB * 32 / ER; ++half) {
            // accumulators -> LDS (l applied for stage-1 latents)
#pragma unroll
            for (int mh = 0; mh < ER / 32; ++mh) {
                const int mb = (ER / 32) * half + mh;
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
                        if constexpr (OSZ == 2)
                            *(u32x2 *)(rowp + c * 2) = u32x2{bf16_pair(o0, o1), bf16_pair(o2, o3)};
                        else
                            *(f32x4 *)(rowp + c * 4) = f32x4{o0, o1, o2, o3};
                    }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's LDS writes land
            // LDS -> global: ER rows x WC columns in 16-byte chunks, lane order row-major
            constexpr int cpr = WC * OSZ / 16;                     // chunks per row
            constexpr int per = 16 / OSZ;                          // columns per chunk
            static_assert((ER * cpr) % 64 == 0, "whole rounds of 64 chunks");
#pragma unroll
            for (int i = 0; i < ER * cpr / 64; ++i) {
                const int ci = lane + 64 * i;
                const int r = ci / cpr, ch = ci % cpr;
                const uint32_t n = (uint32_t)(nw0 + ch * per);    // first column of the chunk
                const u32x4 val = *(const u32x4 *)(stage + r * rbytes + ch * 16);
                const uint32_t off = ((uint32_t)(wm * (BM / WR) + half * ER + r) * ld32 + n) * OSZ;
                if (chunky && n + per <= nlim32) {
                    // non-temporal: the outputs stream out instead of filling the L2
                    // that holds the activation rows other tiles still read
                    __builtin_amdgcn_raw_buffer_store_b128(val, ro, (int)off, 0, 2);
                } else {
#pragma unroll
                    for (int e = 0; e < per; ++e) {
                        if (n + e >= nlim32) break;
                        if constexpr (OSZ == 2)
                            __builtin_amdgcn_raw_buffer_store_b16(
                                (unsigned short)((val[e >> 1] >> (16 * (e & 1))) & 0xffffu), ro, (int)(off + 2 * e), 0, 0);
                        else
                            __builtin_amdgcn_raw_buffer_store_b32(val[e], ro, (int)(off + 4 * e), 0, 0);
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next half
        }
    };
    if (osz == 2)
        epilogue(std::integral_constant<int, 2>{});
    else
        epilogue(std::integral_constant<int, 4>{});
}

// Per-call operand preparation: g -> bf16 (round to nearest even) for the
// stage-1 sign operands, and every packed sign word of V and U unzipped (even
// bits to the low half, odd bits to the high half) for both stages.
constexpr int kPrep = 1024;       // words per item

__global__ __launch_bounds__(kThreads) void k_prep(GRun run, GLin single) {
    if (stale_ws(run)) return;
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
// One thread per group of 4 latents of one token; its pieces' loads go out
// together (8 at a time, unconditional buffer loads: pieces past the last
// read as zeros and are not added), so a thread waits about once per 8 pieces.
__global__ __launch_bounds__(kThreads) void k_reduce(GRun run, GLin single) {
    if (stale_ws(run)) return;
    const int64_t v = blockIdx.x;
    const GLin L = pick(run, single, run.linR, v);
    const int T = run.T;
    const int64_t groups = (int64_t)T * (L.ldt / 4);
    const int64_t gi = (v - L.itemR) * kThreads + threadIdx.x;
    if (gi >= groups) return;
    const int64_t m = gi / (L.ldt / 4);
    const int n = (int)(gi - m * (L.ldt / 4)) * 4;
    const int64_t stride = (int64_t)T * L.ldt * 4;                 // bytes between pieces
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(L.part, stride * L.nsplit);
    const uint32_t base = (uint32_t)((m * L.ldt + n) * 4);
    f32x4 s;
    for (int sp0 = 0; sp0 < L.nsplit; sp0 += 8) {
        u32x4 a[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            a[q] = __builtin_amdgcn_raw_buffer_load_b128(
                rp, sp0 + q < L.nsplit ? base + (uint32_t)((int64_t)(sp0 + q) * stride) : kOOB, 0, 0);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const f32x4 x = __builtin_bit_cast(f32x4, a[q]);
            if (sp0 + q == 0) s = x;
            else if (sp0 + q < L.nsplit) s += x;
        }
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

// fp32 activations -> bf16 (round to nearest even), 4 per thread.
__global__ __launch_bounds__(kThreads) void k_to_bf16(const float *__restrict__ x, uint16_t *__restrict__ xb,
                                                      int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n4) return;
    const f32x4 v = ((const f32x4 *)x)[i];
    ((u32x2 *)xb)[i] = u32x2{bf16_pair(v[0], v[1]), bf16_pair(v[2], v[3])};
}

// The latent API: the GEMM kernels keep t as bf16 [T][ldt] with path p in
// columns p*kw*32 .. (zero padding between the paths); the caller's t is
// [T][P*r_p] with path p in columns p*r_p ...  One thread per (token, column
// of ldt).  Out: t_dst = the kernels' latents (widened for fp32, exact).
__global__ __launch_bounds__(kThreads) void k_t_out(GLin L, int64_t T, void *t_dst, int t_dtype) {
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= T * L.ldt) return;
    const int64_t n = e / L.ldt;
    const int c = (int)(e - n * L.ldt);
    const int p = c / (L.kw * 32), k = c - p * L.kw * 32;
    if (p >= L.P || k >= L.r_p) return;
    const uint16_t b = L.t[e];
    const int64_t o = n * (int64_t)L.P * L.r_p + (int64_t)p * L.r_p + k;
    if (t_dtype == LB_F32) ((float *)t_dst)[o] = bf16_to_f32(b);
    else ((uint16_t *)t_dst)[o] = b;
}

// In: the kernels' latents from the caller's t (rounded to bf16, nearest
// even), padding columns zero.
__global__ __launch_bounds__(kThreads) void k_t_in(GLin L, int64_t T, const void *t_src, int t_dtype) {
    const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (e >= T * L.ldt) return;
    const int64_t n = e / L.ldt;
    const int c = (int)(e - n * L.ldt);
    const int p = c / (L.kw * 32), k = c - p * L.kw * 32;
    uint16_t b = 0;
    if (p < L.P && k < L.r_p) {
        const int64_t o = n * (int64_t)L.P * L.r_p + (int64_t)p * L.r_p + k;
        b = t_dtype == LB_F32 ? f32_to_bf16(((const float *)t_src)[o]) : ((const uint16_t *)t_src)[o];
    }
    L.t[e] = b;
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
// Stage-1 pieces (d_in splits) per linear for a launch over ls[0..n).  The
// launch's workgroups run on kWG1 slots (two per CU), longest pieces first;
// its time is about the makespan of that schedule (in K-tiles of 64 per
// slot) plus the reduce pass that adds the pieces.  The pieces are cut to a
// common target length, the one (among the lengths the linears' K-tiles
// split into) that gives the least such estimate.  Without it one long
// linear (a down projection, d_in 17408 or 28672, beside 5120- or
// 8192-wide ones) sets the launch's length alone.  Writes splits[j].
namespace {
struct SplitModel {
    std::vector<int64_t> nkt, tiles, red_bytes;    // per linear: K-tiles, tiles, reduce bytes per piece
};

// Longest-first makespan of pieces grouped as (length, count), on kWG1
// identical slots; the slots' end times are kept as a multiset.
int64_t lpt_span(std::vector<std::pair<int64_t, int64_t>> pieces) {
    std::sort(pieces.begin(), pieces.end(), [](const std::pair<int64_t, int64_t> &x,
                                               const std::pair<int64_t, int64_t> &y) { return x.first > y.first; });
    std::map<int64_t, int64_t> ends;
    ends[0] = kWG1;
    for (const auto &pc : pieces) {
        if (pc.first <= 0) continue;
        int64_t c = pc.second;
        while (c > 0) {                 // the earliest free slots take the next pieces
            auto it = ends.begin();
            const int64_t e = it->first, m = std::min(c, it->second);
            it->second -= m;
            if (it->second == 0) ends.erase(it);
            ends[e + pc.first] += m;
            c -= m;
        }
    }
    return ends.rbegin()->first;
}

double split_cost(const SplitModel &m, const std::vector<int> &sp) {
    std::vector<std::pair<int64_t, int64_t>> pieces;
    double red = 0;
    for (size_t j = 0; j < sp.size(); ++j) {
        const int64_t ktps = cdiv(m.nkt[j], sp[j]);
        const int64_t np = cdiv(m.nkt[j], ktps);
        const int64_t last = m.nkt[j] - (np - 1) * ktps;
        if (np > 1) pieces.push_back({ktps, (np - 1) * m.tiles[j]});
        pieces.push_back({last, m.tiles[j]});
        if (np > 1) red += (double)np * m.red_bytes[j];
    }
    // in us: a K-tile of 64 on a slot takes about 2 us at the measured rates
    // (two workgroups share a CU); the reduce reads the pieces and writes t
    // at about 5 TB/s
    return 2.0 * (double)lpt_span(pieces) + red / 5e6;
}
}  // namespace

void stage1_splits(const Linear *ls, int n, std::vector<int> &splits) {
    SplitModel m;
    std::vector<int64_t> cand;
    for (int j = 0; j < n; ++j) {
        const Linear &a = ls[j];
        const int64_t ldt = rup((int64_t)a.P * cdiv(a.r_p, 32) * 32, kBK);
        const int64_t nkt = cdiv(a.d_in, kBK);
        m.nkt.push_back(nkt);
        m.tiles.push_back(cdiv(ldt, tile_rows(a.T).bn1) * cdiv(a.T, tile_rows(a.T).bm1));
        m.red_bytes.push_back(a.T * ldt * 4);
        for (int64_t sp = 1; sp <= 64; ++sp) {
            const int64_t l = cdiv(nkt, sp);
            if (l < 8 && sp > 1) break;                 // pieces of at least 8 K-tiles
            cand.push_back(l);
        }
    }
    std::sort(cand.begin(), cand.end());
    cand.erase(std::unique(cand.begin(), cand.end()), cand.end());
    splits.assign((size_t)n, 1);
    double best = split_cost(m, splits);
    std::vector<int> sp((size_t)n);
    for (int64_t target : cand) {
        for (int j = 0; j < n; ++j) sp[(size_t)j] = (int)std::max<int64_t>(1, cdiv(m.nkt[(size_t)j], target));
        const double c = split_cost(m, sp);
        if (c < best - 1e-9) {
            best = c;
            splits = sp;
        }
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
    const TileRows tr = tile_rows(a.T);
    m->mt = (int32_t)cdiv(a.T, tr.bm1);
    m->mt2 = (int32_t)cdiv(a.T, tr.bm2);
    m->nt1 = (int32_t)cdiv(m->ldt, tr.bn1);
    m->nt2 = (int32_t)cdiv(a.d_out, tr.bn2);
    m->nred = m->nsplit > 1 ? (int32_t)cdiv(a.T * (m->ldt / 4), kThreads) : 0;
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
int64_t items2_of(const GLin &m) { return (int64_t)m.nt2 * m.mt2; }

// > 64 KB of dynamic LDS needs an explicit opt-in, once per kernel (the flag
// is per instantiation, so per kernel).
template <auto KERN>
int raise_lds(int bytes) {
    static bool done = false;
    if (!done) {
        if (hipFuncSetAttribute((const void *)KERN, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) !=
            hipSuccess)
            return hip_status(hipGetLastError());
        done = true;
    }
    return LB_OK;
}

template <int STAGE, int BM>
int launch_stage(const GRun &run, const GLin &single, int64_t items, hipStream_t st) {
    // waves 1 x 4 (no two waves build the same sign operand) except stage 1
    // on 256-token tiles, whose long K favours 2 x 2 waves of 64 columns (half
    // the activation reads per matrix instruction); tiles of up to 64 tokens
    // are 256 columns wide (64 per wave: more sign words per K-tile behind
    // each wait)
    constexpr int NBW = STAGE == 1 && BM == 256 ? kNBW1 : (BM <= 64 ? 2 : 1);
    constexpr int WR = STAGE == 1 && BM == 256 ? 2 : 1;
    using SH = Shape<NBW, BM, WR>;
    static_assert(SH::BN == tile_cols(STAGE, BM), "column tiles as planned");
    if (int rc = raise_lds<k_gemm<STAGE, NBW, BM, WR>>(SH::Lds)) return rc;
    k_gemm<STAGE, NBW, BM, WR><<<(unsigned)items, kThreads, SH::Lds, st>>>(run, single);
    return last_launch_status();
}

int launch_gemms(const GRun &run, const GLin &single, hipStream_t st) {
    int rc;
    const TileRows tr = tile_rows(run.T);
    if (run.itemsG > 0) {
        k_prep<<<(unsigned)run.itemsG, kThreads, 0, st>>>(run, single);
        if ((rc = last_launch_status())) return rc;
    }
    if (run.items1 > 0) {
        rc = tr.bm1 == 32 ? launch_stage<1, 32>(run, single, run.items1, st)
           : tr.bm1 == 64 ? launch_stage<1, 64>(run, single, run.items1, st)
           : tr.bm1 == 128 ? launch_stage<1, 128>(run, single, run.items1, st)
           : launch_stage<1, kBM1>(run, single, run.items1, st);
        if (rc) return rc;
    }
    if (run.itemsR > 0) {
        k_reduce<<<(unsigned)run.itemsR, kThreads, 0, st>>>(run, single);
        if ((rc = last_launch_status())) return rc;
    }
    if (run.items2 > 0) {
        rc = tr.bm2 == 32 ? launch_stage<2, 32>(run, single, run.items2, st)
           : tr.bm2 == 64 ? launch_stage<2, 64>(run, single, run.items2, st)
                          : launch_stage<2, 128>(run, single, run.items2, st);
        if (rc) return rc;
    }
    return LB_OK;
}

}  // namespace

bool gemm_linear_supported(const Linear &a) { return gemm_shape_ok(a); }

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

int gemm_stage_forward(const Linear &a, void *ws, int stage, void *t, int t_dtype, hipStream_t st) {
    if (!gemm_shape_ok(a)) return valu_stage_forward(a, ws, stage, t, t_dtype, st);
    GLin m;
    std::vector<int> sp;
    stage1_splits(&a, 1, sp);
    plan(a, &m, sp[0]);
    uint16_t *xb = bind(&m, a, (uint8_t *)ws);
    if (stage == 1 && a.x_dtype == LB_F32) {
        const int64_t n4 = a.T * a.d_in / 4;
        k_to_bf16<<<(unsigned)cdiv(n4, kThreads), kThreads, 0, st>>>((const float *)a.x, xb, n4);
        if (int rc = last_launch_status()) return rc;
        m.x = xb;
    }
    GRun run{};
    run.T = (int)a.T;
    run.y_dtype = a.y_dtype;
    run.itemsG = m.ngp;
    run.table = nullptr;
    const unsigned nt = (unsigned)cdiv(a.T * m.ldt, kThreads);
    if (stage == 1) {
        run.items1 = items1_of(m);
        run.itemsR = m.nred;
        if (int rc = launch_gemms(run, m, st)) return rc;
        k_t_out<<<nt, kThreads, 0, st>>>(m, a.T, t, t_dtype);
        return last_launch_status();
    }
    k_t_in<<<nt, kThreads, 0, st>>>(m, a.T, t, t_dtype);
    if (int rc = last_launch_status()) return rc;
    run.items2 = items2_of(m);
    return launch_gemms(run, m, st);
}

// ---- groups ------------------------------------------------------------------

struct GGroupHost {
    GRun run;
};

// bf16 inputs only (fp32 groups run linear by linear)
bool gemm_group_supported(const Linear *ls, int n) {
    for (int j = 0; j < n; ++j)
        if (!gemm_shape_ok(ls[j]) || ls[j].x_dtype != LB_BF16) return false;
    return n > 0 && ls[0].T > 0;
}

// Workspace of a group: the 256-byte header (the stamp), the per-linear table
// and the item tables (the "control" part), then each linear's scratch.
struct GLayout {
    int64_t iG = 0, i1 = 0, iR = 0, i2 = 0;
    size_t table, linG, lin1, linR, lin2, ord1, ord2, ctrl_end, total;
};

// Dispatch order of a launch's items from their lengths (K-tiles): longest
// first, so the launch ends on short items; workgroups go to the 8 XCDs in
// turn, so each block of 8 * kRun items in that order is dealt out as kRun
// consecutive items per XCD (consecutive items share activation rows in the
// XCD's L2).
//
// When every token tile's items can go to one XCD (the items split evenly
// over the 8 XCDs by token tile modulo 8, e.g. T = 2048: 8 tiles of 256
// tokens), they do: XCD x runs the items of token tiles x, x + 8, ...,
// longest first, so each XCD's L2 holds its tiles' activation rows (x for
// stage 1, t for stage 2) for all their column tiles and linears, instead of
// fetching them again for every run of kRun items.
std::vector<int32_t> dispatch_order(const std::vector<int64_t> &len, const std::vector<int32_t> &tok) {
    const int64_t n = (int64_t)len.size();
    {
        std::vector<std::vector<int32_t>> per(8);
        for (int64_t i = 0; i < n; ++i) per[(size_t)(tok[(size_t)i] & 7)].push_back((int32_t)i);
        bool even = n > 0;
        for (const auto &v : per) even = even && v.size() == per[0].size();
        if (even) {
            std::vector<int32_t> D((size_t)n);
            for (int x = 0; x < 8; ++x) {
                auto &v = per[(size_t)x];
                std::stable_sort(v.begin(), v.end(), [&](int32_t a, int32_t b) { return len[(size_t)a] > len[(size_t)b]; });
                for (size_t j = 0; j < v.size(); ++j) D[j * 8 + (size_t)x] = v[j];
            }
            return D;
        }
    }
    constexpr int kRun = 4;
    std::vector<int32_t> L((size_t)n);
    for (int64_t i = 0; i < n; ++i) L[(size_t)i] = (int32_t)i;
    std::stable_sort(L.begin(), L.end(), [&](int32_t a, int32_t b) { return len[(size_t)a] > len[(size_t)b]; });
    std::vector<int32_t> D((size_t)n);
    for (int64_t c0 = 0; c0 < n; c0 += 8 * kRun) {
        const int64_t cnt = std::min<int64_t>(8 * kRun, n - c0);
        for (int64_t b = 0; b < cnt; ++b)
            D[(size_t)(c0 + b)] = cnt == 8 * kRun ? L[(size_t)(c0 + (b % 8) * kRun + b / 8)] : L[(size_t)(c0 + b)];
    }
    return D;
}

GLayout glayout(const Linear *ls, int n, std::vector<GLin> *tab, std::vector<size_t> *scratch) {
    std::vector<int> sp;
    stage1_splits(ls, n, sp);
    GLayout g;
    size_t lin_bytes = 0;
    if (tab) tab->assign((size_t)n, GLin{});
    if (scratch) scratch->assign((size_t)n, 0);
    for (int j = 0; j < n; ++j) {
        GLin m;
        const size_t b = plan(ls[j], &m, sp[(size_t)j]);
        m.itemG = g.iG;
        m.item1 = g.i1;
        m.itemR = g.iR;
        m.item2 = g.i2;
        g.iG += m.ngp;
        g.i1 += items1_of(m);
        g.iR += m.nred;
        g.i2 += items2_of(m);
        if (tab) (*tab)[(size_t)j] = m;
        if (scratch) (*scratch)[(size_t)j] = b;
        lin_bytes += b;
    }
    size_t at = 256;
    auto take = [&](size_t bytes) { const size_t o = at; at += rup256(bytes); return o; };
    g.table = take(sizeof(GLin) * n);
    g.linG = take((size_t)g.iG * 4);
    g.lin1 = take((size_t)g.i1 * 4);
    g.linR = take((size_t)g.iR * 4);
    g.lin2 = take((size_t)g.i2 * 4);
    g.ord1 = take((size_t)g.i1 * 4);
    g.ord2 = take((size_t)g.i2 * 4);
    g.ctrl_end = at;
    g.total = at + lin_bytes;
    return g;
}

size_t gemm_group_workspace_bytes(const Linear *ls, int n) { return glayout(ls, n, nullptr, nullptr).total; }

size_t gemm_group_state_bytes() { return sizeof(GGroupHost); }

int gemm_group_plan(const Linear *ls, int n, void *ws, size_t ws_bytes, uint64_t tag, void *host_state,
                    GroupImage *img) {
    GGroupHost *hs = (GGroupHost *)host_state;
    *hs = GGroupHost{};
    if (!gemm_group_supported(ls, n)) return LB_EUNSUPPORTED;
    std::vector<GLin> tab;
    std::vector<size_t> scratch;
    const GLayout G = glayout(ls, n, &tab, &scratch);
    if (ws_bytes < G.total) return LB_EWORKSPACE;
    uint8_t *w = (uint8_t *)ws;
    uint8_t *cur = w + G.ctrl_end;
    for (int j = 0; j < n; ++j) {
        bind(&tab[(size_t)j], ls[j], cur);
        cur += scratch[(size_t)j];
    }
    std::vector<int32_t> hG((size_t)G.iG), h1((size_t)G.i1), hR((size_t)G.iR), h2((size_t)G.i2);
    for (int j = 0; j < n; ++j) {
        const GLin &m = tab[(size_t)j];
        for (int64_t k = 0; k < m.ngp; ++k) hG[(size_t)(m.itemG + k)] = j;
        for (int64_t k = 0; k < items1_of(m); ++k) h1[(size_t)(m.item1 + k)] = j;
        for (int64_t k = 0; k < m.nred; ++k) hR[(size_t)(m.itemR + k)] = j;
        for (int64_t k = 0; k < items2_of(m); ++k) h2[(size_t)(m.item2 + k)] = j;
    }
    std::vector<uint8_t> &im = img->bytes;
    im.assign(G.ctrl_end, 0);
    memcpy(im.data(), &tag, sizeof(tag));
    auto put = [&](size_t off, const void *src, size_t bytes) { if (bytes) memcpy(im.data() + off, src, bytes); };
    put(G.table, tab.data(), sizeof(GLin) * n);
    put(G.linG, hG.data(), (size_t)G.iG * 4);
    put(G.lin1, h1.data(), (size_t)G.i1 * 4);
    put(G.linR, hR.data(), (size_t)G.iR * 4);
    put(G.lin2, h2.data(), (size_t)G.i2 * 4);
    // item lengths in K-tiles of 64: stage 1 the item's piece of d_in, stage 2 the latents
    // and their token tiles (item = (piece, token tile, column tile), column fastest)
    std::vector<int64_t> len1((size_t)G.i1), len2((size_t)G.i2);
    std::vector<int32_t> tok1((size_t)G.i1), tok2((size_t)G.i2);
    for (int j = 0; j < n; ++j) {
        const GLin &m = tab[(size_t)j];
        for (int64_t k = 0; k < items1_of(m); ++k) {
            const int64_t split = k / ((int64_t)m.nt1 * m.mt);
            len1[(size_t)(m.item1 + k)] = split + 1 < m.nsplit ? m.ktps : m.nkt1 - (int64_t)(m.nsplit - 1) * m.ktps;
            tok1[(size_t)(m.item1 + k)] = (int32_t)((k / m.nt1) % m.mt);
        }
        for (int64_t k = 0; k < items2_of(m); ++k) {
            len2[(size_t)(m.item2 + k)] = m.nkt2;
            tok2[(size_t)(m.item2 + k)] = (int32_t)((k / m.nt2) % m.mt2);
        }
    }
    const std::vector<int32_t> o1 = dispatch_order(len1, tok1), o2 = dispatch_order(len2, tok2);
    put(G.ord1, o1.data(), (size_t)G.i1 * 4);
    put(G.ord2, o2.data(), (size_t)G.i2 * 4);
    // the scratch needs no initial contents (every byte a run reads it writes first)
    img->zero_off = G.ctrl_end;
    img->zero_bytes = 0;
    GRun &run = hs->run;
    run = GRun{};
    run.T = (int)ls[0].T;
    run.y_dtype = ls[0].y_dtype;
    run.itemsG = G.iG;
    run.items1 = G.i1;
    run.itemsR = G.iR;
    run.items2 = G.i2;
    run.table = (const GLin *)(w + G.table);
    run.linG = (const int32_t *)(w + G.linG);
    run.lin1 = (const int32_t *)(w + G.lin1);
    run.linR = (const int32_t *)(w + G.linR);
    run.lin2 = (const int32_t *)(w + G.lin2);
    run.ord1 = (const int32_t *)(w + G.ord1);
    run.ord2 = (const int32_t *)(w + G.ord2);
    run.stamp = (const uint64_t *)w;
    run.tag = tag;
    run.faults = fault_word_ptr();
    return LB_OK;
}

int gemm_group_run(const void *host_state, hipStream_t st, int stage_mask) {
    const GGroupHost *hs = (const GGroupHost *)host_state;
    GRun run = hs->run;
    if (!(stage_mask & 4)) run.itemsG = 0;
    if (!(stage_mask & 1)) run.items1 = run.itemsR = 0;
    if (!(stage_mask & 2)) run.items2 = 0;
    GLin dummy{};
    return launch_gemms(run, dummy, st);
}

}  // namespace lb
