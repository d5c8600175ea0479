/*
 * littlebit.h -- C ABI of the LittleBit factorised binary linear layer forward
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (sesamedisk page, "What the method actually computes",
 * Proposition 1; scales defined in "How low-rank binarization works"):
 *
 *     y = h (.) ( sign(U) . ( l (.) ( sign(V)^T . ( g (.) x ) ) ) )
 *
 * with sign(U) d_out x r_p and sign(V) d_in x r_p holding +-1, fp16 scale
 * vectors h (d_out), g (d_in), l (r_p), and an optional second ("residual")
 * path of the same form whose output is added (same page, Dual-SVID paragraph;
 * littlebitllm page, "Pipeline" step 04).  Activations stay floating point and
 * accumulation is fp32 (sesamedisk, the note after Proposition 1).
 *
 * Conventions for every entry point:
 *  - All array arguments are DEVICE pointers owned by the caller; the library
 *    never frees or keeps them.  Host pointers are only the small structs
 *    (lb_factors, lb_linear_desc) passed by address, read during the call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it and the call returns without waiting, except where
 *    a function says it blocks.
 *  - Return value: LB_OK (0) or a negative status.  Argument checks happen
 *    before anything is enqueued; a failed check enqueues nothing.  A launch
 *    error reported by the HIP runtime right after the launch returns LB_EHIP.
 *    Faults during execution surface at the caller's next synchronisation.
 *  - Nothing throws across this boundary and nothing aborts the process.
 *  - Activation dtypes: LB_F32 (fp32) or LB_BF16 (bf16 bit patterns).
 *    Scales are fp16 bit patterns (uint16_t).
 *  - Packed sign layout ("word planes"): a factor is packed along its
 *    contraction axis.  Word (w, o) holds the signs of elements 32w..32w+31 of
 *    the packed axis at index o of the other axis, element 32w+b in bit b;
 *    bit 1 means -1 (the value is < 0), bit 0 means +1 (also for +-0 and NaN).
 *    Plane w occupies ld words (ld >= length of the other axis, ld % 4 == 0);
 *    bits past the end of the packed axis and words past the other axis are 0.
 *    The pages store one bit per factor entry (sesamedisk, "How low-rank
 *    binarization works"); the bit order and plane layout are this library's.
 */
#ifndef LITTLEBIT_H
#define LITTLEBIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define LB_OK            0
#define LB_EINVAL       -1   /* bad size, null pointer, overlap, inconsistent rank */
#define LB_EUNSUPPORTED -2   /* valid request this build does not implement */
#define LB_EALIGN       -3   /* pointer or ld misaligned */
#define LB_EWORKSPACE   -4   /* workspace missing or too small */
#define LB_EHIP         -5   /* the HIP runtime reported an error */

/* activation dtypes */
#define LB_F32  0
#define LB_BF16 1

/* flags: path selection (low 4 bits) */
#define LB_PATH_AUTO        0u  /* decode kernels for T <= 32, MFMA GEMMs above */
#define LB_PATH_DECODE      1u  /* force the matrix-core token-streaming decode kernels */
#define LB_PATH_PREFILL     2u  /* force the MFMA GEMM (prefill) kernels */
#define LB_PATH_DECODE_VALU 3u  /* force the plain vector-ALU decode kernels */
#define LB_PATH_MASK        15u

/* Library version, (major << 16) | minor. */
int lb_version(void);

/* Human-readable text of a status code (static storage). */
const char *lb_status_string(int status);

/* Text of the last HIP runtime error this thread saw inside the library (the
 * cause behind an LB_EHIP status); static storage. */
const char *lb_last_hip_error(void);

/* Rank from the bit budget (littlebitllm page, "Pipeline" step 01 and "How
 * small": the rank is sized to the target bits per weight, counting factor bits
 * only; sesamedisk, "How low-rank binarization works": the rank sets the bit
 * budget, and the residual path fits inside the same budget).
 * b = b_num / b_den bits per weight.  r = floor(b*d_in*d_out/(d_in+d_out))
 * rounded down to a multiple of 32, in exact integer arithmetic; with the
 * residual each path gets r/2.  Writes *r_total and *r_path (host pointers).
 * LB_EINVAL if any size or b is not positive or r rounds to 0. */
int lb_rank_for_budget(int64_t d_in, int64_t d_out, int64_t b_num, int64_t b_den,
                       int residual, int64_t *r_total, int64_t *r_path);

/* Smallest valid plane stride for an other-axis length n (n rounded up to 4). */
int64_t lb_packed_ld(int64_t n_other);

/* The plane stride the decode kernels stream fastest: n rounded up to 32
 * words, so every plane starts on a 128-byte line and a 64-row piece of a
 * plane is two whole lines.  The padding words are never read by the forward
 * kernels; they cost memory only (at most 31 words per plane). */
int64_t lb_packed_ld_aligned(int64_t n_other);

/* Number of uint32 words a packed factor occupies: ceil(n_pack/32) * ld, where
 * n_pack is rows (axis 0) or cols (axis 1).  0 for bad arguments. */
int64_t lb_packed_words(int64_t rows, int64_t cols, int axis, int64_t ld);

/* Sign packing (one bit per factor entry; sesamedisk, "How low-rank
 * binarization works").  src: row-major fp32 [rows][cols], device.
 *   axis 0: pack down the rows    -> dst [ceil(rows/32)][ld], ld >= cols
 *           (use for V [d_in][r_p]: planes along d_in, ld >= r_p)
 *   axis 1: pack along the columns -> dst [ceil(cols/32)][ld], ld >= rows
 *           (use for U [d_out][r_p]: planes along r_p, ld >= d_out)
 * dst (device, 16-byte aligned) must hold lb_packed_words(rows, cols, axis, ld)
 * words; every word of it is written.  Bit-exact: bit = (src < 0).
 * LB_EINVAL for non-positive sizes, bad axis or null pointers; LB_EALIGN if
 * ld % 4 != 0 or dst is misaligned. */
int lb_pack_signs(const float *src, int64_t rows, int64_t cols, int axis,
                  uint32_t *dst, int64_t ld, void *stream);

/* Packed factors and scales of one linear, all device pointers.  With the
 * residual on, every buffer holds path 0 then path 1 (path-major).
 *   v_bits [P][ceil(d_in/32)][ld_v]  sign(V_p) packed along d_in (axis 0 of V)
 *   u_bits [P][ceil(r_p/32)][ld_u]   sign(U_p) packed along r_p  (axis 1 of U)
 *   g [P][d_in], l [P][r_p], h [P][d_out]   fp16 bit patterns
 * ld_v >= r_p and ld_u >= d_out, both multiples of 4; bit buffers 16-byte
 * aligned. */
typedef struct lb_factors {
    const uint32_t *v_bits;
    const uint32_t *u_bits;
    const uint16_t *g;
    const uint16_t *l;
    const uint16_t *h;
    int64_t ld_v;
    int64_t ld_u;
} lb_factors;

/* Workspace bytes lb_linear_forward needs for these sizes and flags
 * (latent partial sums, the rank-r intermediate).  0 on bad arguments. */
size_t lb_linear_workspace_bytes(int64_t d_in, int64_t d_out, int64_t r, int64_t T,
                                 int residual, unsigned flags);

/* One linear (Proposition 1, plus the residual path when residual != 0):
 * x [T][d_in] (x_dtype) -> y [T][d_out] (y_dtype), row-major, token-major
 * (rows of X are tokens, as in Proposition 1).  r is the TOTAL rank; with the
 * residual r must be even and each path has rank r/2.  T == 0 is a no-op.
 * ws: device workspace of at least lb_linear_workspace_bytes(...) bytes,
 * 256-byte aligned, contents need not be initialised and are clobbered.
 * x and y must not overlap each other or ws (LB_EINVAL).
 * Path choice (flags): AUTO uses the decode kernels for T <= 32 and the MFMA
 * GEMM kernels above; PREFILL with y_dtype LB_F32 is LB_EUNSUPPORTED (the
 * GEMM path rounds its operands, including g and h, to bf16, outside the fp32
 * tolerance).  Shapes the GEMM kernels do not take (d_in % 8 != 0, x not
 * 16-byte or g not 4-byte aligned) run on the vector-ALU decode kernels.
 * Calls that overlap on the same workspace race. */
int lb_linear_forward(const void *x, int x_dtype, void *y, int y_dtype,
                      const lb_factors *w, int64_t d_in, int64_t d_out, int64_t r,
                      int64_t T, int residual, void *ws, size_t ws_bytes,
                      unsigned flags, void *stream);

/* Workspace bytes lb_mlp_forward needs.  0 on bad arguments. */
size_t lb_mlp_workspace_bytes(int64_t d_model, int64_t d_ff, int64_t r_gu, int64_t r_down,
                              int64_t T, int residual, unsigned flags);

/* SwiGLU block of three LittleBit linears:
 *     y = down( silu(gate(x)) (.) up(x) ),  silu(z) = z / (1 + exp(-z)),
 * gate, up: d_model -> d_ff with total rank r_gu; down: d_ff -> d_model with
 * total rank r_down.  The pages keep the model architecture unchanged
 * (littlebitllm hero; deniz.in, "Factorize first, then binarize"), so the
 * block is the usual SwiGLU MLP with its three linears replaced.  The
 * intermediate is fp32 on the decode path and bf16 on the GEMM path.
 * Other arguments as lb_linear_forward. */
int lb_mlp_forward(const void *x, int x_dtype, void *y, int y_dtype,
                   const lb_factors *gate, const lb_factors *up, const lb_factors *down,
                   int64_t d_model, int64_t d_ff, int64_t r_gu, int64_t r_down,
                   int64_t T, int residual, void *ws, size_t ws_bytes,
                   unsigned flags, void *stream);

/* ---- many independent linears in few launches (layer stacks, q/k/v) ---- */

/* One linear of a group.  All pointers device pointers. */
typedef struct lb_linear_desc {
    const void *x;      /* [T][d_in] */
    void *y;            /* [T][d_out] */
    lb_factors w;
    int64_t d_in, d_out, r;
    int32_t residual;
    int32_t reserved;
} lb_linear_desc;

/* Workspace bytes for a group of n linears at T tokens. 0 on bad arguments. */
size_t lb_grouped_workspace_bytes(const lb_linear_desc *descs, int n, int64_t T, unsigned flags);

/* Build the device work table of a group into ws.  BLOCKS until the table is
 * on the device (a setup call, not for the timed loop).  descs is a host array
 * of n descriptors; it is copied and may be freed afterwards.  All linears use
 * x_dtype / y_dtype and T tokens.  The pointers in descs are captured: later
 * runs read and write the same buffers.  The kernels a group runs:
 *  - 1 <= T <= 32: the matrix-core decode kernels (stage 1 = activation
 *    operands, first contractions and latents; stage 2 = second contractions);
 *  - T > 32, bf16 output, bf16 input and shapes the GEMM kernels take
 *    (d_in % 8 == 0, x 16-byte and g 4-byte aligned): the GEMM kernels
 *    (stage 1 = first contractions and the d_in-piece reduction; stage 2 =
 *    second contractions).  For these, prepare also derives a bf16 copy of g
 *    and a re-ordered copy of the sign words into ws, so a caller that changes
 *    the CONTENTS of the factor buffers must prepare the group again;
 *  - otherwise the linears run one after the other through lb_linear_forward. */
int lb_grouped_prepare(const lb_linear_desc *descs, int n, int64_t T, int x_dtype, int y_dtype,
                       void *ws, size_t ws_bytes, unsigned flags, void *stream);

/* Run a prepared group: every linear's y = layer(x), in a few launches for the
 * whole group (all first contractions, then all second contractions).  A
 * decode group at T <= 2 (bf16 output) or T = 1 (fp32) whose operands fit
 * the LDS runs as ONE launch: each
 * linear's stage 2 starts as soon as its own stage 1 and latents are done.
 * That launch numbers its runs in ws (counters that keep counting), so runs
 * of one group must be issued one after the other, from one thread at a
 * time, each on a stream ordered after the previous run; runs on the same
 * workspace that overlap race, and the workspace must not be written between
 * runs. */
int lb_grouped_run(void *ws, void *stream);

/* Forget a prepared group (its host-side record; ws itself stays the
 * caller's).  Not while a run of the group may be enqueued from another
 * thread; work already enqueued completes normally.  Preparing a group again
 * on the same ws replaces the previous record.  LB_EINVAL for a ws with no
 * group. */
int lb_grouped_release(void *ws);

/* One half of lb_grouped_run: stage 1 (all first contractions, sign(V)^T
 * applied to g (.) x, and the rank-r latents) or stage 2 (all second
 * contractions and the outputs).  Running stage 1 then stage 2 on one stream
 * equals lb_grouped_run; stage 2 reads what the preceding stage 1 wrote.
 * For timing and scheduling the two halves separately.  LB_EINVAL for a
 * stage other than 1 or 2; LB_EUNSUPPORTED for a group that runs linear by
 * linear. */
int lb_grouped_run_stage(void *ws, int stage, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LITTLEBIT_H */
