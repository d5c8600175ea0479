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
 *    Deliberately plane-major, i.e. the TRANSPOSE of the row-major word layout
 *    [other axis][ld_words] a reader might expect (V as [r_p][d_in/32]):
 *    here V is [d_in/32][ld_v] and U is [r_p/32][ld_u].  A 16-byte load then
 *    gives a lane four consecutive latents (stage 1) or output rows (stage 2)
 *    of one plane, so a wave's loads are contiguous.  Words in the other
 *    layout give wrong outputs without an error: pack with lb_pack_signs.
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
#define LB_EDEVICE      -6   /* a kernel reported a fault (lb_device_faults) */

/* activation dtypes */
#define LB_F32  0
#define LB_BF16 1

/* flags: path selection (low 4 bits) */
#define LB_PATH_AUTO        0u  /* decode kernels for T <= 8 (fp32 out: T <= 32), MFMA GEMMs above */
#define LB_PATH_DECODE      1u  /* force the matrix-core token-streaming decode kernels */
#define LB_PATH_PREFILL     2u  /* force the MFMA GEMM (prefill) kernels */
#define LB_PATH_DECODE_VALU 3u  /* force the plain vector-ALU decode kernels */
#define LB_PATH_MASK        15u

/* flags: for groups only (lb_grouped_prepare, lb_linear_forward_grouped).
 * LB_GROUP_FAULT_TEST exists to test the fault report: in a group that runs
 * as one launch per pass (see lb_grouped_run), every stage-2 workgroup waits
 * for one latent group more than the linear has and gives up after a few
 * polls, so every run reports LB_FAULT_HANDOFF_TIMEOUT and its outputs are
 * wrong.  Every kernel still ends normally and the group's counters return to
 * zero.  Never set it outside such a test. */
#define LB_GROUP_FAULT_TEST (1u << 8)

/* Fault bits a kernel can report (lb_device_faults). */
#define LB_FAULT_HANDOFF_TIMEOUT 1u  /* a stage-2 workgroup of a one-launch pass gave up waiting for
                                        its linear's latents: that run's outputs are wrong */
#define LB_FAULT_STALE_WORKSPACE 2u  /* a prepared group's workspace no longer carried the stamp the
                                        group was prepared with (the memory was reused or written
                                        since): the launch did nothing and its outputs are unset */

/* Library version, (major << 16) | minor. */
int lb_version(void);

/* Human-readable text of a status code (static storage). */
const char *lb_status_string(int status);

/* Text of the last HIP runtime error this thread saw inside the library (the
 * cause behind an LB_EHIP status); static storage. */
const char *lb_last_hip_error(void);

/* Faults the kernels reported on the current device since the last call.
 * BLOCKS until the work enqueued on `stream` is done, then reads and clears
 * the device's fault word (one per device, owned by the library, shared by
 * every stream and caller on that device).  Writes the LB_FAULT_* bits to
 * *faults (host pointer; may be NULL).  Returns LB_OK if none was set,
 * LB_EDEVICE if any was, LB_EHIP if the runtime failed. */
int lb_device_faults(void *stream, uint32_t *faults);

/* The kernel family lb_linear_forward would use for these sizes and flags,
 * with packed strides from lb_packed_ld_aligned and aligned pointers:
 * LB_PATH_DECODE (matrix-core decode), LB_PATH_PREFILL (bf16 GEMM) or
 * LB_PATH_DECODE_VALU (vector ALU), or a negative status for a request
 * lb_linear_forward would reject.  Host only; enqueues nothing. */
int lb_linear_path(int64_t d_in, int64_t d_out, int64_t r, int64_t T, int residual,
                   int x_dtype, int y_dtype, unsigned flags);

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
 * (latent partial sums, the rank-r intermediate): the most that any path a
 * call of these sizes may take needs, for either activation and output dtype
 * and for any pointers (AUTO, for example, sends a shape or a pointer the
 * GEMM kernels do not take to the decode or vector-ALU kernels).  Enough for
 * every lb_linear_forward, lb_linear_stage1 and lb_linear_stage2 call of these
 * sizes and flags.  0 on bad arguments. */
size_t lb_linear_workspace_bytes(int64_t d_in, int64_t d_out, int64_t r, int64_t T,
                                 int residual, unsigned flags);

/* One linear (Proposition 1, plus the residual path when residual != 0):
 * x [T][d_in] (x_dtype) -> y [T][d_out] (y_dtype), row-major, token-major
 * (rows of X are tokens, as in Proposition 1).  r is the TOTAL rank; with the
 * residual r must be even and each path has rank r/2.  T == 0 is a no-op.
 * ws: device workspace of at least lb_linear_workspace_bytes(...) bytes,
 * 256-byte aligned, contents need not be initialised and are clobbered.
 * x and y must not overlap each other or ws (LB_EINVAL).
 * Path choice (flags): AUTO uses the decode kernels for T <= 8 and the MFMA
 * GEMM kernels above for bf16 outputs (the GEMMs are faster from 9 tokens
 * on), the decode kernels for T <= 32 for fp32 outputs; DECODE forces
 * the decode kernels up to 32 tokens; PREFILL with y_dtype LB_F32 is LB_EUNSUPPORTED (the
 * GEMM path rounds its operands, including g and h, to bf16, outside the fp32
 * tolerance).  Shapes the GEMM kernels do not take (d_in % 8 != 0, x not
 * 16-byte or g not 4-byte aligned) run on the vector-ALU decode kernels.
 * Calls that overlap on the same workspace race. */
int lb_linear_forward(const void *x, int x_dtype, void *y, int y_dtype,
                      const lb_factors *w, int64_t d_in, int64_t d_out, int64_t r,
                      int64_t T, int residual, void *ws, size_t ws_bytes,
                      unsigned flags, void *stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): lb_linear_forward
 * with the library's own workspace, a fixed device array of
 * LB_NOALLOC_SCRATCH_BYTES per GPU (allocated with the code object, held
 * until the process ends).  Allocates nothing.  Same arguments, results and
 * errors as lb_linear_forward, except that a request whose kernels need more
 * workspace than the array holds returns LB_EWORKSPACE (every configuration
 * linear fits at T <= 32; compare
 * lb_linear_workspace_bytes with LB_NOALLOC_SCRATCH_BYTES).  Every call on a
 * GPU shares that GPU's array: calls that overlap on one GPU (on different
 * streams, or from different threads without ordering) race.  The array keeps
 * the last call's contents; the kernels need none. */
#define LB_NOALLOC_SCRATCH_BYTES (32u << 20)
int lb_linear_forward_noalloc(const void *x, int x_dtype, void *y, int y_dtype,
                              const lb_factors *w, int64_t d_in, int64_t d_out, int64_t r,
                              int64_t T, int residual, unsigned flags, void *stream);

/* The two halves of lb_linear_forward around the rank-r intermediate, the
 * latents t [T][r] (row-major, token-major; with the residual, path p in
 * columns p*r/2 .. (p+1)*r/2 - 1): t = l_p (.) (sign(V_p)^T (g_p (.) x)).
 * A k or v projection can keep t per token instead of its d_out-wide output
 * (sesamedisk page, "The real result": up to 21.3x smaller for Llama2-7B,
 * 4096 / 192) and expand any number of cached tokens later with stage 2.
 *   stage 1: x [T][d_in] (x_dtype) -> t (t_dtype, LB_F32 or LB_BF16)
 *   stage 2: t (t_dtype) -> y [T][d_out] (y_dtype) = sum_p h_p (.) (sign(U_p) t_p)
 * Both take the layer's full sizes and factors, the workspace of
 * lb_linear_workspace_bytes and the flags of lb_linear_forward; stage 1 also
 * takes the y_dtype of the layer's output, which selects the kernels (and so
 * the precision) as lb_linear_forward does.  Stage 1 then stage 2 gives the
 * bits of lb_linear_forward when t holds the kernels' own latent precision:
 * LB_F32 always, LB_BF16 on the GEMM (prefill) kernels.  A bf16 t on the other
 * kernels rounds the latents once more (within the bf16 tolerance).  t must
 * not overlap x, y or ws.  Errors as lb_linear_forward. */
int lb_linear_stage1(const void *x, int x_dtype, void *t, int t_dtype, int y_dtype,
                     const lb_factors *w, int64_t d_in, int64_t d_out, int64_t r, int64_t T,
                     int residual, void *ws, size_t ws_bytes, unsigned flags, void *stream);
int lb_linear_stage2(const void *t, int t_dtype, void *y, int y_dtype, const lb_factors *w,
                     int64_t d_in, int64_t d_out, int64_t r, int64_t T, int residual,
                     void *ws, size_t ws_bytes, unsigned flags, void *stream);

/* One decoder layer of a model whose seven linears are LittleBit linears
 * (the model architecture is otherwise unchanged: littlebitllm page, hero;
 * deniz.in, "Factorize first, then binarize"), at decode time, minus
 * attention over a KV cache.  Pre-norm (the Llama / Qwen layout):
 *     a = x / rms(x);  q, k, v = Q(a), K(a), V(a)
 *     o_in = v with each kv head serving its group of n_heads / n_kv_heads
 *            query heads (attention over a context of one token)
 *     x1 = x + O(o_in);  b = x1 / rms(x1)
 *     y = x1 + Down(silu(Gate(b)) (.) Up(b))
 * rms(x) = sqrt(mean(x^2) + eps) per token; the RMSNorms' per-channel weights
 * are folded into the g of the linears they feed (g scales the same input
 * channels).  q and k are computed (they cost what they cost) but, with one
 * token of context, do not change o_in.  Shapes: q, o d_model x d_model (total
 * rank r_qo); k, v d_model -> d_model / n_heads * n_kv_heads (r_kv); gate, up
 * d_model -> d_ff (r_gu); down d_ff -> d_model (r_down); `residual` gives
 * every linear the residual path.  x, y: bf16 [T][d_model] device, 16-byte
 * aligned, not overlapping; 0 <= T <= 32 (the decode kernels;
 * LB_EUNSUPPORTED beyond; T = 0 checks the layer and does nothing; the
 * workspace query returns 0 for it and for bad arguments).  Work on `stream`:
 * an RMS kernel (which also clears the runs' scratch), q/k/v as one group,
 * o (reading v through the kv-head map, or after an expansion kernel when
 * T > 8 and heads are grouped), a second RMS kernel, gate/up as one group,
 * down; each group or linear is one launch at T <= 2 and three beyond.  Every
 * intermediate lives in ws (>= lb_decoder_layer_workspace_bytes, 256-byte
 * aligned, no contents needed).  Layers chain by passing one's y as the next
 * one's x. */
typedef struct lb_decoder_layer {
    lb_factors q, k, v, o, gate, up, down;
    int64_t d_model, d_ff, n_heads, n_kv_heads;
    int64_t r_qo, r_kv, r_gu, r_down;
    int32_t residual;
    float eps;
} lb_decoder_layer;

size_t lb_decoder_layer_workspace_bytes(const lb_decoder_layer *layer, int64_t T);
int lb_decoder_layer_forward(const lb_decoder_layer *layer, const void *x, void *y, int64_t T,
                             void *ws, size_t ws_bytes, void *stream);

/* Dual-SVID initialisation of a LittleBit linear from a dense weight
 * (sesamedisk, "How low-rank binarization works", the Dual-SVID paragraph;
 * mlsanity, abstract).  Off the forward path: it writes the factors the
 * forward calls read.
 *   1. truncated SVD W ~ U_r S_r V_r^T (r_p = r / P triplets), the singular
 *      values split evenly: U' = U_r sqrt(S_r), V' = V_r sqrt(S_r);
 *   2. binary factors sign(U'), sign(V') (bit = value < 0);
 *   3. |U'| ~ h l_u^T and |V'| ~ g l_v^T, best rank-1 fits (their top
 *      singular pair, nonnegative, sqrt(sigma_1) in each vector); l = l_u (.) l_v;
 *      h, g, l stored as fp16 (round to nearest even);
 *   4. residual != 0: path 1 is the same on W - W_1, W_1 being path 0 as stored.
 * w: fp32 [d_out][d_in] row-major, device, 4-byte aligned, not modified.
 * r: total rank (even with the residual), r / P <= min(d_out, d_in).
 * out: where the factors go, in the layout lb_linear_forward reads (the
 *   buffers it points to are written: v_bits [P][ceil(d_in/32)][ld_v],
 *   u_bits [P][ceil(r_p/32)][ld_u], g, l, h fp16 bits), ld_v >= r_p,
 *   ld_u >= d_out.  u_out / v_out: optional fp32 [P][d_out][r_p] and
 *   [P][d_in][r_p] copies of U' and V' (null: not written).  A singular
 *   vector's sign is arbitrary: U' and V' columns may come out negated
 *   together, which leaves the layer unchanged.
 * ws: >= lb_dual_svid_workspace_bytes, 256-byte aligned, no contents needed.
 * The SVD is one-sided Jacobi on the GPU; the call waits for the stream after
 * each sweep to test convergence, so it returns with the work done (not
 * capturable).  LB_EUNSUPPORTED if 40 sweeps do not converge or
 * d_out * d_in >= 2^31. */
size_t lb_dual_svid_workspace_bytes(int64_t d_out, int64_t d_in, int64_t r, int residual);
int lb_dual_svid(const float *w, int64_t d_out, int64_t d_in, int64_t r, int residual,
                 const lb_factors *out, float *u_out, float *v_out, void *ws, size_t ws_bytes,
                 void *stream);

/* Joint-ITQ rotation of a path's latent factors (LittleBit-2: littlebitllm,
 * hero and "The method"; trove, "How it works", step 2; deniz.in,
 * "LittleBit-2 fixes the initialization": a rotation of the latent space that
 * lines the SVD-derived factors up with the binary hypercube and folds into
 * them).  Off the forward path.  For an orthogonal R, (U'R)(V'R)^T = U'V'^T;
 * R is chosen to minimise
 *     Q(R) = ||sign(U'R) - U'R||_F^2 + ||sign(V'R) - V'R||_F^2
 * by `iters` alternations of: codes B = sign of the rotated factors (+1 for
 * zero), then R = the orthogonal polar factor of U'^T B_u + V'^T B_v (the
 * orthogonal Procrustes solution, computed by Newton-Schulz iteration in fp32).
 * u: fp32 [d_out][r_p] U', v: fp32 [d_in][r_p] V' (device, row-major), both
 *   replaced by the rotated factors U'R, V'R.  r_p <= min(d_out, d_in).
 * rot0: optional fp32 [r_p][r_p] starting rotation (null: the identity, the
 *   unrotated factors); rot: optional fp32 [r_p][r_p] output, the final R.
 * objective: optional fp64 [iters + 1] device array: Q at the start and after
 *   each alternation (never increasing, up to fp32 rounding).
 * ws: >= lb_joint_itq_workspace_bytes, 256-byte aligned, no contents needed.
 * The call waits for the stream (it reads the polar iteration's progress) and
 * returns with the work done; not capturable.  LB_EUNSUPPORTED when a polar
 * decomposition did not converge in 64 iterations (u, v hold the factors
 * rotated by the last R that did), or (d_out + d_in) * r_p >= 2^31, or
 * r_p >= 2^15. */
size_t lb_joint_itq_workspace_bytes(int64_t d_out, int64_t d_in, int64_t r_p);
int lb_joint_itq(float *u, float *v, int64_t d_out, int64_t d_in, int64_t r_p, int iters,
                 const float *rot0, float *rot, double *objective, void *ws, size_t ws_bytes, void *stream);

/* Dual-SVID initialisation with the Joint-ITQ rotation (LittleBit-2): as
 * lb_dual_svid, with each path's U' and V' turned by lb_joint_itq's rotation
 * (itq_iters alternations from the identity) between the SVD split and the
 * signs and scales; the residual path is fitted to what the first path, as
 * stored, leaves.  itq_iters = 0 gives lb_dual_svid's result.  u_out / v_out
 * receive the rotated factors.  ws: >= lb_dual_svid_itq_workspace_bytes.
 * Waits for the stream; LB_EUNSUPPORTED as lb_dual_svid, or when a polar
 * decomposition did not converge. */
size_t lb_dual_svid_itq_workspace_bytes(int64_t d_out, int64_t d_in, int64_t r, int residual);
int lb_dual_svid_itq(const float *w, int64_t d_out, int64_t d_in, int64_t r, int residual, int itq_iters,
                     const lb_factors *out, float *u_out, float *v_out, void *ws, size_t ws_bytes,
                     void *stream);

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

/* One independent linear of lb_linear_forward_grouped: the arguments of
 * lb_linear_forward (x [T][d_in], y [T][d_out], device pointers). */
typedef struct lb_linear_call {
    const void *x;
    void *y;
    lb_factors w;
    int64_t d_in, d_out, r, T;
    int32_t residual;
    int32_t x_dtype, y_dtype;
    uint32_t flags;     /* path flags, and LB_GROUP_FAULT_TEST */
} lb_linear_call;

/* Workspace bytes lb_linear_forward_grouped needs for these calls.  0 on bad
 * arguments. */
size_t lb_linear_grouped_workspace_bytes(const lb_linear_call *calls, int n);

/* n independent linears in few launches (q/k/v, a layer, a layer stack):
 * every calls[i].y = layer_i(calls[i].x), as n calls of lb_linear_forward
 * would give.  Stateless: nothing carries over from earlier calls, ws
 * (device, 256-byte aligned, >= lb_linear_grouped_workspace_bytes) needs no
 * contents and is clobbered, and the call may be captured in a graph.  Calls
 * with equal (T, x_dtype, y_dtype, flags) run together as one group, in the
 * order of their first appearance; groups run one after another on `stream`.
 * Each group run first copies its work tables into ws (host to device, about
 * 100 bytes per linear plus 12-20 bytes per work item) and clears its
 * counters; the tables are planned on the host on first use of an argument set
 * and cached (the last 8 sets: key = the calls' bytes, ws, ws_bytes and the
 * device; the cache holds pinned host copies of the tables; a set whose call
 * was captured in a graph keeps its copy, which the graph's copy node reads,
 * until the process ends).  For a group that runs many times,
 * lb_grouped_prepare / lb_grouped_run skip the copy.
 * Errors as lb_linear_forward; every call is checked before anything is
 * enqueued.  No output may overlap an input, another output or ws. */
int lb_linear_forward_grouped(const lb_linear_call *calls, int n, void *ws, size_t ws_bytes,
                              void *stream);

/* Workspace bytes for a group of n linears at T tokens. 0 on bad arguments. */
size_t lb_grouped_workspace_bytes(const lb_linear_desc *descs, int n, int64_t T, unsigned flags);

/* Build the device work table of a group into ws and keep a host record of
 * the group, keyed by ws (lb_grouped_release forgets it; preparing another
 * group on the same ws replaces it).  BLOCKS until the table is on the device
 * (a setup call, not for the timed loop); ws must not be written until the
 * group is released, except by the group's own runs.  descs is a host array
 * of n descriptors; it is copied and may be freed afterwards.  All linears use
 * x_dtype / y_dtype and T tokens.  The pointers in descs are captured: later
 * runs read and write the same buffers.  The kernels a group runs:
 *  - the matrix-core decode kernels where lb_linear_forward's path choice
 *    picks them (1 <= T <= 8, or up to 32 with fp32 outputs or the DECODE
 *    flag) (stage 1 = activation operands, first contractions and latents;
 *    stage 2 = second contractions);
 *  - where it picks the GEMM kernels (bf16 output), bf16 input and shapes they take
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
 * the LDS runs as ONE launch: each linear's stage 2 starts as soon as its own
 * stage 1 and latents are done.  Its workgroups hand the latents over through
 * counters in ws, which every run leaves at zero, so a run needs no state from
 * the host: a run may be captured in a graph and replayed.  Runs that overlap
 * on the same workspace race.  Every launch first checks the stamp
 * lb_grouped_prepare wrote into ws: if ws was reused or overwritten since,
 * the launch does nothing and reports LB_FAULT_STALE_WORKSPACE.  A stage-2
 * wait that gives up reports LB_FAULT_HANDOFF_TIMEOUT.  Either is read with
 * lb_device_faults; after one, prepare the group again.  LB_EINVAL for a ws
 * with no prepared group. */
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

/* ---- measured ceilings (measurement helpers; no part of the layer) ---- */

/* A streaming read of bytes (>= 16; buf 16-byte aligned, device) by `blocks`
 * workgroups of 256 threads, each reading a contiguous share with 16-byte
 * non-temporal loads, 8 in flight per thread: the HBM read rate a decode sign
 * stream can reach.  out (device)
 * receives one uint32_t per workgroup (the XOR of what it read).  Enqueued
 * on stream; time it with events.  LB_EINVAL on bad arguments. */
int lb_ceiling_stream_read(const void *buf, size_t bytes, void *out, int blocks, void *stream);

/* `blocks` workgroups of 4 waves, each wave issuing iters x 8 independent
 * v_mfma_f32_32x32x16_bf16 (32768 flops each) on register operands: the
 * bf16 matrix rate the prefill GEMMs can reach.  random_operands 0: the same
 * few, mostly constant operand words in every instruction; 1: the
 * instructions cycle through four pseudo-random A and B operands each (random
 * signs and mantissas), whose toggling inputs draw the power a GEMM on real
 * data draws.  out (device) receives blocks * 256 floats.  Enqueued on
 * stream.  LB_EINVAL on bad arguments (random_operands other than 0 or 1). */
int lb_ceiling_mfma_bf16(int iters, int random_operands, void *out, int blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LITTLEBIT_H */
