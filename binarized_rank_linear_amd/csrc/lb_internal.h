// lb_internal.h -- shared declarations of the HIP implementation of littlebit.h.
//
// Device helpers for the storage types and the resolved argument block that
// the host entry points hand to the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <vector>

#include "littlebit.h"

namespace lb {

// Resolved arguments of one linear (one call of lb_linear_forward).
struct Linear {
    const void *x;
    void *y;
    // SwiGLU input (decode kernels, bf16 x only): when set, the linear's input
    // is silu(x) (.) x2 elementwise, x2 [T][d_in] bf16
    const void *x2 = nullptr;
    // decode kernels only: a per-token scale of the input ([T] fp32: an
    // RMSNorm's 1/rms), and a residual [T][d_out] (y's dtype) added to y
    const float *xs = nullptr;
    const void *resid = nullptr;
    // decode kernels, fused stage 1 only (mfma_fused_stage1): input channel i
    // reads x[n][(i / xm_dh / xm_grp) * xm_dh + i % xm_dh] from rows of
    // d_in / xm_grp (each head of xm_dh channels of x serves xm_grp heads);
    // xm_dh = 0: x as it is
    int32_t xm_dh = 0, xm_grp = 1;
    int x_dtype, y_dtype;
    const uint32_t *v_bits;   // [P][kw_v][ld_v]
    const uint32_t *u_bits;   // [P][kw_u][ld_u]
    const uint16_t *g, *l, *h;
    int64_t ld_v, ld_u;
    int64_t d_in, d_out, r_p;
    int P;
    int64_t T;

    __host__ __device__ int64_t kw_v() const { return (d_in + 31) / 32; }   // planes of V
    __host__ __device__ int64_t kw_u() const { return (r_p + 31) / 32; }    // planes of U
};

// ---- storage types ---------------------------------------------------------

__device__ __forceinline__ float f16_to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float load_act(const void *p, int dtype, int64_t i) {
    return dtype == LB_F32 ? ((const float *)p)[i] : bf16_to_f32(((const uint16_t *)p)[i]);
}

__device__ __forceinline__ void store_act(void *p, int dtype, int64_t i, float v) {
    if (dtype == LB_F32) ((float *)p)[i] = v;
    else ((uint16_t *)p)[i] = f32_to_bf16(v);
}

// Multiply by +-1 given as a sign mask (0 or 0x80000000): a sign flip.
__device__ __forceinline__ float flip(float v, uint32_t signmask) {
    return __uint_as_float(__float_as_uint(v) ^ signmask);
}

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }
__host__ __device__ constexpr int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
__host__ __device__ constexpr int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }

// ---- launchers (each returns LB_OK or LB_EHIP) ------------------------------

int launch_pack(const float *src, int64_t rows, int64_t cols, int axis, uint32_t *dst,
                int64_t ld, hipStream_t s);

// Plain vector-ALU decode path.
size_t valu_workspace_bytes(const Linear &a);
int valu_forward(const Linear &a, void *ws, hipStream_t s);
// The latent API on each kernel family: stage 1 writes the latents t
// [T][P*r_p] (t_dtype) as the layer computes them; stage 2 computes the output
// from given latents.  Stage 1 then stage 2 equals the whole layer bit for bit
// when t_dtype holds the family's own latent precision (fp32 on the decode
// kernels, bf16 or fp32 on the GEMM kernels, fp32 on the vector-ALU kernels).
int valu_stage_forward(const Linear &a, void *ws, int stage, void *t, int t_dtype, hipStream_t s);
int mfma_decode_stage(const Linear &a, void *ws, int stage, void *t, int t_dtype, hipStream_t s);
int gemm_stage_forward(const Linear &a, void *ws, int stage, void *t, int t_dtype, hipStream_t s);

// The set-up of a group of linears: what its workspace must hold before a
// run.  Bytes [0, bytes.size()) of the workspace are `bytes` (header with the
// stamp, tables, zeroed counters); [zero_off, zero_off + zero_bytes) are zero.
struct GroupImage {
    std::vector<uint8_t> bytes;
    size_t zero_off = 0, zero_bytes = 0;
};

// Matrix-core decode path (fp4 signs x fp8 activation limbs).
bool mfma_decode_supported(int64_t T, int y_dtype);
// Whether stage 1 runs in its fused form at this T (input maps apply there).
bool mfma_fused_stage1(int64_t T, int y_dtype);
// Whether the decode kernels' 32-bit buffer offsets cover this linear.
bool mfma_decode_shape_ok(const Linear &a);
size_t mfma_decode_workspace_bytes(const Linear &a);
int mfma_decode_forward(const Linear &a, void *ws, hipStream_t s);
// Up to kMaxInline linears (same T and dtypes) in one run, with their
// schedule in the kernel arguments instead of device tables: nothing to set
// up, so a stateless call can use it.  Where the one-launch pass applies
// (mfma_inline_pass) the run is a clear of the workspace and one launch (or
// the launch alone when the caller has cleared it: zeroed); else the
// three-launch form.
constexpr int kMaxInline = 3;
bool mfma_inline_pass(const Linear *ls, int n);
size_t mfma_inline_workspace_bytes(const Linear *ls, int n);
int mfma_inline_forward(const Linear *ls, int n, void *ws, hipStream_t s, bool zeroed = false);
// Groups of independent linears on the matrix-core decode path.
size_t mfma_group_workspace_bytes(const Linear *ls, int n, int64_t T, int y_dtype);
size_t mfma_group_state_bytes();
// Plans a group on workspace ws: fills the host state and the image.
// fault_test: the one-launch pass's waits ask for one latent group more than
// exists and give up after a few polls (LB_GROUP_FAULT_TEST).
int mfma_group_plan(const Linear *ls, int n, int64_t T, int y_dtype, void *ws, size_t ws_bytes, uint64_t tag,
                    bool fault_test, void *host_state, GroupImage *img);
int mfma_group_run(const void *host_state, hipStream_t s, int stage_mask = 3);

// Reads and clears this device's fault word (after the work on s is done).
int take_faults(hipStream_t s, uint32_t *faults);
// Sets bytes / 4 words at p to v (a kernel, so it may be captured in a graph).
int fill_words(void *p, size_t bytes, uint32_t v, hipStream_t s);

// GEMM (prefill) path: bf16 matrix cores; shapes it does not take (d_in % 8,
// misaligned x) run on the vector-ALU kernels.
bool gemm_linear_supported(const Linear &a);
size_t gemm_workspace_bytes(const Linear &a);
int gemm_forward(const Linear &a, void *ws, hipStream_t s);
// Groups of independent linears on the GEMM path: the factor preparation
// (bf16 g, unzipped sign words), stage 1 (+ reduce), stage 2.
bool gemm_group_supported(const Linear *ls, int n);
size_t gemm_group_workspace_bytes(const Linear *ls, int n);
size_t gemm_group_state_bytes();
int gemm_group_plan(const Linear *ls, int n, void *ws, size_t ws_bytes, uint64_t tag, void *host_state,
                    GroupImage *img);
// stage_mask: bit 0 stage 1, bit 1 stage 2, bit 2 the factor preparation
// (before stage 1), which a prepared group runs once at set-up.
int gemm_group_run(const void *host_state, hipStream_t s, int stage_mask = 3);
// The fault word of the current device (kernels of other sources report
// through this pointer).
uint32_t *fault_word_ptr();

// Joint-ITQ (lb_itq.hip): F = [U'; V'] ([D][r] fp32, D = d_out + d_in) is
// replaced by F R, R the rotation after `iters` alternations from rot0 (the
// identity when null).  rot_out ([r][r]) and objective ([iters + 1] fp64)
// are optional.  ws: itq_workspace_bytes(D, r), 256-byte aligned.  Waits for
// the stream; LB_EUNSUPPORTED when a polar decomposition did not converge.
size_t itq_workspace_bytes(int64_t D, int64_t r);
int itq_rotate(float *F, int64_t D, int64_t r, int iters, const float *rot0, float *rot_out, double *objective,
               void *ws, hipStream_t s);

// SwiGLU gate: a = silu(gate) * up, elementwise over n values (fp32 in place).
int launch_swiglu_f32(float *gate_io, const float *up, int64_t n, hipStream_t s);

// Records the text of the last HIP error seen on this thread (lb_last_hip_error).
void note_hip_error(hipError_t e);

inline int hip_status(hipError_t e) {
    if (e == hipSuccess) return LB_OK;
    note_hip_error(e);
    return LB_EHIP;
}
inline int last_launch_status() { return hip_status(hipGetLastError()); }

}  // namespace lb
