// lb_internal.h -- shared declarations of the HIP implementation of littlebit.h.
//
// Device helpers for the storage types and the resolved argument block that
// the host entry points hand to the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "littlebit.h"

namespace lb {

// Resolved arguments of one linear (one call of lb_linear_forward).
struct Linear {
    const void *x;
    void *y;
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

// Matrix-core decode path (fp4 signs x fp8 activation limbs).
bool mfma_decode_supported(int64_t T, int y_dtype);
size_t mfma_decode_workspace_bytes(const Linear &a);
int mfma_decode_forward(const Linear &a, void *ws, hipStream_t s);
// Groups of independent linears on the matrix-core decode path: two launches per run.
size_t mfma_group_workspace_bytes(const Linear *ls, int n, int64_t T, int y_dtype);
size_t mfma_group_state_bytes();
int mfma_group_prepare(const Linear *ls, int n, int64_t T, int y_dtype, void *ws, size_t ws_bytes,
                       void *host_state, hipStream_t s);
int mfma_group_run(const void *host_state, hipStream_t s, int stage_mask = 3);

// GEMM (prefill) path: bf16 matrix cores; shapes it does not take (d_in % 8,
// misaligned x) run on the vector-ALU kernels.
size_t gemm_workspace_bytes(const Linear &a);
int gemm_forward(const Linear &a, void *ws, hipStream_t s);
// Groups of independent linears on the GEMM path: stage 1 (+ reduce), stage 2.
bool gemm_group_supported(const Linear *ls, int n);
size_t gemm_group_workspace_bytes(const Linear *ls, int n);
size_t gemm_group_state_bytes();
// Also prepares the captured factors (bf16 g, unzipped sign words) on stream s
// and waits for it.
int gemm_group_prepare(const Linear *ls, int n, void *ws, size_t ws_bytes, void *host_state,
                       hipStream_t s);
int gemm_group_run(const void *host_state, hipStream_t s, int stage_mask = 3);

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
