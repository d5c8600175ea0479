// lb_mlp.hip -- elementwise part of the SwiGLU block: a = silu(gate) * up.
#include "lb_internal.h"

namespace lb {

// silu(z) = z / (1 + exp(-z)).  For z below about -88 exp(-z) is +inf in fp32
// and the quotient is -0, so large negative pre-activations give no NaN.
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__global__ __launch_bounds__(256) void k_swiglu_f32(float *__restrict__ g, const float *__restrict__ u,
                                                    int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) g[i] = silu(g[i]) * u[i];
}

int launch_swiglu_f32(float *gate_io, const float *up, int64_t n, hipStream_t s) {
    if (n <= 0) return LB_OK;
    k_swiglu_f32<<<(unsigned)cdiv(n, 256), 256, 0, s>>>(gate_io, up, n);
    return last_launch_status();
}

}  // namespace lb
