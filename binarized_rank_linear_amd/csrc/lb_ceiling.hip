// lb_ceiling.hip -- the two measured ceilings the layer's figures are compared
// against, besides the published peaks: a streaming read of device memory
// (what the decode kernels' sign streams can reach) and back-to-back bf16
// matrix instructions on register operands (what the prefill GEMMs can reach).
// Measurement helpers only; no part of the layer runs here.
#include "lb_internal.h"

namespace lb {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Workgroup b reads its own contiguous 1/gridDim share of the buffer, 4 KB
// per step (256 threads x 16 bytes), 8 steps in flight per thread; the XOR of
// everything read goes to out[b] so no load can be dropped.
__global__ __launch_bounds__(256) void k_stream_read(const u32x4 *__restrict__ p, int64_t n16, uint32_t *out) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t b0 = (int64_t)blockIdx.x * per;
    const int64_t b1 = b0 + per < n16 ? b0 + per : n16;
    u32x4 acc = {0u, 0u, 0u, 0u};
    int64_t i = b0 + threadIdx.x;
    for (; i + 7 * 256 < b1; i += 8 * 256) {
        u32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = __builtin_nontemporal_load(p + i + k * 256);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc ^= v[k];
    }
    for (; i < b1; i += 256) acc ^= p[i];
    const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    __shared__ uint32_t s[256];
    s[threadIdx.x] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int k = 0; k < 256; ++k) r ^= s[k];
        out[blockIdx.x] = r;
    }
}

// A bf16 pair of lane-varying values 1.0-ish in magnitude with random signs and
// mantissas: sign and low mantissa bits from a 32-bit mix of the lane and a
// salt, exponent fixed at 2^0 or 2^-1 (so no product or sum leaves the normal
// range over any iteration count the benchmark uses).
__device__ inline uint32_t rand_pair(uint32_t l, uint32_t salt) {
    uint32_t h = (l + 1u) * 0x9e3779b1u ^ salt * 0x85ebca77u;
    h ^= h >> 15;
    h *= 0x2c1b3c6du;
    h ^= h >> 12;
    return (h & 0x807f807fu) | 0x3f003f00u | ((h >> 8) & 0x00800080u);
}

// Each wave runs `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 on
// register operands (8 accumulators, so the instructions never wait for each
// other's results); the accumulators' sum goes to out so none is dropped.
// With random_operands = 0 every instruction reads the same few, mostly
// constant, operand words; with 1 the 8 instructions of a round cycle through
// four pseudo-random A and four pseudo-random B operands, so the inputs of
// consecutive instructions differ in about half their bits, as in a GEMM on
// real data (the matrix units draw more power on toggling inputs).
template <bool RANDOM>
__global__ __launch_bounds__(256) void k_mfma_bf16(int iters, float *out) {
    const uint32_t l = threadIdx.x;
    u32x4 a[4], b[4];
    if (RANDOM) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[q][e] = rand_pair(l, 8u * q + e);
                b[q][e] = rand_pair(l, 8u * q + e + 4u);
            }
    } else {
        a[0] = u32x4{l * 0x00010001u, l ^ 0x3f803f80u, 0x3f803f80u, l};
        b[0] = u32x4{0x3c003c00u ^ l, 0x3f80bf80u, l << 3, 0x40004000u};
    }
    f32x16 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) c[j][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const u32x4 x = RANDOM ? a[j & 3] : a[0];
            const u32x4 y = RANDOM ? b[(j + (j >> 2)) & 3] : b[0];
            c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y),
                                                          c[j], 0, 0, 0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += c[j][e];
    out[(int64_t)blockIdx.x * 256 + l] = s;
}

}  // namespace
}  // namespace lb

extern "C" int lb_ceiling_stream_read(const void *buf, size_t bytes, void *out, int blocks, void *stream) {
    if (!buf || !out || bytes < 16 || blocks <= 0 || ((uintptr_t)buf & 15) || ((uintptr_t)out & 3)) return LB_EINVAL;
    lb::k_stream_read<<<blocks, 256, 0, (hipStream_t)stream>>>((const lb::u32x4 *)buf, (int64_t)(bytes / 16),
                                                                (uint32_t *)out);
    return lb::last_launch_status();
}

extern "C" int lb_ceiling_mfma_bf16(int iters, int random_operands, void *out, int blocks, void *stream) {
    if (!out || iters <= 0 || blocks <= 0 || ((uintptr_t)out & 3) || (random_operands != 0 && random_operands != 1))
        return LB_EINVAL;
    if (random_operands)
        lb::k_mfma_bf16<true><<<blocks, 256, 0, (hipStream_t)stream>>>(iters, (float *)out);
    else
        lb::k_mfma_bf16<false><<<blocks, 256, 0, (hipStream_t)stream>>>(iters, (float *)out);
    return lb::last_launch_status();
}
