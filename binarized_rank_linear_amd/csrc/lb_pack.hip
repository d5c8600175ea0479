// lb_pack.hip -- sign packing (sesamedisk page, "How low-rank binarization
// works": each binary factor entry is stored as a single bit).  Bit b of word
// (w, o) = (src element 32w+b of the packed axis at other-axis index o) < 0.
// Offline, once per layer.
#include "lb_internal.h"

namespace lb {

// Pack down the rows: dst[w][c] from src[32w + b][c].  One thread per output
// word; for each b the wave reads 64 consecutive floats of one row.
__global__ __launch_bounds__(256) void k_pack_axis0(const float *__restrict__ src, int64_t rows,
                                                    int64_t cols, uint32_t *__restrict__ dst,
                                                    int64_t ld) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t w = blockIdx.y;
    if (c >= ld) return;
    uint32_t word = 0;
    if (c < cols) {
        const int64_t r0 = w * 32;
        const int nb = (int)imin(32, rows - r0);
        for (int b = 0; b < nb; ++b) {
            const float v = src[(r0 + b) * cols + c];
            word |= (uint32_t)(v < 0.0f) << b;
        }
    }
    dst[w * ld + c] = word;
}

// Pack along the columns: dst[w][r] from src[r][32w + b].  One wave per
// (row, 64-column span): lanes read 64 consecutive floats and a ballot forms
// two words; padding rows r in [rows, ld) get zero words.
__global__ __launch_bounds__(256) void k_pack_axis1(const float *__restrict__ src, int64_t rows,
                                                    int64_t cols, uint32_t *__restrict__ dst,
                                                    int64_t ld) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t span = blockIdx.y;            // columns [64*span, 64*span + 64)
    if (r >= ld) return;
    const int64_t c = span * 64 + lane;
    const bool neg = (r < rows && c < cols) ? (src[r * cols + c] < 0.0f) : false;
    const uint64_t m = __ballot(neg);
    const int64_t planes = cdiv(cols, 32);
    if (lane == 0) dst[(2 * span) * ld + r] = (uint32_t)m;
    if (lane == 1 && 2 * span + 1 < planes) dst[(2 * span + 1) * ld + r] = (uint32_t)(m >> 32);
}

int launch_pack(const float *src, int64_t rows, int64_t cols, int axis, uint32_t *dst,
                int64_t ld, hipStream_t s) {
    if (axis == 0) {
        dim3 grid((unsigned)cdiv(ld, 256), (unsigned)cdiv(rows, 32));
        k_pack_axis0<<<grid, 256, 0, s>>>(src, rows, cols, dst, ld);
    } else {
        dim3 grid((unsigned)cdiv(ld, 4), (unsigned)cdiv(cols, 64));
        k_pack_axis1<<<grid, 256, 0, s>>>(src, rows, cols, dst, ld);
    }
    return last_launch_status();
}

}  // namespace lb
