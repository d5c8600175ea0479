// lb_noalloc.hip -- lb_linear_forward_noalloc: lb_linear_forward for callers
// that cannot allocate (code under graph capture, tight serving loops,
// harnesses that forbid allocation).  Its workspace is a file-scope device
// array of a fixed size, one copy per GPU, held until the process ends.
#include <mutex>

#include "lb_internal.h"

namespace {

static_assert(LB_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch is a whole number of 256-byte lines");

// The workspace of every lb_linear_forward_noalloc call on this GPU.  In host
// code `scratch` names a host-side stand-in, not device memory: host code uses
// the address hipGetSymbolAddress returns for the current device (scratch_on).
static __device__ __align__(256) uint8_t scratch[LB_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];      // scratch's device address, per device (null: not looked up yet)

// The scratch's address on the current device, looked up once per device
// with that device current.
int scratch_on(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return lb::hip_status(hipGetLastError());
    if (dev < 0 || dev >= kMaxDevices) return LB_EUNSUPPORTED;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return lb::hip_status(e);
        if (!p) return LB_EHIP;
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return LB_OK;
}

}  // namespace

extern "C" int lb_linear_forward_noalloc(const void *x, int x_dtype, void *y, int y_dtype, const lb_factors *w,
                                         int64_t d_in, int64_t d_out, int64_t r, int64_t T, int residual,
                                         unsigned flags, void *stream) {
    void *ws = nullptr;
    if (int rc = scratch_on(&ws)) return rc;
    // lb_linear_forward checks every argument, and returns LB_EWORKSPACE when
    // the path this request takes needs more than the scratch holds; it
    // allocates nothing, and the kernels need no particular scratch contents.
    return lb_linear_forward(x, x_dtype, y, y_dtype, w, d_in, d_out, r, T, residual, ws,
                             (size_t)LB_NOALLOC_SCRATCH_BYTES, flags, stream);
}
