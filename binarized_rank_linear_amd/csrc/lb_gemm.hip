// lb_gemm.hip -- MFMA GEMM (prefill) path (placeholder: plain decode kernels).
#include "lb_internal.h"

namespace lb {

size_t gemm_workspace_bytes(const Linear &a) { return valu_workspace_bytes(a); }

int gemm_forward(const Linear &a, void *ws, hipStream_t s) { return valu_forward(a, ws, s); }

}  // namespace lb
