// lb_decode_mfma.hip -- matrix-core decode path (placeholder: plain decode kernels).
#include "lb_internal.h"

namespace lb {

size_t mfma_decode_workspace_bytes(const Linear &a) { return valu_workspace_bytes(a); }

int mfma_decode_forward(const Linear &a, void *ws, hipStream_t s) { return valu_forward(a, ws, s); }

}  // namespace lb
