// chunk_dk64_fused.hip -- chunk-forward kernels for dk = 64 with the fused steps
// around the recurrence compiled in (beta_hat from low-rank factors, ShortConv
// of q, k, v, the feedthrough d).  The kernel itself is in chunk_kernel.h.
#include "chunk_kernel.h"

namespace rodimus {
RODIMUS_DEFINE_CHUNK(64, 1, dk64_fu)
}  // namespace rodimus
