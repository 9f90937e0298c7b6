// chunk_dk32_fused.hip -- chunk-forward kernels for dk = 32 with the fused steps
// around the recurrence compiled in (beta_hat from low-rank factors, ShortConv
// of q, k, v, the feedthrough d).  The kernel itself is in chunk_kernel.h.
#include "chunk_kernel.h"

namespace rodimus {
RODIMUS_DEFINE_CHUNK(32, 1, dk32_fu)
}  // namespace rodimus
