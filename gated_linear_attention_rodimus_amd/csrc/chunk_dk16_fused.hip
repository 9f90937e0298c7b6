// chunk_dk16_fused.hip -- chunk-forward kernels for dk = 16 with the fused steps
// around the recurrence compiled in (beta_hat from low-rank factors, ShortConv
// of q, k, v, the feedthrough d).  The kernel itself is in chunk_kernel.h.
#include "chunk_kernel.h"

namespace rodimus {
RODIMUS_DEFINE_CHUNK(16, 1, dk16_fu)
}  // namespace rodimus
