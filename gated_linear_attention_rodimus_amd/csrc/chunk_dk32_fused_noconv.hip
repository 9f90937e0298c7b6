// chunk_dk32_fused_noconv.hip -- chunk-forward kernels for dk = 32 with the
// fused steps that need no history rows (beta_hat from low-rank factors, the
// feedthrough d): the fused kernels without the ShortConv, which keep no
// convolution window, taps or extra v rows.  The kernel itself is in
// chunk_kernel.h.
#include "chunk_kernel.h"

namespace rodimus {
RODIMUS_DEFINE_CHUNK(32, 2, dk32_fn)
}  // namespace rodimus
