// chunk_dk128_fused_noconv.hip -- chunk-forward kernels for dk = 128 with the
// fused steps that need no history rows (beta_hat from low-rank factors, the
// feedthrough d): the fused kernels without the ShortConv, which keep no
// convolution window, taps or extra v rows.  The kernel itself is in
// chunk_kernel.h.
#include "chunk_kernel.h"

namespace rodimus {
RODIMUS_DEFINE_CHUNK(128, 2, dk128_fn)
}  // namespace rodimus
