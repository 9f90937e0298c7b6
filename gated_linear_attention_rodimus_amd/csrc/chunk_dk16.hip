// chunk_dk16.hip -- chunk-forward kernels for dk = 16 (all dv tiles and chunk
// lengths, bf16 and fp32 inputs).  The kernel itself is in chunk_kernel.h.
#include "chunk_kernel.h"

namespace rodimus {
RODIMUS_DEFINE_CHUNK(16, 0, dk16)
}  // namespace rodimus
