// chunk_dk64.hip -- chunk-forward kernels for dk = 64 (all dv tiles and chunk
// lengths, bf16 and fp32 inputs).  The kernel itself is in chunk_kernel.h.
#include "chunk_kernel.h"

namespace rodimus {
RODIMUS_DEFINE_CHUNK(64, 0, dk64)
}  // namespace rodimus
