// chunk_dk128.hip -- chunk-forward kernels for dk = 128 (all dv tiles and chunk
// lengths, bf16 and fp32 inputs).  The kernel itself is in chunk_kernel.h.
#include "chunk_kernel.h"

namespace rodimus {
RODIMUS_DEFINE_CHUNK(128, 0, dk128)
}  // namespace rodimus
