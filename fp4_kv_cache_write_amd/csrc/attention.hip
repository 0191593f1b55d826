// Sparse gather-attention (placeholder until the kernel lands).
#include "common.h"
#include "internal.h"

namespace csa2 {

size_t sparse_decode_ws(int, int, int) { return 0; }

int launch_sparse_decode(const csa2_cache_t&, int, int, const int32_t*, const uint16_t*,
                         const int32_t*, int, const uint16_t*, int, float, uint16_t*, float*, void*,
                         hipStream_t) {
  return CSA2_EUNSUPPORTED;
}

}  // namespace csa2
