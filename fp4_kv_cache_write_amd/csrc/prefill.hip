// Chunked prefill (placeholder until the kernel lands).
#include "common.h"
#include "internal.h"

namespace csa2 {

size_t prefill_ws(int, int, int64_t, int, int) { return 0; }

int launch_prefill_chunk(const csa2_cache_t&, int, int, const int32_t*, int64_t, int,
                         const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*, int, int,
                         float, uint16_t*, int32_t*, void*, hipStream_t) {
  return CSA2_EUNSUPPORTED;
}

}  // namespace csa2
