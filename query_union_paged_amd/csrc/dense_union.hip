// Direct KV-page union (design-study comparison).  Work in progress: the
// launcher reports hipErrorNotSupported until the pair kernels land.
#include "pw_internal.h"

namespace pw {

size_t dense_union_workspace(const pw_shape&) { return 0; }

hipError_t launch_dense_union(const pw_shape&, const uint16_t*, const uint8_t*, const uint8_t*,
                              const float*, const int32_t*, uint16_t*, void*, size_t,
                              hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace pw
