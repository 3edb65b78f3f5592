// Chunked SSD prefill (not yet available: m2_prefill reports M2_ERR_UNSUPPORTED).
#include "m2_internal.h"

namespace m2d {

size_t prefill_ws_bytes(const m2_layer_s &, int, int, int) { return 0; }

hipError_t launch_prefill(const m2_layer_s &, const m2_state_s &, const float *, float *, int, int, int,
                          const int32_t *, int, void *, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace m2d
