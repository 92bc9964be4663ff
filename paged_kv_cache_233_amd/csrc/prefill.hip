// Chunked-prefill attention over paged KV (placeholder until the MFMA kernel
// lands): reports that the operation is not available yet.
#include "internal.h"

namespace pkv {

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  (void)a;
  (void)stream;
  return hipErrorNotSupported;
}

}  // namespace pkv
