// Matrix-product predictor bases (block-DPLR cross-layer, temporal key->value).
// Not built yet: every request reports hipErrorNotSupported, which the entry
// points turn into an error status.
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

bool predict_available() { return false; }

size_t encode_workspace_bytes(const CodecArgs& c, int64_t n_tokens) {
  (void)c;
  (void)n_tokens;
  return 0;
}

hipError_t launch_predict(const EncodeLaunch& a, float* base_out, hipStream_t s) {
  (void)a;
  (void)base_out;
  (void)s;
  return hipErrorNotSupported;
}

}  // namespace kvc
