// NanoKV-Fast style mixed-dimensional attention (not built yet).
#include "kvc_device.h"
#include "kvc_internal.h"

namespace kvc {

hipError_t launch_attend_mixed(const AttendLaunch& a, hipStream_t s) {
  (void)a;
  (void)s;
  return hipErrorNotSupported;
}

}  // namespace kvc
