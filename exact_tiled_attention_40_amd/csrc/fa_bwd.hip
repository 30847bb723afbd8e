#include "fa_device.hpp"
#include "fa_internal.h"
namespace fa {
hipError_t launch_backward(const AttnShape&, const void*, const void*, const void*, const void*, const float*,
                           const void*, void*, void*, void*, float*, float*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace fa
