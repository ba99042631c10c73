#include "common.hpp"
namespace eao {
hipError_t launch_fp8_prep(const float*, uint8_t*, float*, const int8_t*, int, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_fwd_fp8(const uint8_t*, const uint8_t*, const uint8_t*, uint16_t*, float*, const float*,
                          const float*, const float*, int, int, int, int, int, bool, float, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace eao
