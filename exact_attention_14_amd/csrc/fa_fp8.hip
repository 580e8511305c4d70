// FP8 path: sign generation, block quantisation, and the e4m3 forward kernel.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

hipError_t launch_fill_signs(float*, int, unsigned long long, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_quant_fp8(const void*, void*, float*, int, int, int, int, bool, const float*,
                            hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_fwd_fp8(const void*, const void*, const void*, const float*, const float*,
                          const float*, void*, float*, int, int, int, int, bool, float,
                          hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace fa
