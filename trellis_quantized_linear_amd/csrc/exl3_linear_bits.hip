// The linear kernels of one bit width, EXL3_BITS (2..8), set by the build:
// this file is compiled once per width, and the host launcher in
// exl3_kernels.hip calls launch_linear_bits<EXL3_BITS>.
#include "exl3_device.h"

#ifndef EXL3_BITS
#error "EXL3_BITS (2..8) must be defined"
#endif

namespace exl3 {

template <int BITS>
int launch_linear_bits(const LinearArgs &a, int kernel, bool chained, void *stream) {
  return launch_linear_t<BITS>(a, kernel, chained, stream);
}

template int launch_linear_bits<EXL3_BITS>(const LinearArgs &, int, bool, void *);

}  // namespace exl3
