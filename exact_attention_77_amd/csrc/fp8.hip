// fp8.hip -- placeholder until the fp8 pre-pass and attention kernels land.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace fa {
int launch_fp8_quantize(const QuantArgs&, void*) { return static_cast<int>(hipErrorNotSupported); }
int launch_fwd_fp8(const Fp8Args&, void*) { return static_cast<int>(hipErrorNotSupported); }
}  // namespace fa
