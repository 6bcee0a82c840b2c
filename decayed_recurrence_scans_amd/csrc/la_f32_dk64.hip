// la_f32_dk64.hip -- f32 inputs, Dk = 64: instantiations of the linear-attention kernel.
#include "la_fwd_launch.h"

namespace drs {
template hipError_t la_launch_dk<float, 64>(const LAGroup &, int, int, hipStream_t, bool);
}  // namespace drs
