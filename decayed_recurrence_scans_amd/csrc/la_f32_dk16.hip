// la_f32_dk16.hip -- f32 inputs, Dk = 16: instantiations of the linear-attention kernel.
#include "la_fwd_launch.h"

namespace drs {
template hipError_t la_launch_dk<float, 16>(const LAParams &, int, int, hipStream_t, bool);
}  // namespace drs
