// la_f32_dk128.hip -- f32 inputs, Dk = 128: instantiations of the linear-attention kernel.
#include "la_fwd_launch.h"

namespace drs {
template hipError_t la_launch_dk<float, 128>(const LAParams &, int, int, hipStream_t, bool);
}  // namespace drs
