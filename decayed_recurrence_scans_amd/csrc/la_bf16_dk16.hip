// la_bf16_dk16.hip -- bf16 inputs, Dk = 16: instantiations of the linear-attention kernel.
#include "la_fwd_launch.h"

namespace drs {
template hipError_t la_launch_dk<uint16_t, 16>(const LAParams &, int, int, hipStream_t, bool);
}  // namespace drs
