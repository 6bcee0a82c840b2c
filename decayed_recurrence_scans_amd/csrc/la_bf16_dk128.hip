// la_bf16_dk128.hip -- bf16 inputs, Dk = 128: instantiations of the linear-attention kernel.
#include "la_fwd_launch.h"

namespace drs {
template hipError_t la_launch_dk<uint16_t, 128>(const LAGroup &, int, int, hipStream_t, bool);
}  // namespace drs
