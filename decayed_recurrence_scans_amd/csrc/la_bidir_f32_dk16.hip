// la_bidir_f32_dk16.hip -- fp32 inputs, Dk = 16: instantiations of the fused bidirectional
// linear-attention kernel.
#include "la_fwd_launch.h"

namespace drs {
template hipError_t la_bidir_dk<float, 16>(const LAGroup &, int, int, hipStream_t, bool);
}  // namespace drs
