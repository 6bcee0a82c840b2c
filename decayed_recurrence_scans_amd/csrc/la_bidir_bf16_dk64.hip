// la_bidir_bf16_dk64.hip -- bf16 inputs, Dk = 64: instantiations of the fused bidirectional
// linear-attention kernel.
#include "la_fwd_launch.h"

namespace drs {
template hipError_t la_bidir_dk<uint16_t, 64>(const LAGroup &, int, int, hipStream_t, bool);
}  // namespace drs
