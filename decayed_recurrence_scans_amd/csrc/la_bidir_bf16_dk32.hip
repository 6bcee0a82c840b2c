// la_bidir_bf16_dk32.hip -- bf16 inputs, Dk = 32: instantiations of the fused bidirectional
// linear-attention kernel.
#include "la_fwd_launch.h"

namespace drs {
template hipError_t la_bidir_dk<uint16_t, 32>(const LAGroup &, int, int, hipStream_t, bool);
}  // namespace drs
