// la_chunk_f32.hip -- fp32-input instantiations of the chunked linear-attention kernel.
#include "la_launch.h"

namespace drs {
hipError_t la_launch_f32(const LAParams &p, int DK, int DVS, int C, hipStream_t stream, bool dry_run) {
    return la_launch_typed<float>(p, DK, DVS, C, stream, dry_run);
}
}  // namespace drs
