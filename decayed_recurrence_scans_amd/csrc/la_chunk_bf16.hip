// la_chunk_bf16.hip -- bf16-input instantiations of the chunked linear-attention kernel.
#include "la_launch.h"

namespace drs {
hipError_t la_launch_bf16(const LAParams &p, int DK, int DVS, int C, hipStream_t stream, bool dry_run) {
    return la_launch_typed<uint16_t>(p, DK, DVS, C, stream, dry_run);
}
}  // namespace drs
