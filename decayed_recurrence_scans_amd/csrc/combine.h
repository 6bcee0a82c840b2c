// combine.h -- elementwise sum of two outputs (the bidirectional forms).
#pragma once

#include <hip/hip_runtime.h>

namespace drs {

// y[i] <- y[i] + x[i] for i < n, summed in fp32 and rounded once to the storage
// type (bf16: to nearest even).  vec: both pointers 16-byte aligned.
hipError_t add_into_launch(void *y, const void *x, size_t n, bool bf16, bool vec, hipStream_t stream);

}  // namespace drs
