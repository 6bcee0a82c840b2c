// wkv.h -- host interface of the WKV kernels (wkv.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace drs {

struct WKVParams {
    const float *w, *u, *k, *v, *state_in;
    float *y, *state_out;
    float *ws;          // time-parallel path only: [nseg + 1][3][B][C] fp32
    int B, T, C;
    int seg_len, nseg;
};

void wkv_scan_plan(int B, int T, int C, int *seg_len, int *nseg);
bool wkv_use_scan(int B, int T, int C);
hipError_t wkv_launch_seq(const WKVParams &p, hipStream_t stream);
hipError_t wkv_launch_scan(const WKVParams &p, hipStream_t stream);

}  // namespace drs
