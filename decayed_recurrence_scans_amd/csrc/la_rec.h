// la_rec.h -- recurrent (step-by-step) linear-attention kernel: decode steps,
// short sequences and the per-key-channel decay mode.
#pragma once

#include <hip/hip_runtime.h>

namespace drs {

// la_forward takes this path by default for T up to this length (a decode step
// is T = 1); the chunked kernels take longer sequences.
constexpr int kLaRecMaxT = 16;

struct LARecParams {
    const void *q, *k, *v;
    void *y;
    const float *decay;             // NULL | [H] | [B,H,T] | [B,H,T,Dk] by mode
    const float *state_in, *cum_k_in;
    float *state_out, *cum_k_out;
    int B, H, T, Dk, Dv;
    int mode;                       // 0 none, 1 head, 2 step, 3 per key channel
    int reverse, normalize;
    int vec_state;                  // state pointers are 16-byte aligned
    int tb;                         // time steps staged in LDS at once
    int y_f32;                      // bf16 inputs, y stored as fp32 (internal: gradient scans)
};

// Threads per workgroup and LDS bytes of one launch.
int la_rec_threads(int Dk, int Dv);
size_t la_rec_lds_bytes(const LARecParams &p);

hipError_t la_rec_launch(const LARecParams &p, bool bf16, hipStream_t stream);

}  // namespace drs
