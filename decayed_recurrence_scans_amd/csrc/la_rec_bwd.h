// la_rec_bwd.h -- backward of linear attention one step at a time (the state and
// its gradient held in registers): every decay mode, with or without the
// normaliser.  la_backward takes it for the normalised form and for one factor
// per key channel, where the chunked gradient scans do not apply.
#pragma once

#include <hip/hip_runtime.h>

namespace drs {

struct LARecBwdParams {
    const void *q, *k, *v, *dy;     // [B,H,T,Dk|Dv] in the call's type
    const float *decay;             // NULL | [H] | [B,H,T] | [B,H,T,Dk] by mode
    const float *state_in, *cum_k_in;       // the forward's initial state and key sum (NULL: zero)
    const float *dstate_out, *dcum_k_out;   // gradients reaching the final ones (NULL: zero)
    void *dq, *dk, *dv;             // outputs in the call's type
    float *ddecay;                  // NULL, or the factor gradient: [B,H,T] (step), [B,H,T,Dk] (elem);
                                    // mode head writes per-unit sums to `hpart` instead
    float *dstate_in, *dcum_k_in;   // NULL or [B,H,Dk,Dv], [B,H,Dk]
    // workspace (fp64: the sweeps compute in fp64)
    double *dq64;                   // [B,H,T,Dk] dq before rounding (with ddecay)
    double *a64;                    // [B,H,T,Dv] dL/d(numerator) = dy / den (normalised)
    double *c64;                    // [B,H,T]    dL/d(denominator) (normalised)
    double *sfin, *zfin;            // [B,H,Dk,Dv], [B,H,Dk] the recomputed final state / key sum
    float *hpart;                   // [B,H] per-unit sums of the per-head factor gradient
    int B, H, T, Dk, Dv;
    int mode;                       // 0 none, 1 head, 2 step, 3 per key channel
    int reverse, normalize;
    int tb;                         // time steps staged in LDS at once
};

// Bytes of workspace the two kernels need for these sizes and outputs.
size_t la_rec_bwd_ws_bytes(int B, int H, int T, int Dk, int Dv, bool normalize, bool ddecay, bool final_terms);

// The forward sweep (dq, and the numerator / denominator gradients), then the
// reverse sweep (dk, dv, the factor gradient, the initial-state gradients);
// with a per-head factor also the sum over the batch.
hipError_t la_rec_bwd_launch(const LARecBwdParams &p, bool bf16, hipStream_t stream);

}  // namespace drs
