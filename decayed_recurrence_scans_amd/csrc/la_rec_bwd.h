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
    // time segments (nseg > 1): each sweep runs its segments in parallel from entering
    // states folded out of per-segment summaries
    double *aggF;                   // [B,H,nseg] forward summaries: S (Dk x Dv), z (Dk), factor product (Dk)
    double *aggR;                   // [B,H,nseg] reverse summaries: G (Dk x Dv), Gz (Dk)
    double *rloc;                   // factor gradient: [B,H,T,Dk] (per key channel) | [B,H,T]: suffix sums
                                    // inside each segment (visiting order), before the later segments' totals
    double *eseg;                   // [B,H,nseg,Dk] the segments' totals of those sums
    int nseg, seg_len;
    int B, H, T, Dk, Dv;
    int mode;                       // 0 none, 1 head, 2 step, 3 per key channel
    int reverse, normalize;
    int tb;                         // time steps staged in LDS at once
};

// Time segments of the sweeps for these sizes (about one workgroup per compute unit).
int la_rec_bwd_nseg(int B, int H, int T);

// Bytes of workspace the kernels need for these sizes and outputs (mode 3, per key
// channel, needs the most).
size_t la_rec_bwd_ws_bytes(int B, int H, int T, int Dk, int Dv, int mode, bool normalize, bool ddecay,
                           bool final_terms);

// Sets the workspace pointers, nseg and seg_len of p (sizes, mode, normalize and the
// ddecay output already set) in a workspace of la_rec_bwd_ws_bytes bytes.
void la_rec_bwd_layout(char *ws, LARecBwdParams &p, bool final_terms);

// The forward summaries and sweep (dq, and the numerator / denominator gradients),
// then the reverse summaries and sweep (dk, dv, the factor gradient, the initial-state
// gradients); with segments the factor gradient's completion, with a per-head factor
// also the sum over the batch.
hipError_t la_rec_bwd_launch(const LARecBwdParams &p, bool bf16, hipStream_t stream);

}  // namespace drs
