// wkv.h -- host interface of the WKV kernels (wkv.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace drs {

struct WKVParams {
    const float *w, *u, *k, *v, *state_in;
    float *y, *state_out;
    float *ws;          // two-pass scan: [nseg + 1][3][B][C] fp32 (after the counters)
    int B, T, C;
    int seg_len, nseg;
    // chained single pass
    unsigned *ws_ctr;               // look-back counters (first 256 bytes of the workspace)
    unsigned long long *ws_flags;   // [units * nblk]
    float *ws_agg;                  // [units * nblk][4][64] block aggregates (aa, bb, pp, -)
    int ncblk, nblk;                // 64-channel blocks per batch row; time blocks
    int walk;                       // one workgroup walks all time blocks (no look-back)
    int ticket;                     // virtual ids from the atomic ticket (else the workgroup id)
    int own_aggs;                   // compute every earlier block's aggregate instead of waiting
    unsigned spin_limit;
};

// Chained single pass: a workgroup of kWkvChainWaves waves owns 64 channels of
// one batch row over one time block of kWkvChainWaves * kWkvChainSub steps.
constexpr int kWkvChainSub = 64;
constexpr int kWkvChainWaves = 4;
constexpr int kWkvChainBlock = kWkvChainSub * kWkvChainWaves;
constexpr int kWkvChainMaxBlocks = 64;    // fold cost grows with the block count
// Walk mode once there are this many 64-channel units: with two workgroups per
// compute unit the chip is full without splitting the time axis.
constexpr long kWkvWalkUnits = 512;
// Walk mode: waves per workgroup and steps per wave per time block.
constexpr int kWkvWalkWaves = 8;
constexpr int kWkvWalkSub = 16;

// Workspace layout shared by the WKV paths: 256 bytes of look-back counters first.
constexpr size_t kWkvCtrBytes = 256;
size_t wkv_chain_ws_bytes(int B, int T, int C);
bool wkv_chain_supported(int B, int T, int C);
hipError_t wkv_launch_chain(const WKVParams &p, hipStream_t stream);

// Row-owning sweep (forced only): workgroups of 256 W channels (4 per lane) times
// spans of S steps; ncblk = channel groups, nblk = spans.
void wkv_rows_plan(int B, int T, int C, int *ngroups, int *nspan);
bool wkv_rows_supported(int B, int T, int C);
size_t wkv_rows_ws_bytes(int B, int T, int C);
// Plan and workspace pointers of a rows call (p.B, p.T, p.C set) in a workspace of that size.
void wkv_rows_layout(char *ws, WKVParams &p);
hipError_t wkv_launch_rows(const WKVParams &p, hipStream_t stream);

void wkv_scan_plan(int B, int T, int C, int *seg_len, int *nseg);
bool wkv_use_scan(int B, int T, int C);
hipError_t wkv_launch_seq(const WKVParams &p, hipStream_t stream);
hipError_t wkv_launch_scan(const WKVParams &p, hipStream_t stream);

}  // namespace drs

namespace drs {

// Backward of WKV (wkv_bwd.hip): a forward sweep stores the state entering every
// 64-step block; a reverse walk over the blocks rebuilds the outputs and runs the
// gradient sums backward, both time-parallel within a block.  With few channel
// groups the blocks run in parallel instead, joined by per-channel scans of their
// summaries.
struct WKVBwdParams {
    const float *w, *u, *k, *v, *state_in, *dy;
    float *dk, *dv;
    float *dw, *du;                 // [C] or NULL
    float *dstate_in;               // [3][B][C] or NULL: gradient of the carried state (aa, bb, pp)
    double *ckpt;                   // workspace [B][blocks][6][C]: state entering each 64-step block
    double *bsum;                   // split mode: [B][blocks][6][C] block summaries (forward, then reverse)
    double *rcar;                   // split mode: [B][blocks][4][C] reverse sums entering each block
    float *part;                    // workspace [2][B][parts][C]: partial sums of the u and w gradients
    int B, T, C;
    int split;                      // 0: walks; 1, 2: split-mode passes (internal)
    int nseg, per;                  // split mode: segments of `per` blocks per channel group
};
// Split mode (time-parallel over blocks) for few channel groups.
bool wkv_bwd_split(int B, int T, int C);
size_t wkv_bwd_ws_bytes(int B, int T, int C);
// Pointers into a workspace of wkv_bwd_ws_bytes (the first 256 bytes are left alone).
void wkv_bwd_layout(int B, int T, int C, char *ws, WKVBwdParams &p);
hipError_t wkv_launch_bwd(const WKVBwdParams &p, hipStream_t stream);

}  // namespace drs
