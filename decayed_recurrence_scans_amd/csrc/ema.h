// ema.h -- host interface of the gated element-wise EMA kernels (ema.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace drs {

struct EmaParams {
    const void *x, *f;              // [B,T,C] values and factors (fp32 or bf16)
    void *y;                        // [B,T,C] outputs, the dtype of x
    const float *state_in;          // [B,C] or NULL (zero)
    float *state_out;               // [B,C] or NULL
    int B, T, C;
    int reverse;
    int ncblk, nblk;                // 64-channel blocks per batch row; time blocks
    int walk;                       // one workgroup walks all time blocks (no look-back)
    unsigned *ws_ctr;               // look-back counters (first 256 bytes of the workspace)
    unsigned long long *ws_flags;   // [units * nblk]
    float *ws_agg;                  // [units * nblk][64][2] block aggregates (scan, factor product)
    unsigned spin_limit;
};

constexpr int kEmaSub = 32;                    // steps per wave, kept in registers
constexpr int kEmaWaves = 4;                   // waves per workgroup
constexpr int kEmaBlock = kEmaSub * kEmaWaves; // steps per time block
constexpr long kEmaWalkUnits = 512;            // 64-channel units that fill the GPU (two per CU)
constexpr long kEmaMaxLookbackBlocks = 64;     // fold cost grows with the block count
constexpr long kEmaOneRound = 512;             // workgroups resident at once (two per CU)
constexpr size_t kEmaCtrBytes = 256;

bool ema_supported(int B, int T, int C, int esize);
bool ema_walk(int B, int T, int C);
size_t ema_ws_bytes(int B, int T, int C);
hipError_t ema_launch(const EmaParams &p, bool bf16, hipStream_t s);

// Fused bidirectional EMA (walk layout; uses x, f, y, B, T, C, ncblk, nblk and
// ws_agg = the workspace after its first kEmaCtrBytes).
size_t ema_bidir_ws_bytes(int B, int T, int C);
hipError_t ema_bidir_launch(const EmaParams &p, bool bf16, hipStream_t s);

}  // namespace drs
