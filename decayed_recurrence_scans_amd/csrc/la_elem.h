// la_elem.h -- chunked linear attention with one decay factor per key channel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace drs {

constexpr int kElemChunk = 16;           // rows per chunk
constexpr int kElemTargetGroups = 512;   // two workgroups per compute unit: one round
constexpr float kElemLog2Floor = -15.f;  // per-step log2 factor floor (see la_elem.hip)

struct LAElemParams {
    const uint16_t *q, *k, *v;     // bf16 [B,H,T,Dk|Dv]
    uint16_t *y;
    const float *decay;            // [B,H,T,Dk]
    const float *state_in;         // [B,H,Dk,Dv] or NULL
    float *state_out;              // or NULL
    float *ws;                     // per unit: initial state [Dk*Dv], then [nseg][Dk*Dv + Dk]
    int B, H, T;
    int nchunks, nseg, L;          // chunks, segments, chunks per segment
    int reverse;
};

// Segments for these sizes; false when the kernels do not cover them.
bool la_elem_plan(int B, int H, int T, int Dk, int Dv, int *nseg, int *L);
size_t la_elem_ws_bytes(int B, int H, int T, int Dk, int Dv);   // 0 when unsupported
hipError_t la_elem_launch(const LAElemParams &p, int Dk, int Dv, hipStream_t stream);

}  // namespace drs
