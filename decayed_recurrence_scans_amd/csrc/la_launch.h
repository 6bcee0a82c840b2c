// la_launch.h -- host launchers of the chunked linear-attention kernel.
#pragma once

#include "la_chunk_impl.h"

namespace drs {

constexpr int kLAWaves = 4;

constexpr int kLdsBytes = 160 * 1024;   // LDS per compute unit on gfx950

// Variants whose LDS image does not fit (fp32, Dk = 128, chunk 64) report
// hipErrorNotSupported; the C ABI turns that into DRS_ERR_UNSUPPORTED.
// With dry_run the call only reports whether the variant exists.
template <typename TI, int DK, int DVS, int C>
hipError_t la_launch_one(const LAParams &p, hipStream_t stream, bool dry_run) {
    if constexpr (LALayout<TI, DK, DVS, C, kLAWaves>::TOTAL_B > kLdsBytes) {
        (void)p; (void)stream; (void)dry_run;
        return hipErrorNotSupported;
    } else {
        if (dry_run) return hipSuccess;
        dim3 grid(p.B * p.H * p.nslice);
        hipLaunchKernelGGL((la_chunk_fwd<TI, DK, DVS, C, kLAWaves>), grid, dim3(64 * kLAWaves), 0, stream, p);
        return hipGetLastError();
    }
}

template <typename TI, int DK, int DVS>
hipError_t la_launch_c(const LAParams &p, int C, hipStream_t stream, bool dry_run) {
    switch (C) {
        case 16: return la_launch_one<TI, DK, DVS, 16>(p, stream, dry_run);
        case 32: return la_launch_one<TI, DK, DVS, 32>(p, stream, dry_run);
        case 64: return la_launch_one<TI, DK, DVS, 64>(p, stream, dry_run);
        default: return hipErrorNotSupported;
    }
}

// Kernel variants compiled per input type: every Dk in {16,32,64,128} with a
// 16-wide Dv slice, and a 32-wide slice for Dk >= 64.
template <typename TI>
hipError_t la_launch_typed(const LAParams &p, int DK, int DVS, int C, hipStream_t stream, bool dry_run) {
    if (DVS == 16) {
        switch (DK) {
            case 16: return la_launch_c<TI, 16, 16>(p, C, stream, dry_run);
            case 32: return la_launch_c<TI, 32, 16>(p, C, stream, dry_run);
            case 64: return la_launch_c<TI, 64, 16>(p, C, stream, dry_run);
            case 128: return la_launch_c<TI, 128, 16>(p, C, stream, dry_run);
        }
    } else if (DVS == 32) {
        switch (DK) {
            case 64: return la_launch_c<TI, 64, 32>(p, C, stream, dry_run);
            case 128: return la_launch_c<TI, 128, 32>(p, C, stream, dry_run);
        }
    }
    return hipErrorNotSupported;
}

hipError_t la_launch_bf16(const LAParams &p, int DK, int DVS, int C, hipStream_t stream, bool dry_run);
hipError_t la_launch_f32(const LAParams &p, int DK, int DVS, int C, hipStream_t stream, bool dry_run);

}  // namespace drs
