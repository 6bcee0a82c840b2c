// la_fwd_launch.h -- host launchers of the linear-attention kernel.
#pragma once

#include "la_fwd_impl.h"

namespace drs {

constexpr int kLdsBytes = 160 * 1024;   // LDS per compute unit on gfx950

// With dry_run the call only reports whether the variant exists (no HIP call).
template <typename TI, int DK, int DV, int C, bool ONEPASS>
hipError_t la_launch_one(const LAParams &p, hipStream_t stream, bool dry_run) {
    if constexpr (FwdLayout<TI, DK, DV, C, ONEPASS ? kOnePassChunks : 1>::LDS_B > kLdsBytes) {
        (void)p; (void)stream; (void)dry_run;
        return hipErrorNotSupported;
    } else {
        if (dry_run) return hipSuccess;
        const dim3 grid((unsigned)p.nbh * (unsigned)p.nseg), block(4 * DV);
        const bool norm = p.normalize != 0;
        switch (p.mode * 2 + (norm ? 1 : 0)) {
#define DRS_LA_CASE(N, MODE, NORM) \
            case N: hipLaunchKernelGGL((la_fwd_kernel<TI, DK, DV, C, MODE, NORM, ONEPASS>), grid, block, 0, stream, p); break;
            DRS_LA_CASE(0, 0, false)
            DRS_LA_CASE(1, 0, true)
            DRS_LA_CASE(2, 1, false)
            DRS_LA_CASE(3, 1, true)
            DRS_LA_CASE(4, 2, false)
            DRS_LA_CASE(5, 2, true)
#undef DRS_LA_CASE
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
}

// Single pass where the plan asked for it (segments of at most kOnePassChunks chunks;
// head dimensions up to 64, where the kept outputs fit in registers).
template <typename TI, int DK, int DV, int C>
hipError_t la_launch_variant(const LAParams &p, hipStream_t stream, bool dry_run) {
    if (p.onepass) {
        if constexpr (DK <= 64 && DV <= 64) return la_launch_one<TI, DK, DV, C, true>(p, stream, dry_run);
        else return hipErrorNotSupported;
    }
    return la_launch_one<TI, DK, DV, C, false>(p, stream, dry_run);
}

template <typename TI, int DK, int DV>
hipError_t la_launch_c(const LAParams &p, int C, hipStream_t stream, bool dry_run) {
    switch (C) {
        case 16: return la_launch_variant<TI, DK, DV, 16>(p, stream, dry_run);
        case 32: return la_launch_variant<TI, DK, DV, 32>(p, stream, dry_run);
        case 64: return la_launch_variant<TI, DK, DV, 64>(p, stream, dry_run);
        default: return hipErrorNotSupported;
    }
}

// One translation unit per (input type, Dk) instantiates this.
template <typename TI, int DK>
hipError_t la_launch_dk(const LAParams &p, int DV, int C, hipStream_t stream, bool dry_run) {
    switch (DV) {
        case 16: return la_launch_c<TI, DK, 16>(p, C, stream, dry_run);
        case 32: return la_launch_c<TI, DK, 32>(p, C, stream, dry_run);
        case 64: return la_launch_c<TI, DK, 64>(p, C, stream, dry_run);
        case 128: return la_launch_c<TI, DK, 128>(p, C, stream, dry_run);
        default: return hipErrorNotSupported;
    }
}

#define DRS_LA_EXTERN(TI, DK) \
    extern template hipError_t la_launch_dk<TI, DK>(const LAParams &, int, int, hipStream_t, bool);
DRS_LA_EXTERN(uint16_t, 16)
DRS_LA_EXTERN(uint16_t, 32)
DRS_LA_EXTERN(uint16_t, 64)
DRS_LA_EXTERN(uint16_t, 128)
DRS_LA_EXTERN(float, 16)
DRS_LA_EXTERN(float, 32)
DRS_LA_EXTERN(float, 64)
DRS_LA_EXTERN(float, 128)
#undef DRS_LA_EXTERN

}  // namespace drs
