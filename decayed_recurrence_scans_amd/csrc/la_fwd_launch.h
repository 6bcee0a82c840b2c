// la_fwd_launch.h -- host launchers of the linear-attention kernel.
#pragma once

#include "la_fwd_impl.h"

namespace drs {

constexpr int kLdsBytes = 160 * 1024;   // LDS per compute unit on gfx950

// With dry_run the call only reports whether the variant exists (no HIP call).
template <typename TI, int DK, int DV, int C, bool ONEPASS>
hipError_t la_launch_one(const LAGroup &g, hipStream_t stream, bool dry_run) {
    if constexpr (FwdLayout<TI, DK, DV, C, ONEPASS ? kOnePassChunks : 1>::LDS_B > kLdsBytes) {
        (void)g; (void)stream; (void)dry_run;
        return hipErrorNotSupported;
    } else {
        if (dry_run) return hipSuccess;
        const LAParams &p = g.p[0];
        const dim3 grid(g.per_grid * (unsigned)g.count), block(4 * DV);
        const bool norm = p.normalize != 0;
        switch (p.mode * 2 + (norm ? 1 : 0)) {
#define DRS_LA_CASE(N, MODE, NORM) \
            case N: hipLaunchKernelGGL((la_fwd_kernel<TI, DK, DV, C, MODE, NORM, ONEPASS>), grid, block, 0, stream, g); break;
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
hipError_t la_launch_variant(const LAGroup &g, hipStream_t stream, bool dry_run) {
    if (g.p[0].onepass) {
        if constexpr (DK <= 64 && DV <= 64) return la_launch_one<TI, DK, DV, C, true>(g, stream, dry_run);
        else return hipErrorNotSupported;
    }
    return la_launch_one<TI, DK, DV, C, false>(g, stream, dry_run);
}

template <typename TI, int DK, int DV>
hipError_t la_launch_c(const LAGroup &g, int C, hipStream_t stream, bool dry_run) {
    switch (C) {
        case 16: return la_launch_variant<TI, DK, DV, 16>(g, stream, dry_run);
        case 32: return la_launch_variant<TI, DK, DV, 32>(g, stream, dry_run);
        case 64: return la_launch_variant<TI, DK, DV, 64>(g, stream, dry_run);
        default: return hipErrorNotSupported;
    }
}

// One translation unit per (input type, Dk) instantiates this.  Every problem of the
// group has the same shape, decay mode, normaliser and plan (the template arguments).
template <typename TI, int DK>
hipError_t la_launch_dk(const LAGroup &g, int DV, int C, hipStream_t stream, bool dry_run) {
    switch (DV) {
        case 16: return la_launch_c<TI, DK, 16>(g, C, stream, dry_run);
        case 32: return la_launch_c<TI, DK, 32>(g, C, stream, dry_run);
        case 64: return la_launch_c<TI, DK, 64>(g, C, stream, dry_run);
        case 128: return la_launch_c<TI, DK, 128>(g, C, stream, dry_run);
        default: return hipErrorNotSupported;
    }
}

// The fused bidirectional kernel: one chunk size per (input type, Dk), the default
// one of the chunked path (bf16: 64; fp32: 64 up to Dk = 32, else 32).
template <typename TI, int DK>
constexpr int la_bidir_chunk() { return (sizeof(TI) == 2 || DK <= 32) ? 64 : 32; }

template <typename TI, int DK, int DV, int C>
hipError_t la_launch_bidir(const LAGroup &g, hipStream_t stream, bool dry_run) {
    if constexpr (FwdLayout<TI, DK, DV, C, kBidirChunks>::LDS_B > kLdsBytes) {
        (void)g; (void)stream; (void)dry_run;
        return hipErrorNotSupported;
    } else {
        if (dry_run) return hipSuccess;
        const dim3 grid(g.per_grid * (unsigned)g.count), block(4 * DV);
        switch (g.p[0].mode) {
            case 0: hipLaunchKernelGGL((la_fwd_kernel<TI, DK, DV, C, 0, false, true, true>), grid, block, 0, stream, g); break;
            case 1: hipLaunchKernelGGL((la_fwd_kernel<TI, DK, DV, C, 1, false, true, true>), grid, block, 0, stream, g); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
}

// Dk, Dv up to 64 (the kept outputs live in registers), C the type's chunk size.
template <typename TI, int DK>
hipError_t la_bidir_dk(const LAGroup &g, int DV, int C, hipStream_t stream, bool dry_run) {
    constexpr int CB = la_bidir_chunk<TI, DK>();
    if (C != CB) return hipErrorNotSupported;
    switch (DV) {
        case 16: return la_launch_bidir<TI, DK, 16, CB>(g, stream, dry_run);
        case 32: return la_launch_bidir<TI, DK, 32, CB>(g, stream, dry_run);
        case 64: return la_launch_bidir<TI, DK, 64, CB>(g, stream, dry_run);
        default: return hipErrorNotSupported;
    }
}

#define DRS_LA_BIDIR_EXTERN(TI, DK) \
    extern template hipError_t la_bidir_dk<TI, DK>(const LAGroup &, int, int, hipStream_t, bool);
DRS_LA_BIDIR_EXTERN(uint16_t, 16)
DRS_LA_BIDIR_EXTERN(uint16_t, 32)
DRS_LA_BIDIR_EXTERN(uint16_t, 64)
DRS_LA_BIDIR_EXTERN(float, 16)
DRS_LA_BIDIR_EXTERN(float, 32)
DRS_LA_BIDIR_EXTERN(float, 64)
#undef DRS_LA_BIDIR_EXTERN

#define DRS_LA_EXTERN(TI, DK) \
    extern template hipError_t la_launch_dk<TI, DK>(const LAGroup &, int, int, hipStream_t, bool);
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
