// api.hip -- the C ABI of libdrs: argument validation, kernel selection, launch.
//
// Every check happens on the host before anything is enqueued, so a non-zero
// return leaves all outputs untouched.  No exception crosses the boundary.
#include <stdint.h>

#include "drs.h"
#include "la_launch.h"
#include "wkv.h"


namespace {

constexpr int kTargetWorkgroups = 256;   // one per compute unit of an MI355X

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int la_default_chunk(drs_dtype dt, int Dk, int DVS) {
    if (dt == DRS_BF16) return (Dk == 128 && DVS == 32) ? 32 : 64;
    if (Dk <= 32) return 64;
    return Dk == 64 ? 32 : 16;
}

bool wkv_scan_chosen(int B, int T, int C, unsigned flags) {
    if (flags & DRS_FORCE_SEQ) return false;
    if (flags & DRS_FORCE_SCAN) return true;
    return drs::wkv_use_scan(B, T, C);
}

}  // namespace

extern "C" {

DRS_API int la_forward(const void *q, const void *k, const void *v, drs_dtype dt, const float *decay,
                       drs_decay mode, const float *state_in, const float *cum_k_in, void *y,
                       float *state_out, float *cum_k_out, int B, int H, int T, int Dk, int Dv, int chunk,
                       unsigned flags, void *stream) {
    if (!q || !k || !v || !y) return DRS_ERR_INVALID;
    if (B < 1 || H < 1 || T < 1) return DRS_ERR_INVALID;
    if (dt != DRS_F32 && dt != DRS_BF16) return DRS_ERR_INVALID;
    if (mode != DRS_DECAY_NONE && mode != DRS_DECAY_HEAD && mode != DRS_DECAY_STEP) return DRS_ERR_INVALID;
    if ((decay == nullptr) != (mode == DRS_DECAY_NONE)) return DRS_ERR_INVALID;
    if (flags & ~(DRS_REVERSE | DRS_NORMALIZE)) return DRS_ERR_INVALID;
    const bool normalize = (flags & DRS_NORMALIZE) != 0;
    if (!normalize && (cum_k_in || cum_k_out)) return DRS_ERR_INVALID;
    if (cum_k_out && cum_k_out == cum_k_in) return DRS_ERR_INVALID;
    if (y == q || y == k || y == v) return DRS_ERR_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y)) return DRS_ERR_INVALID;
    if ((decay && !aligned4(decay)) || (state_in && !aligned4(state_in)) ||
        (state_out && !aligned4(state_out)) || (cum_k_in && !aligned4(cum_k_in)) ||
        (cum_k_out && !aligned4(cum_k_out)))
        return DRS_ERR_INVALID;
    if (!supported_dim(Dk) || !supported_dim(Dv)) return DRS_ERR_UNSUPPORTED;
    if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64) return DRS_ERR_UNSUPPORTED;

    int DVS = 16;
    if (Dk >= 64 && Dv % 32 == 0 && (long)B * H * (Dv / 32) >= kTargetWorkgroups) DVS = 32;
    const int C = chunk ? chunk : la_default_chunk(dt, Dk, DVS);
    const long nwg = (long)B * H * (Dv / DVS);
    if (nwg > 0x7fffffffL) return DRS_ERR_UNSUPPORTED;

    drs::LAParams p;
    p.q = q; p.k = k; p.v = v; p.y = y;
    p.decay = decay;
    p.state_in = state_in; p.cum_k_in = cum_k_in;
    p.state_out = state_out; p.cum_k_out = cum_k_out;
    p.B = B; p.H = H; p.T = T; p.Dv = Dv; p.nslice = Dv / DVS;
    p.mode = (int)mode;
    p.reverse = (flags & DRS_REVERSE) ? 1 : 0;
    p.normalize = normalize ? 1 : 0;
    p.nchunks = (T + C - 1) / C;
    p.ngroups = (p.nchunks + drs::kLAWaves - 1) / drs::kLAWaves;

    hipStream_t s = static_cast<hipStream_t>(stream);
    auto launch = [&](bool dry) {
        return (dt == DRS_BF16) ? drs::la_launch_bf16(p, Dk, DVS, C, s, dry)
                                : drs::la_launch_f32(p, Dk, DVS, C, s, dry);
    };
    if (launch(true) != hipSuccess) return DRS_ERR_UNSUPPORTED;   // no HIP call made yet
    (void)hipGetLastError();
    return launch(false) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
}

DRS_API size_t wkv_workspace_bytes(int B, int T, int C, unsigned flags) {
    if (B < 1 || T < 1 || C < 1) return 0;
    if (!wkv_scan_chosen(B, T, C, flags)) return 0;
    int L, n;
    drs::wkv_scan_plan(B, T, C, &L, &n);
    return (size_t)(n + 1) * 3 * (size_t)B * (size_t)C * sizeof(float);
}

DRS_API int wkv_forward(const float *w, const float *u, const float *k, const float *v, const float *state_in,
                        float *y, float *state_out, int B, int T, int C, unsigned flags, void *workspace,
                        size_t workspace_bytes, void *stream) {
    if (!w || !u || !k || !v || !y) return DRS_ERR_INVALID;
    if (B < 1 || T < 1 || C < 1) return DRS_ERR_INVALID;
    if (flags & ~(DRS_FORCE_SEQ | DRS_FORCE_SCAN)) return DRS_ERR_INVALID;
    if ((flags & DRS_FORCE_SEQ) && (flags & DRS_FORCE_SCAN)) return DRS_ERR_INVALID;
    if (y == k || y == v) return DRS_ERR_INVALID;
    const void *ptrs[] = {w, u, k, v, y, state_in, state_out, workspace};
    for (const void *pp : ptrs)
        if (pp && !aligned4(pp)) return DRS_ERR_INVALID;
    if (B > 65535) return DRS_ERR_UNSUPPORTED;

    drs::WKVParams p;
    p.w = w; p.u = u; p.k = k; p.v = v; p.state_in = state_in;
    p.y = y; p.state_out = state_out;
    p.ws = static_cast<float *>(workspace);
    p.B = B; p.T = T; p.C = C;
    p.seg_len = T; p.nseg = 1;

    const bool scan = wkv_scan_chosen(B, T, C, flags);
    if (scan) {
        drs::wkv_scan_plan(B, T, C, &p.seg_len, &p.nseg);
        if (p.nseg > 65535) return DRS_ERR_UNSUPPORTED;
        const size_t need = (size_t)(p.nseg + 1) * 3 * (size_t)B * (size_t)C * sizeof(float);
        if (!workspace || workspace_bytes < need) return DRS_ERR_WORKSPACE;
    }
    (void)hipGetLastError();
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = scan ? drs::wkv_launch_scan(p, s) : drs::wkv_launch_seq(p, s);
    return e == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
}

DRS_API const char *drs_status_string(int status) {
    switch (status) {
        case DRS_OK: return "ok";
        case DRS_ERR_INVALID: return "invalid argument";
        case DRS_ERR_UNSUPPORTED: return "unsupported size or option";
        case DRS_ERR_WORKSPACE: return "workspace missing or too small";
        case DRS_ERR_DEVICE: return "HIP launch failed";
        default: return "unknown status";
    }
}

DRS_API int drs_version(void) { return 100; }

}  // extern "C"
