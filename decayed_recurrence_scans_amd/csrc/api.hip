// api.hip -- the C ABI of libdrs: argument validation, kernel selection, launch.
//
// Every check happens on the host before anything is enqueued, so a non-zero
// return leaves all outputs untouched.  No exception crosses the boundary.
#include <stdint.h>

#include <mutex>

#include "combine.h"
#include "drs.h"
#include "ema.h"
#include "la_bwd.h"
#include "la_elem.h"
#include "la_fwd_launch.h"
#include "la_rec.h"
#include "la_rec_bwd.h"
#include "wkv.h"

// The scratch of la_forward_noalloc: one copy per GPU, held until the process
// ends.  In host code this name is only a stand-in for the symbol: the device
// address of a GPU's copy comes from hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) unsigned char scratch[DRS_NOALLOC_SCRATCH_BYTES];

namespace {

// Waves a chunked linear-attention launch aims for (segments per (b, h) follow from it).
#ifndef DRS_LA_TARGET_WAVES
#define DRS_LA_TARGET_WAVES 2048           // eight per compute unit of an MI355X
#endif
constexpr int kTargetWaves = DRS_LA_TARGET_WAVES;
constexpr unsigned kSpinLimit = 1u << 20; // look-back polls before giving up (~50 ms)

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// How one la_forward call is cut into workgroups, and the workspace it needs.
struct LAPlan {
    int C, nchunks, nbh, nseg, L;
    size_t slot_floats, off_flags, off_agg, ws_bytes;
};

int la_default_chunk(int dt, int Dk) {
    if (dt == DRS_BF16) return 64;
    if (Dk <= 32) return 64;
    return Dk == 64 ? 32 : 16;
}

// Returns false for sizes the kernels do not cover.
bool la_make_plan(int dt, int B, int H, int T, int Dk, int Dv, int chunk, LAPlan *pl) {
    if (!supported_dim(Dk) || !supported_dim(Dv)) return false;
    if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64) return false;
    pl->C = chunk ? chunk : la_default_chunk(dt, Dk);
    const long nbh = (long)B * H;
    const long nw = Dv / 16;                       // waves per workgroup
    pl->nchunks = (int)((T + (long)pl->C - 1) / pl->C);
    long nseg = (kTargetWaves / nw + nbh - 1) / nbh;
    if (nseg > pl->nchunks) nseg = pl->nchunks;
    if (nseg < 1) nseg = 1;
    const long L = (pl->nchunks + nseg - 1) / nseg;
    nseg = (pl->nchunks + L - 1) / L;
    if (nbh * nseg > 0x7fffffffL) return false;
    pl->nbh = (int)nbh;
    pl->nseg = (int)nseg;
    pl->L = (int)L;
    const int KB = dt == DRS_BF16 ? 32 : 16;
    const int DKP = Dk < KB ? KB : Dk;
    pl->slot_floats = (size_t)16 * DKP + DKP + 4;
    const size_t nslots = (size_t)nbh * nw * nseg;
    pl->off_flags = 256;
    pl->off_agg = pl->off_flags + round256(nslots * 8 * drs::kFlagStride);
    pl->ws_bytes = pl->off_agg + round256(nslots * pl->slot_floats * 4);
    return true;
}

enum class WkvPath { kSeq, kScan, kChain, kRows };

// Path for these sizes and flags; the FORCE flags pin it (a forced chain may be
// unsupported for the sizes: checked by the caller).  The chained kernel when
// its workgroups walk the sequence (enough channel groups) or all fit in one
// resident round (two per CU); beyond one round each wave of workgroups starts
// cold and waits on the previous one, and the two-pass scan measured faster
// (e.g. 113 vs 191 us at B=2, T=4096, C=4096; 57 vs 85 us at 16 x 1024 x 1024).
constexpr long kWkvChainOneRound = 512;
WkvPath wkv_choose(int B, int T, int C, unsigned flags) {
    if (flags & DRS_FORCE_SEQ) return WkvPath::kSeq;
    if (flags & DRS_FORCE_SCAN) return WkvPath::kScan;
    if (flags & DRS_FORCE_CHAIN) return WkvPath::kChain;
    if (flags & DRS_FORCE_ROWS) return WkvPath::kRows;
    if (drs::wkv_chain_supported(B, T, C) && T > drs::kWkvChainSub) {
        const long units = (long)B * (((long)C + 63) / 64), nblk = ((long)T + drs::kWkvChainBlock - 1) / drs::kWkvChainBlock;
        if (units >= drs::kWkvWalkUnits || units * nblk <= kWkvChainOneRound) return WkvPath::kChain;
    }
    return drs::wkv_use_scan(B, T, C) ? WkvPath::kScan : WkvPath::kSeq;
}

size_t wkv_ws_bytes(int B, int T, int C, WkvPath path) {
    if (path == WkvPath::kChain) return drs::wkv_chain_ws_bytes(B, T, C);
    if (path == WkvPath::kRows) return drs::wkv_rows_ws_bytes(B, T, C);
    if (path == WkvPath::kScan) {
        int L, n;
        drs::wkv_scan_plan(B, T, C, &L, &n);
        return drs::kWkvCtrBytes + (size_t)(n + 1) * 3 * (size_t)B * (size_t)C * sizeof(float);
    }
    return 0;
}

constexpr unsigned kWkvForce = DRS_FORCE_SEQ | DRS_FORCE_SCAN | DRS_FORCE_CHAIN | DRS_FORCE_ROWS;

hipError_t la_launch(int dt, const drs::LAGroup &p, int Dk, int Dv, int C, hipStream_t s, bool dry) {
    if (dt == DRS_BF16) {
        switch (Dk) {
            case 16: return drs::la_launch_dk<uint16_t, 16>(p, Dv, C, s, dry);
            case 32: return drs::la_launch_dk<uint16_t, 32>(p, Dv, C, s, dry);
            case 64: return drs::la_launch_dk<uint16_t, 64>(p, Dv, C, s, dry);
            case 128: return drs::la_launch_dk<uint16_t, 128>(p, Dv, C, s, dry);
        }
    } else {
        switch (Dk) {
            case 16: return drs::la_launch_dk<float, 16>(p, Dv, C, s, dry);
            case 32: return drs::la_launch_dk<float, 32>(p, Dv, C, s, dry);
            case 64: return drs::la_launch_dk<float, 64>(p, Dv, C, s, dry);
            case 128: return drs::la_launch_dk<float, 128>(p, Dv, C, s, dry);
        }
    }
    return hipErrorNotSupported;
}

hipError_t la_launch(int dt, const drs::LAParams &p, int Dk, int Dv, int C, hipStream_t s, bool dry) {
    drs::LAGroup g;
    g.p[0] = p;
    g.per_grid = (unsigned)p.nbh * (unsigned)p.nseg;
    g.count = 1;
    return la_launch(dt, g, Dk, Dv, C, s, dry);
}

hipError_t la_bidir_launch(int dt, const drs::LAGroup &g, int Dk, int Dv, int C, hipStream_t s, bool dry) {
    if (dt == DRS_BF16) {
        switch (Dk) {
            case 16: return drs::la_bidir_dk<uint16_t, 16>(g, Dv, C, s, dry);
            case 32: return drs::la_bidir_dk<uint16_t, 32>(g, Dv, C, s, dry);
            case 64: return drs::la_bidir_dk<uint16_t, 64>(g, Dv, C, s, dry);
        }
    } else {
        switch (Dk) {
            case 16: return drs::la_bidir_dk<float, 16>(g, Dv, C, s, dry);
            case 32: return drs::la_bidir_dk<float, 32>(g, Dv, C, s, dry);
            case 64: return drs::la_bidir_dk<float, 64>(g, Dv, C, s, dry);
        }
    }
    return hipErrorNotSupported;
}

// Plan of the fused bidirectional kernel: the chunked plan itself where its segments
// have at most kBidirChunks chunks (every chunk's queries and outputs stay resident),
// with two exchange areas -- forward flags then reverse flags, forward slots then
// reverse slots -- after the 256 bytes of counters.  Longer segments take the
// composed path: splitting them further for the fused kernel measured slower than the
// two scans (e.g. 207 vs 178 us at B = 32, H = 8, T = 2048, D = 64, where the chunked
// plan has 16-chunk segments; even at 8-chunk segments it only broke even), as every
// segment folds the aggregates of all the others.  A segment waits on every other
// segment of its unit, so a unit's segments must be able to run at once: at most
// kBidirMaxSeg of them (a quarter of one resident round of 64-column workgroups).
constexpr long kBidirMaxSeg = 128;
bool la_bidir_plan(int dt, int B, int H, int T, int Dk, int Dv, LAPlan *pl) {
    if (Dk > 64 || Dv > 64) return false;
    if (!la_make_plan(dt, B, H, T, Dk, Dv, 0, pl)) return false;
    if (pl->L > drs::kBidirChunks || pl->nseg > kBidirMaxSeg) return false;
    const size_t nslots = (size_t)pl->nbh * (Dv / 16) * pl->nseg;
    pl->off_flags = 256;
    pl->off_agg = pl->off_flags + round256(2 * nslots * 8 * drs::kFlagStride);
    pl->ws_bytes = pl->off_agg + round256(2 * nslots * pl->slot_floats * 4);
    return true;
}

constexpr unsigned kLaForce = DRS_FORCE_RECURRENT | DRS_FORCE_CHUNKED;

// The step-by-step kernel takes short sequences (decode steps), forced calls and
// the per-key-channel decay mode where the chunked one for it does not apply
// (fp32 inputs, normalization, factors not 16-byte aligned); the chunked kernels
// take the rest.
bool la_use_recurrent(int T, int mode, const float *decay, unsigned flags, int dt) {
    if (flags & DRS_FORCE_RECURRENT) return true;
    if (flags & DRS_FORCE_CHUNKED) return false;
    if (T <= drs::kLaRecMaxT) return true;
    return mode == DRS_DECAY_ELEM && (dt != DRS_BF16 || (flags & DRS_NORMALIZE) || !aligned16(decay));
}

// Whether la_bidirectional takes the fused kernel (flags as given to it).
bool la_bidir_fused(int dt, int mode, const float *decay, int T, int Dk, int Dv, int chunk, unsigned flags) {
    if (flags & (DRS_NORMALIZE | DRS_LA_COMPOSE)) return false;
    if (mode != DRS_DECAY_NONE && mode != DRS_DECAY_HEAD) return false;
    if (Dk > 64 || Dv > 64) return false;
    if (chunk != 0 && chunk != la_default_chunk(dt, Dk)) return false;
    return !la_use_recurrent(T, mode, decay, flags, dt);
}

// The decay mode is not an argument here: a chunked call gets room for either
// chunked kernel (scalar factors, or one per key channel).
size_t la_ws_bytes(int B, int H, int T, int Dk, int Dv, int dt, int chunk, unsigned flags) {
    if (B < 1 || H < 1 || T < 1 || (dt != DRS_F32 && dt != DRS_BF16)) return 0;
    if ((flags & DRS_FORCE_RECURRENT) || (!(flags & DRS_FORCE_CHUNKED) && T <= drs::kLaRecMaxT)) return 0;
    LAPlan pl;
    if (!la_make_plan(dt, B, H, T, Dk, Dv, chunk, &pl)) return 0;
    const size_t elem = dt == DRS_BF16 ? drs::la_elem_ws_bytes(B, H, T, Dk, Dv) : 0;
    return elem > pl.ws_bytes ? elem : pl.ws_bytes;
}

// Validates one linear-attention call, and enqueues it unless `dry`.  Every
// check is made in the dry call, so a caller that enqueues several calls checks
// them all first.
int la_call(const void *q, const void *k, const void *v, int dt, const float *decay, int mode,
            const float *state_in, const float *cum_k_in, void *y, float *state_out, float *cum_k_out, int B,
            int H, int T, int Dk, int Dv, int chunk, unsigned flags, void *workspace, size_t workspace_bytes,
            hipStream_t s, bool dry, bool y_f32 = false, bool accumulate = false,
            drs::LAParams *prepared = nullptr, int *prepared_chunk = nullptr) {
    // prepared: set on the chunked path for scalar factors (nothing launched); left
    // with nbh = 0 on the other paths
    if (!q || !k || !v || !y) return DRS_ERR_INVALID;
    if (B < 1 || H < 1 || T < 1) return DRS_ERR_INVALID;
    if (dt != DRS_F32 && dt != DRS_BF16) return DRS_ERR_INVALID;
    if (mode != DRS_DECAY_NONE && mode != DRS_DECAY_HEAD && mode != DRS_DECAY_STEP && mode != DRS_DECAY_ELEM)
        return DRS_ERR_INVALID;
    if ((decay == nullptr) != (mode == DRS_DECAY_NONE)) return DRS_ERR_INVALID;
    if (flags & ~(DRS_REVERSE | DRS_NORMALIZE | kLaForce | DRS_LA_OWN_AGGREGATES)) return DRS_ERR_INVALID;
    if ((flags & kLaForce) == kLaForce) return DRS_ERR_INVALID;
    const bool normalize = (flags & DRS_NORMALIZE) != 0;
    if (!normalize && (cum_k_in || cum_k_out)) return DRS_ERR_INVALID;
    if (y == q || y == k || y == v) return DRS_ERR_INVALID;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y)) return DRS_ERR_INVALID;
    const void *small[] = {decay, state_in, state_out, cum_k_in, cum_k_out};
    for (const void *pp : small)
        if (pp && !aligned4(pp)) return DRS_ERR_INVALID;
    if (workspace && !aligned16(workspace)) return DRS_ERR_INVALID;
    if (!supported_dim(Dk) || !supported_dim(Dv)) return DRS_ERR_UNSUPPORTED;
    const size_t esize = dt == DRS_BF16 ? 2 : 4;
    // one unit's rows are addressed through 31-bit buffer ranges
    const size_t widest = (size_t)T * (Dk > Dv ? Dk : Dv) * (y_f32 ? 4 : esize);
    if (widest >= ((size_t)1 << 31)) return DRS_ERR_UNSUPPORTED;

    if (accumulate && (mode == DRS_DECAY_ELEM || la_use_recurrent(T, mode, decay, flags, dt)))
        return DRS_ERR_UNSUPPORTED;   // only the chunked kernel for scalar factors accumulates
    if (la_use_recurrent(T, mode, decay, flags, dt)) {
        if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64) return DRS_ERR_UNSUPPORTED;
        if ((long)B * H > 0x7fffffffL) return DRS_ERR_UNSUPPORTED;
        if (dry) return DRS_OK;
        drs::LARecParams p = {};
        p.q = q; p.k = k; p.v = v; p.y = y;
        p.decay = decay;
        p.state_in = state_in; p.cum_k_in = cum_k_in;
        p.state_out = state_out; p.cum_k_out = cum_k_out;
        p.B = B; p.H = H; p.T = T; p.Dk = Dk; p.Dv = Dv;
        p.mode = (int)mode;
        p.reverse = (flags & DRS_REVERSE) ? 1 : 0;
        p.normalize = normalize ? 1 : 0;
        p.vec_state = ((!state_in || aligned16(state_in)) && (!state_out || aligned16(state_out))) ? 1 : 0;
        p.tb = T < drs::kLaRecMaxT ? T : drs::kLaRecMaxT;
        p.y_f32 = (y_f32 && dt == DRS_BF16) ? 1 : 0;
        (void)hipGetLastError();
        return drs::la_rec_launch(p, dt == DRS_BF16, s) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
    }

    if (mode == DRS_DECAY_ELEM) {
        // one factor per key channel: its own chunked kernel (bf16, no normalization)
        if (dt != DRS_BF16 || normalize || y_f32) return DRS_ERR_UNSUPPORTED;
        if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64) return DRS_ERR_UNSUPPORTED;
        if (!aligned16(decay) || (size_t)T * Dk * 4 >= ((size_t)1 << 31)) return DRS_ERR_UNSUPPORTED;
        drs::LAElemParams ep = {};
        if (!drs::la_elem_plan(B, H, T, Dk, Dv, &ep.nseg, &ep.L)) return DRS_ERR_UNSUPPORTED;
        const size_t need = drs::la_elem_ws_bytes(B, H, T, Dk, Dv);
        if (!workspace || workspace_bytes < need) return DRS_ERR_WORKSPACE;
        if (dry) return DRS_OK;
        ep.q = static_cast<const uint16_t *>(q); ep.k = static_cast<const uint16_t *>(k);
        ep.v = static_cast<const uint16_t *>(v); ep.y = static_cast<uint16_t *>(y);
        ep.decay = decay; ep.state_in = state_in; ep.state_out = state_out;
        ep.ws = reinterpret_cast<float *>(static_cast<char *>(workspace) + 256);
        ep.B = B; ep.H = H; ep.T = T;
        ep.nchunks = (T + drs::kElemChunk - 1) / drs::kElemChunk;
        ep.reverse = (flags & DRS_REVERSE) ? 1 : 0;
        (void)hipGetLastError();
        return drs::la_elem_launch(ep, Dk, Dv, s) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
    }
    LAPlan pl;
    if (!la_make_plan(dt, B, H, T, Dk, Dv, chunk, &pl)) return DRS_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < pl.ws_bytes) return DRS_ERR_WORKSPACE;

    char *ws = static_cast<char *>(workspace);
    drs::LAParams p;
    p.q = q; p.k = k; p.v = v; p.y = y;
    p.decay = decay;
    p.state_in = state_in; p.cum_k_in = cum_k_in;
    p.state_out = state_out; p.cum_k_out = cum_k_out;
    p.ws_ctr = reinterpret_cast<unsigned *>(ws);
    p.ws_flags = reinterpret_cast<unsigned long long *>(ws + pl.off_flags);
    p.ws_agg = reinterpret_cast<float *>(ws + pl.off_agg);
    p.B = B; p.H = H; p.T = T;
    p.mode = (int)mode;
    p.reverse = (flags & DRS_REVERSE) ? 1 : 0;
    p.normalize = normalize ? 1 : 0;
    p.nchunks = pl.nchunks; p.nbh = pl.nbh; p.nseg = pl.nseg; p.L = pl.L;
    p.spin_limit = kSpinLimit;
    p.onepass = (pl.L <= drs::kOnePassChunks && Dk <= 64 && Dv <= 64) ? 1 : 0;
    // in place: the final state (or key sum) waits until every segment has read the initial one
    p.alias_state = ((state_out != nullptr && state_out == state_in) ||
                     (cum_k_out != nullptr && cum_k_out == cum_k_in)) ? 1 : 0;
    p.y_f32 = (y_f32 && dt == DRS_BF16) ? 1 : 0;
    p.accumulate = accumulate ? 1 : 0;
    // start-order ids only where the last segment waits for every other one (in place)
    p.ticket = p.alias_state;
    p.own_aggs = (flags & DRS_LA_OWN_AGGREGATES) ? 1 : 0;
    p.tag = 0;

    if (la_launch(dt, p, Dk, Dv, pl.C, s, true) != hipSuccess) return DRS_ERR_UNSUPPORTED;   // no HIP call yet
    if (prepared) {
        *prepared = p;
        *prepared_chunk = pl.C;
    }
    if (dry) return DRS_OK;
    (void)hipGetLastError();
    return la_launch(dt, p, Dk, Dv, pl.C, s, false) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
}

// Workspace bytes that this call's path uses (0 for the step-by-step kernel), and
// how many of the leading bytes must be zero before it runs (the chunked kernel's
// counters and flags).  For arguments la_call accepts.
void la_path_scratch(int dt, const float *decay, int mode, int B, int H, int T, int Dk, int Dv,
                     int chunk, unsigned flags, size_t *need, size_t *zero) {
    *need = *zero = 0;
    if (la_use_recurrent(T, mode, decay, flags, dt)) return;
    if (mode == DRS_DECAY_ELEM) {
        *need = drs::la_elem_ws_bytes(B, H, T, Dk, Dv);
        return;
    }
    LAPlan pl;
    if (!la_make_plan(dt, B, H, T, Dk, Dv, chunk, &pl)) return;
    *need = pl.ws_bytes;
    *zero = pl.off_agg;
}

// Device address of `scratch` on the current device, looked up once per device
// with that device current (each GPU holds its own copy at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

void *scratch_address() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// Clears n 16-byte words (a kernel, not hipMemsetAsync: it may be captured into a
// graph and replayed).
__global__ void zero_words(drs::u32x4 *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = drs::u32x4{0u, 0u, 0u, 0u};
}

size_t ema_ws_bytes_checked(int B, int T, int C, int dt) {
    if (B < 1 || T < 1 || C < 1 || (dt != DRS_F32 && dt != DRS_BF16)) return 0;
    if (!drs::ema_supported(B, T, C, dt == DRS_BF16 ? 2 : 4)) return 0;
    return drs::ema_ws_bytes(B, T, C);
}

int ema_call(const void *x, const void *f, int dt, const float *state_in, void *y, float *state_out, int B,
             int T, int C, unsigned flags, void *workspace, size_t workspace_bytes, hipStream_t s, bool dry) {
    if (!x || !f || !y) return DRS_ERR_INVALID;
    if (B < 1 || T < 1 || C < 1) return DRS_ERR_INVALID;
    if (dt != DRS_F32 && dt != DRS_BF16) return DRS_ERR_INVALID;
    if (flags & ~DRS_REVERSE) return DRS_ERR_INVALID;
    if (y == x || y == f) return DRS_ERR_INVALID;
    const size_t esize = dt == DRS_BF16 ? 2 : 4;
    const uintptr_t amask = esize - 1;
    if ((reinterpret_cast<uintptr_t>(x) & amask) || (reinterpret_cast<uintptr_t>(f) & amask) ||
        (reinterpret_cast<uintptr_t>(y) & amask))
        return DRS_ERR_INVALID;
    const void *small[] = {state_in, state_out};
    for (const void *pp : small)
        if (pp && !aligned4(pp)) return DRS_ERR_INVALID;
    if (workspace && !aligned16(workspace)) return DRS_ERR_INVALID;
    if (!drs::ema_supported(B, T, C, (int)esize)) return DRS_ERR_UNSUPPORTED;
    const size_t need = drs::ema_ws_bytes(B, T, C);
    if (need && (!workspace || workspace_bytes < need)) return DRS_ERR_WORKSPACE;
    if (dry) return DRS_OK;

    drs::EmaParams p = {};
    p.x = x; p.f = f; p.y = y;
    p.state_in = state_in; p.state_out = state_out;
    p.B = B; p.T = T; p.C = C;
    p.reverse = (flags & DRS_REVERSE) ? 1 : 0;
    p.ncblk = (C + 63) / 64;
    p.nblk = (T + drs::kEmaBlock - 1) / drs::kEmaBlock;
    p.walk = drs::ema_walk(B, T, C) ? 1 : 0;
    if (!p.walk) {
        char *ws = static_cast<char *>(workspace);
        const size_t nslots = (size_t)B * p.ncblk * p.nblk;
        p.ws_ctr = reinterpret_cast<unsigned *>(ws);
        p.ws_flags = reinterpret_cast<unsigned long long *>(ws + drs::kEmaCtrBytes);
        p.ws_agg = reinterpret_cast<float *>(ws + drs::kEmaCtrBytes + round256(nslots * 8));
        p.spin_limit = kSpinLimit;
    }
    (void)hipGetLastError();
    return drs::ema_launch(p, dt == DRS_BF16, s) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
}

// The second output of a bidirectional call lives after the scan's own workspace,
// never over the first 256 bytes (the counters that later calls rely on).
size_t tail_offset(size_t scan_bytes) { return round256(scan_bytes < 256 ? 256 : scan_bytes); }

}  // namespace

extern "C" {

DRS_API size_t la_workspace_bytes(int B, int H, int T, int Dk, int Dv, int dt, int chunk, unsigned flags) {
    return la_ws_bytes(B, H, T, Dk, Dv, dt, chunk, flags);
}

DRS_API int la_forward(const void *q, const void *k, const void *v, int dt, const float *decay,
                       int mode, const float *state_in, const float *cum_k_in, void *y,
                       float *state_out, float *cum_k_out, int B, int H, int T, int Dk, int Dv, int chunk,
                       unsigned flags, void *workspace, size_t workspace_bytes, void *stream) {
    return la_call(q, k, v, dt, decay, mode, state_in, cum_k_in, y, state_out, cum_k_out, B, H, T, Dk, Dv, chunk,
                   flags, workspace, workspace_bytes, static_cast<hipStream_t>(stream), false);
}

static_assert(drs::kMaxGroup == DRS_MAX_GROUP, "group size of the kernel and of the ABI");

// One la_call's arguments, for the grouped runner below.
struct LACallArgs {
    const void *q, *k, *v;
    const float *decay;
    int mode;
    const float *state_in, *cum_k_in;
    void *y;
    float *state_out, *cum_k_out;
    int Dk, Dv;
    unsigned flags;
    bool y_f32;
};

// Group layout: the workspace's 256 bytes of counters (problem i's look-back counters
// start at word kGroupCtrWord[i], so the layout keeps the one-call contract: those
// bytes zero before first use, re-armed by every call), then one region per problem
// for its flags and aggregates.  The first two problems' counters lie in different
// 128-byte lines: every workgroup ends with an atomic on its problem's finish count,
// and with both problems' counters in one line a grouped headline step took 73 us
// instead of 53.
constexpr int kGroupCtrWord[drs::kMaxGroup] = {0, 32, 16, 48};
// Problem i also tags its flags with i: each counter set has an epoch of its own, and
// a flag left in the area by a call on another counter set must not match.
size_t la_group_region(const LACallArgs &a, int dt, int B, int H, int T, int chunk) {
    const size_t w = la_ws_bytes(B, H, T, a.Dk, a.Dv, dt, chunk, a.flags & (kLaForce | DRS_NORMALIZE));
    return w > 256 ? round256(w - 256) : 0;
}
size_t la_group_bytes(const LACallArgs *a, int n, int dt, int B, int H, int T, int chunk) {
    size_t total = 256;
    for (int i = 0; i < n; ++i) total += la_group_region(a[i], dt, B, H, T, chunk);
    return total;
}

// Runs n <= kMaxGroup calls of one (B, H, T): one launch when all of them take the
// chunked kernel for scalar factors with the same shape, decay mode, normaliser and
// plan; else one call after another on the workspace as a single call uses it.  Every
// check is made before anything is enqueued; `dry` stops there.
int la_run_group(const LACallArgs *a, int n, int dt, int B, int H, int T, int chunk, void *workspace,
                 size_t workspace_bytes, hipStream_t s, bool dry) {
    char *ws = static_cast<char *>(workspace);
    const size_t need = la_group_bytes(a, n, dt, B, H, T, chunk);
    if (need > 256 && (!ws || workspace_bytes < need)) return DRS_ERR_WORKSPACE;
    drs::LAGroup g;
    g.count = n;
    int C0 = 0;
    bool one = n > 1;
    size_t off = 256;
    for (int i = 0; i < n; ++i) {
        const size_t reg = la_group_region(a[i], dt, B, H, T, chunk);
        char *view = ws ? ws + off - 256 : nullptr;   // flags and aggregates from view + 256
        g.p[i] = drs::LAParams{};
        int C = 0;
        const int st = la_call(a[i].q, a[i].k, a[i].v, dt, a[i].decay, a[i].mode, a[i].state_in, a[i].cum_k_in,
                               a[i].y, a[i].state_out, a[i].cum_k_out, B, H, T, a[i].Dk, a[i].Dv, chunk, a[i].flags,
                               view, view ? reg + 256 : 0, s, true, a[i].y_f32, false, &g.p[i], &C);
        if (st != DRS_OK) return st;
        if (g.p[i].nbh == 0 || (i > 0 && (a[i].mode != a[0].mode || a[i].Dk != a[0].Dk || a[i].Dv != a[0].Dv ||
                                          g.p[i].normalize != g.p[0].normalize || C != C0 ||
                                          g.p[i].nseg != g.p[0].nseg || g.p[i].onepass != g.p[0].onepass)))
            one = false;
        if (i == 0) C0 = C;
        g.p[i].ws_ctr = reinterpret_cast<unsigned *>(ws) + kGroupCtrWord[i];
        g.p[i].tag = (unsigned)i;
        off += reg;
    }
    if (dry) return DRS_OK;
    (void)hipGetLastError();
    if (one) {
        g.per_grid = (unsigned)g.p[0].nbh * (unsigned)g.p[0].nseg;
        return la_launch(dt, g, a[0].Dk, a[0].Dv, C0, s, false) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
    }
    for (int i = 0; i < n; ++i) {
        const int st = la_call(a[i].q, a[i].k, a[i].v, dt, a[i].decay, a[i].mode, a[i].state_in, a[i].cum_k_in,
                               a[i].y, a[i].state_out, a[i].cum_k_out, B, H, T, a[i].Dk, a[i].Dv, chunk, a[i].flags,
                               workspace, workspace_bytes, s, false, a[i].y_f32);
        if (st != DRS_OK) return st;
    }
    return DRS_OK;
}

DRS_API size_t la_forward_group_workspace_bytes(int count, int B, int H, int T, int Dk, int Dv, int dt, int chunk,
                                                unsigned flags) {
    if (count < 1 || count > drs::kMaxGroup) return 0;
    LACallArgs a{};
    a.Dk = Dk;
    a.Dv = Dv;
    a.flags = flags;
    const size_t one = la_group_region(a, dt, B, H, T, chunk);
    return one ? 256 + (size_t)count * one : 0;
}

DRS_API int la_forward_group(const drs_la_problem *probs, int count, int dt, int B, int H, int T, int Dk, int Dv,
                             int chunk, void *workspace, size_t workspace_bytes, void *stream) {
    if (!probs || count < 1 || count > drs::kMaxGroup) return DRS_ERR_INVALID;
    // no output of one problem may be an argument of another (they may run at once)
    for (int i = 0; i < count; ++i) {
        const void *outs[] = {probs[i].y, probs[i].state_out, probs[i].cum_k_out};
        for (int j = 0; j < count; ++j) {
            if (j == i) continue;
            const void *args[] = {probs[j].q, probs[j].k, probs[j].v, probs[j].decay, probs[j].state_in,
                                  probs[j].cum_k_in, probs[j].y, probs[j].state_out, probs[j].cum_k_out};
            for (const void *o : outs)
                for (const void *x : args)
                    if (o && o == x) return DRS_ERR_INVALID;
        }
    }
    if (workspace && !aligned16(workspace)) return DRS_ERR_INVALID;
    LACallArgs a[drs::kMaxGroup];
    for (int i = 0; i < count; ++i)
        a[i] = LACallArgs{probs[i].q, probs[i].k, probs[i].v, probs[i].decay, probs[i].mode, probs[i].state_in,
                          probs[i].cum_k_in, probs[i].y, probs[i].state_out, probs[i].cum_k_out, Dk, Dv,
                          probs[i].flags, false};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int st = la_run_group(a, count, dt, B, H, T, chunk, workspace, workspace_bytes, s, true);
    if (st != DRS_OK) return st;
    return la_run_group(a, count, dt, B, H, T, chunk, workspace, workspace_bytes, s, false);
}

DRS_API int la_forward_noalloc(const void *q, const void *k, const void *v, int dt, const float *decay,
                               int mode, const float *state_in, const float *cum_k_in, void *y,
                               float *state_out, float *cum_k_out, int B, int H, int T, int Dk, int Dv, int chunk,
                               unsigned flags, void *stream) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    // every check of la_forward first, with no HIP call: a missing workspace is the
    // only complaint left for a call whose path needs one
    int st = la_call(q, k, v, dt, decay, mode, state_in, cum_k_in, y, state_out, cum_k_out, B, H, T, Dk, Dv, chunk,
                     flags, nullptr, 0, s, true);
    if (st != DRS_OK && st != DRS_ERR_WORKSPACE) return st;
    size_t need, zero;
    la_path_scratch(dt, decay, mode, B, H, T, Dk, Dv, chunk, flags, &need, &zero);
    if (need > DRS_NOALLOC_SCRATCH_BYTES) return DRS_ERR_SCRATCH;
    void *ws = nullptr;
    const size_t ws_bytes = need ? DRS_NOALLOC_SCRATCH_BYTES : 0;
    if (need && !(ws = scratch_address())) return DRS_ERR_DEVICE;
    st = la_call(q, k, v, dt, decay, mode, state_in, cum_k_in, y, state_out, cum_k_out, B, H, T, Dk, Dv, chunk,
                 flags, ws, ws_bytes, s, true);
    if (st != DRS_OK) return st;
    (void)hipGetLastError();
    if (zero) {
        const size_t words = zero / 16;
        const unsigned blocks = (unsigned)(words / 256 + 1 < 1024 ? words / 256 + 1 : 1024);
        hipLaunchKernelGGL(zero_words, dim3(blocks), dim3(256), 0, s, static_cast<drs::u32x4 *>(ws), words);
        if (hipGetLastError() != hipSuccess) return DRS_ERR_DEVICE;
    }
    return la_call(q, k, v, dt, decay, mode, state_in, cum_k_in, y, state_out, cum_k_out, B, H, T, Dk, Dv, chunk,
                   flags, ws, ws_bytes, s, false);
}

DRS_API size_t la_bidirectional_workspace_bytes(int B, int H, int T, int Dk, int Dv, int dt, int chunk,
                                                unsigned flags) {
    if (B < 1 || H < 1 || T < 1 || (dt != DRS_F32 && dt != DRS_BF16)) return 0;
    if (!supported_dim(Dk) || !supported_dim(Dv)) return 0;
    const size_t esize = dt == DRS_BF16 ? 2 : 4;
    const unsigned f = flags & ~DRS_LA_COMPOSE;
    const size_t composed = tail_offset(la_ws_bytes(B, H, T, Dk, Dv, dt, chunk, f)) + (size_t)B * H * T * Dv * esize;
    // the fused kernel (the decay mode is not an argument: room for either path)
    LAPlan pl;
    if (la_bidir_fused(dt, DRS_DECAY_HEAD, nullptr, T, Dk, Dv, chunk, flags) &&
        la_bidir_plan(dt, B, H, T, Dk, Dv, &pl) && pl.ws_bytes > composed)
        return pl.ws_bytes;
    return composed;
}

DRS_API int la_bidirectional(const void *q, const void *k, const void *v, int dt, const float *decay,
                             int mode, void *y, int B, int H, int T, int Dk, int Dv, int chunk,
                             unsigned flags, void *workspace, size_t workspace_bytes, void *stream) {
    if (flags & DRS_REVERSE) return DRS_ERR_INVALID;
    const size_t need = la_bidirectional_workspace_bytes(B, H, T, Dk, Dv, dt, chunk, flags);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const unsigned fused = la_bidir_fused(dt, mode, decay, T, Dk, Dv, chunk, flags);
    flags &= ~DRS_LA_COMPOSE;
    int st = la_call(q, k, v, dt, decay, mode, nullptr, nullptr, y, nullptr, nullptr, B, H, T, Dk, Dv, chunk,
                     flags, workspace, workspace_bytes, s, true);
    if (st != DRS_OK) return st;
    if (!workspace || need == 0 || workspace_bytes < need) return DRS_ERR_WORKSPACE;
    LAPlan pl;
    if (fused && la_bidir_plan(dt, B, H, T, Dk, Dv, &pl)) {
        // both orders in one kernel: y written once
        char *ws = static_cast<char *>(workspace);
        drs::LAGroup g;
        drs::LAParams &p = g.p[0];
        p = drs::LAParams{};
        p.q = q; p.k = k; p.v = v; p.y = y;
        p.decay = decay;
        p.ws_ctr = reinterpret_cast<unsigned *>(ws);
        p.ws_flags = reinterpret_cast<unsigned long long *>(ws + pl.off_flags);
        p.ws_agg = reinterpret_cast<float *>(ws + pl.off_agg);
        p.B = B; p.H = H; p.T = T;
        p.mode = mode;
        p.nchunks = pl.nchunks; p.nbh = pl.nbh; p.nseg = pl.nseg; p.L = pl.L;
        p.spin_limit = kSpinLimit;
        p.onepass = 1;
        p.own_aggs = (flags & DRS_LA_OWN_AGGREGATES) ? 1 : 0;
        g.per_grid = (unsigned)pl.nbh * (unsigned)pl.nseg;
        g.count = 1;
        if (la_bidir_launch(dt, g, Dk, Dv, pl.C, s, true) == hipSuccess) {
            (void)hipGetLastError();
            return la_bidir_launch(dt, g, Dk, Dv, pl.C, s, false) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
        }
    }
    // forward into y, then the reverse call (both use the scan's own workspace: they
    // run in stream order).  The chunked kernel for scalar factors adds its result
    // to y as it stores; the other kernels write the tail of the workspace, and a
    // third kernel adds it into y.
    if (!la_use_recurrent(T, mode, decay, flags, dt) && mode != DRS_DECAY_ELEM) {
        st = la_call(q, k, v, dt, decay, mode, nullptr, nullptr, y, nullptr, nullptr, B, H, T, Dk, Dv, chunk,
                     flags, workspace, workspace_bytes, s, false);
        if (st != DRS_OK) return st;
        return la_call(q, k, v, dt, decay, mode, nullptr, nullptr, y, nullptr, nullptr, B, H, T, Dk, Dv, chunk,
                       flags | DRS_REVERSE, workspace, workspace_bytes, s, false, false, true);
    }
    void *tmp = static_cast<char *>(workspace) + tail_offset(la_ws_bytes(B, H, T, Dk, Dv, dt, chunk, flags));
    st = la_call(q, k, v, dt, decay, mode, nullptr, nullptr, y, nullptr, nullptr, B, H, T, Dk, Dv, chunk, flags,
                 workspace, workspace_bytes, s, false);
    if (st != DRS_OK) return st;
    st = la_call(q, k, v, dt, decay, mode, nullptr, nullptr, tmp, nullptr, nullptr, B, H, T, Dk, Dv, chunk,
                 flags | DRS_REVERSE, workspace, workspace_bytes, s, false);
    if (st != DRS_OK) return st;
    const size_t n = (size_t)B * H * T * Dv;
    return drs::add_into_launch(y, tmp, n, dt == DRS_BF16, true, s) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
}

// Workspace of la_backward: the scans' own scratch (shared: they run in stream
// order), then transposed states, shifted factors, the gradient of the state
// entering the sequence, per-step terms and per-unit sums.
struct LABwdLayout {
    size_t scan, s0t, dsft, gshift, ds0, c, partial, dq32, dk32, total;
};

bool la_bwd_layout(int B, int H, int T, int Dk, int Dv, int dt, int chunk, unsigned flags, LABwdLayout *L) {
    if (B < 1 || H < 1 || T < 1 || (dt != DRS_F32 && dt != DRS_BF16)) return false;
    if (!supported_dim(Dk) || !supported_dim(Dv)) return false;
    const unsigned f = flags & kLaForce;
    // the three gradient scans as one group: the counters, then a region per scan
    LACallArgs g[3] = {};
    g[0].Dk = g[1].Dk = Dv; g[0].Dv = g[1].Dv = Dk;
    g[2].Dk = Dk; g[2].Dv = Dv;
    g[0].flags = g[1].flags = g[2].flags = f;
    const size_t units = (size_t)B * H, st = round256(units * Dk * Dv * 4), tt = round256(units * T * 4);
    L->scan = 0;
    L->s0t = la_group_bytes(g, 3, dt, B, H, T, chunk);   // at least the 256 bytes of counters
    L->dsft = L->s0t + st;
    L->gshift = L->dsft + st;
    L->ds0 = L->gshift + tt;
    L->c = L->ds0 + st;
    L->partial = L->c + tt;
    L->dq32 = L->partial + round256(units * 4);
    // bf16 with a factor gradient: dq, dk first in fp32 (the terms q.dq - k.dk
    // are formed before rounding)
    const size_t g32 = dt == DRS_BF16 ? round256(units * T * Dk * 4) : 0;
    L->dk32 = L->dq32 + g32;
    L->total = L->dk32 + g32;
    return true;
}

// The gradients of the unnormalised form with scalar factors: three decayed scans on
// the chunked forward kernels (and the factor gradient).  The arguments are checked by
// the caller; `dry` stops after the scans' own checks.  Its scratch starts at
// `workspace` (the first 256 bytes are the scans' look-back counters).
static int la_bwd_scans(const void *q, const void *k, const void *v, int dt, const float *decay, int mode,
                 const float *state_in, const float *state_out, const void *dy, const float *dstate_out, void *dq,
                 void *dk, void *dv, float *ddecay, float *dstate_in, int B, int H, int T, int Dk, int Dv, int chunk,
                 unsigned flags, void *workspace, size_t workspace_bytes, hipStream_t s, bool dry) {
    LABwdLayout Lw;
    if (!la_bwd_layout(B, H, T, Dk, Dv, dt, chunk, flags, &Lw)) return DRS_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < Lw.total) return DRS_ERR_WORKSPACE;

    char *ws = static_cast<char *>(workspace);
    const int units = B * H;
    const bool rev = (flags & DRS_REVERSE) != 0;
    const unsigned force = flags & kLaForce;
    float *s0t = state_in ? reinterpret_cast<float *>(ws + Lw.s0t) : nullptr;
    float *dsft = dstate_out ? reinterpret_cast<float *>(ws + Lw.dsft) : nullptr;
    // factors of the two gradient scans: the factor of the step visited next; a
    // per-head factor serves as is when no final-state gradient enters the scan
    const bool shifted = mode == DRS_DECAY_STEP || (mode == DRS_DECAY_HEAD && dstate_out);
    const float *gback = shifted ? reinterpret_cast<float *>(ws + Lw.gshift) : decay;
    const int mback = shifted ? (int)DRS_DECAY_STEP : mode;
    float *ds0 = dstate_in ? (mode == DRS_DECAY_NONE ? dstate_in : reinterpret_cast<float *>(ws + Lw.ds0)) : nullptr;
    const unsigned fwd = (rev ? DRS_REVERSE : 0u) | force, bwd = (rev ? 0u : DRS_REVERSE) | force;
    const bool via32 = ddecay && dt == DRS_BF16;
    void *dq_s = via32 ? static_cast<void *>(ws + Lw.dq32) : dq;
    void *dk_s = via32 ? static_cast<void *>(ws + Lw.dk32) : dk;

    // dq_t = S_t dy_t: the forward scan of v k^T, read by dy.  dk_t = G_t v_t: the
    // opposite-order scan of dy q^T, read by v.  dv_t = G_t^T k_t: the opposite-order
    // scan of q dy^T, read by k; its final state is the gradient reaching the first
    // visited step.  Independent of each other: one launch where they share a kernel.
    const LACallArgs scans[3] = {
        {dy, v, k, decay, mode, s0t, nullptr, dq_s, nullptr, nullptr, Dv, Dk, fwd, via32},
        {v, dy, q, gback, mback, dsft, nullptr, dk_s, nullptr, nullptr, Dv, Dk, bwd, via32},
        {k, q, dy, gback, mback, dstate_out, nullptr, dv, ds0, nullptr, Dk, Dv, bwd, false}};
    // every check of the three scans first, so that an error leaves nothing enqueued
    int st = la_run_group(scans, 3, dt, B, H, T, chunk, workspace, Lw.s0t, s, true);
    if (st != DRS_OK || dry) return st;

    (void)hipGetLastError();
    bool ok = true;
    if (s0t) ok = ok && drs::transpose_units_launch(state_in, s0t, units, Dk, Dv, s) == hipSuccess;
    if (dsft) ok = ok && drs::transpose_units_launch(dstate_out, dsft, units, Dk, Dv, s) == hipSuccess;
    if (shifted)
        ok = ok && drs::shift_decay_launch(decay, (int)mode, const_cast<float *>(gback), units, H, T, rev ? 1 : 0, s) ==
                       hipSuccess;
    if (!ok) return DRS_ERR_DEVICE;
    st = la_run_group(scans, 3, dt, B, H, T, chunk, workspace, Lw.s0t, s, false);
    if (st != DRS_OK) return st;
    // the initial-state gradient g_first * ds0: inside the factor-gradient kernel when
    // that runs, else a kernel of its own
    const bool scale = dstate_in && mode != DRS_DECAY_NONE;
    if (scale && !ddecay)
        ok = ok && drs::scale_state_launch(ds0, decay, (int)mode, dstate_in, units, H, T, Dk * Dv, rev ? 1 : 0, s) ==
                       hipSuccess;
    if (ddecay) {
        float *c = reinterpret_cast<float *>(ws + Lw.c);
        if (via32)
            ok = ok && drs::decay_terms_cast_launch(q, static_cast<const float *>(dq_s), k,
                                                    static_cast<const float *>(dk_s), c, dq, dk, (long)units * T, Dk,
                                                    s) == hipSuccess;
        else
            ok = ok && drs::decay_terms_launch(static_cast<const float *>(q), static_cast<const float *>(dq),
                                               static_cast<const float *>(k), static_cast<const float *>(dk), c,
                                               (long)units * T, Dk, s) == hipSuccess;
        // counter word 8 of the workspace's first 256 bytes (the grouped scans use words
        // 0..3, 32..35 and 16..19)
        ok = ok && drs::decay_grad_launch(c, decay, (int)mode, dstate_out, state_out, Dk * Dv, ddecay,
                                          reinterpret_cast<float *>(ws + Lw.partial), B, H, T, rev ? 1 : 0,
                                          scale ? ds0 : nullptr, scale ? dstate_in : nullptr,
                                          reinterpret_cast<unsigned *>(ws) + 8, s) == hipSuccess;
    }
    return ok ? DRS_OK : DRS_ERR_DEVICE;
}

// The normalised form with one factor per head, one per step or none, bf16 inputs:
// unnormalised fp32 scans on the chunked kernels.  With n = S^T q, d = z^T q (y = n / d):
//   a = dy / d, c = -(dy . n) / d^2;
//   dq = S a + z c;  dk = G v + Gz;  dv = G^T k;
//   G = the decayed sum over the later steps of q a^T (+ dS_final), Gz likewise of c q
//   (+ dz_final);
// the initial state's and key sum's gradients are G and Gz at the first step times its
// factor, and the factor gradient follows from the suffix sums of q . dq - k . dk plus
// <dS_final, S_final> + dz_final . z_final, as for the unnormalised form.
// Each product is a scan of the forward kernel: n (q, k, v), d (q, k, ones), S a
// (a, v, k), z c (c, ones, k), G^T k (k, q, a), G v (v, a, q), Gz (ones, c, q); a
// 1-wide operand is padded to 16 columns.  dq and dk are differences of their two
// parts (tens of times larger than the result), so every scan, and a, c, run in fp32
// on fp32 copies of q, k, v: with bf16 a and c the parts' rounding missed the bf16 bar.
struct LANormBwdLayout {
    size_t q32, k32, v32, na, d16, c16, ones, dq32, dk32, dv32, s0t, z0col, z0row, dsft, dzrow, gz;
    size_t gshift, sT, zT, ds0, dz0, dsz, sz, c, partial, total;
};
// Chunk of one of these fp32 scans (chunk 0: the default): 32-row chunks where the
// scan's output is at least 64 wide (measured at B = 4, H = 16, T = 4096: 266 vs 297 us
// for 128 x 128, 88 vs 98 us for 16 x 128), the default 16 for the 16-wide output of d
// (118 vs 185 us).
static int la_norm_bwd_chunk(int chunk, int Dv_scan) { return chunk ? chunk : (Dv_scan >= 64 ? 32 : 0); }
static bool la_norm_bwd_layout(int B, int H, int T, int Dk, int Dv, int chunk, unsigned force, LANormBwdLayout *L) {
    if (!supported_dim(Dk) || !supported_dim(Dv)) return false;
    size_t scan = 0;   // one scratch for the scans (they run in stream order), from offset 0
    const int shapes[4][2] = {{Dk, Dv}, {Dk, 16}, {Dv, Dk}, {16, Dk}};
    for (const auto &sh : shapes) {
        const size_t w = la_ws_bytes(B, H, T, sh[0], sh[1], DRS_F32, la_norm_bwd_chunk(chunk, sh[1]), force);
        if (w > scan) scan = w;
    }
    const size_t rows = (size_t)B * H * T, units = (size_t)B * H, st = units * Dk * Dv * 4, zt = units * Dk * 16 * 4;
    size_t off = round256(scan < 256 ? 256 : scan);
    auto take = [&](size_t bytes) { const size_t o = off; off += round256(bytes); return o; };
    L->q32 = take(rows * Dk * 4); L->k32 = take(rows * Dk * 4); L->v32 = take(rows * Dv * 4);
    L->na = take(rows * Dv * 4); L->d16 = take(rows * 16 * 4); L->c16 = take(rows * 16 * 4);
    L->ones = take(rows * 16 * 4);
    L->dq32 = take(rows * Dk * 4); L->dk32 = take(rows * Dk * 4); L->dv32 = take(rows * Dv * 4);
    L->s0t = take(st); L->z0col = take(zt); L->z0row = take(zt);
    L->dsft = take(st); L->dzrow = take(zt); L->gz = take(zt);
    // factors: the reverse scans' shifted factors, the initial states' gradients before
    // the first factor, and the factor gradient's final states, terms and partial sums
    L->gshift = take(rows * 4); L->sT = take(st); L->zT = take(zt); L->ds0 = take(st); L->dz0 = take(units * Dk * 4);
    L->dsz = take(units * (Dk * Dv + Dk) * 4); L->sz = take(units * (Dk * Dv + Dk) * 4);
    L->c = take(rows * 4); L->partial = take(units * 4);
    L->total = off;
    return true;
}
static bool la_norm_bwd_chunked(int dt, int mode, int T, unsigned flags) {
    return dt == DRS_BF16 && (flags & DRS_NORMALIZE) && mode != DRS_DECAY_ELEM && !(flags & DRS_FORCE_RECURRENT) &&
           T > drs::kLaRecMaxT;
}
static int la_norm_bwd_scans(const void *q, const void *k, const void *v, const float *decay, int mode,
                             const float *state_in, const float *cum_k_in, const void *dy, const float *dstate_out,
                             const float *dcum_k_out, void *dq, void *dk, void *dv, float *ddecay, float *dstate_in,
                             float *dcum_k_in, int B, int H, int T, int Dk, int Dv, int chunk, unsigned flags,
                             void *workspace, size_t workspace_bytes, hipStream_t s) {
    const unsigned force = flags & kLaForce;
    LANormBwdLayout L;
    if (!la_norm_bwd_layout(B, H, T, Dk, Dv, chunk, force, &L)) return DRS_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < L.total) return DRS_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    auto F = [&](size_t o) { return reinterpret_cast<float *>(ws + o); };
    const int units = B * H;
    const long rows = (long)units * T;
    const bool rev = (flags & DRS_REVERSE) != 0;
    const unsigned fwd = (rev ? DRS_REVERSE : 0u) | force, bwd = (rev ? 0u : DRS_REVERSE) | force;
    const bool decays = mode != DRS_DECAY_NONE;
    const bool fin = dstate_out || dcum_k_out;
    float *q32 = F(L.q32), *k32 = F(L.k32), *v32 = F(L.v32), *na = F(L.na), *d16 = F(L.d16), *c16 = F(L.c16);
    float *ones = F(L.ones), *dq32 = F(L.dq32), *dk32 = F(L.dk32), *dv32 = F(L.dv32);
    float *s0t = state_in ? F(L.s0t) : nullptr, *z0col = cum_k_in ? F(L.z0col) : nullptr;
    float *z0row = cum_k_in ? F(L.z0row) : nullptr, *dsft = dstate_out ? F(L.dsft) : nullptr;
    float *dzrow = dcum_k_out ? F(L.dzrow) : nullptr, *gz = dcum_k_in ? F(L.gz) : nullptr;
    // the reverse scans take the factor of the step visited next (a per-head factor as
    // it is while their states start from zero)
    const bool shifted = mode == DRS_DECAY_STEP || (mode == DRS_DECAY_HEAD && fin);
    const float *gback = shifted ? F(L.gshift) : decay;
    const int mback = shifted ? (int)DRS_DECAY_STEP : mode;
    // the initial states' gradients: G and Gz at the first visited step, times its factor
    float *ds0 = dstate_in ? (decays ? F(L.ds0) : dstate_in) : nullptr;
    // the factor gradient needs the final state and key sum of the forward scans
    const bool dg = ddecay && decays;
    float *sT = dg && fin ? F(L.sT) : nullptr, *zT = dg && fin ? F(L.zT) : nullptr;
    struct Scan {
        const void *q, *k, *v;
        const float *g;
        int mode;
        const float *state_in;
        void *y;
        float *state_out;
        int Dk, Dv;
        unsigned flags;
        bool accumulate;
    };
    const Scan scans[7] = {
        {q32, k32, v32, decay, mode, state_in, na, sT, Dk, Dv, fwd, false},           // n = S^T q
        {q32, k32, ones, decay, mode, z0col, d16, zT, Dk, 16, fwd, false},            // d = z^T q (column 0)
        {na, v32, k32, decay, mode, s0t, dq32, nullptr, Dv, Dk, fwd, false},          // S a (na holds a by then)
        {c16, ones, k32, decay, mode, z0row, dq32, nullptr, 16, Dk, fwd, true},       // + z c
        {k32, q32, na, gback, mback, dstate_out, dv32, ds0, Dk, Dv, bwd, false},      // dv = G^T k; G at the first step
        {v32, na, q32, gback, mback, dsft, dk32, nullptr, Dv, Dk, bwd, false},        // G v
        {ones, c16, q32, gback, mback, dzrow, dk32, gz, 16, Dk, bwd, true}};          // + Gz; Gz at the first step
    // every check first, so that an error leaves nothing enqueued
    for (const Scan &c : scans) {
        const int st = la_call(c.q, c.k, c.v, DRS_F32, c.g, c.mode, c.state_in, nullptr, c.y, c.state_out, nullptr, B,
                               H, T, c.Dk, c.Dv, la_norm_bwd_chunk(chunk, c.Dv), c.flags, workspace, workspace_bytes, s,
                               true, false, c.accumulate);
        if (st != DRS_OK) return st;
    }
    (void)hipGetLastError();
    bool ok = drs::cast_up_launch(q, q32, (size_t)rows * Dk, s) == hipSuccess &&
              drs::cast_up_launch(k, k32, (size_t)rows * Dk, s) == hipSuccess &&
              drs::cast_up_launch(v, v32, (size_t)rows * Dv, s) == hipSuccess &&
              drs::ones16_launch(ones, (size_t)rows, s) == hipSuccess;
    if (s0t) ok = ok && drs::transpose_units_launch(state_in, s0t, units, Dk, Dv, s) == hipSuccess;
    if (dsft) ok = ok && drs::transpose_units_launch(dstate_out, dsft, units, Dk, Dv, s) == hipSuccess;
    if (z0col) ok = ok && drs::pad16_launch(cum_k_in, z0col, units, Dk, true, s) == hipSuccess &&
                    drs::pad16_launch(cum_k_in, z0row, units, Dk, false, s) == hipSuccess;
    if (dzrow) ok = ok && drs::pad16_launch(dcum_k_out, dzrow, units, Dk, false, s) == hipSuccess;
    if (shifted)
        ok = ok && drs::shift_decay_launch(decay, mode, const_cast<float *>(gback), units, H, T, rev ? 1 : 0, s) ==
                       hipSuccess;
    if (!ok) return DRS_ERR_DEVICE;
    for (int i = 0; i < 7; ++i) {
        const Scan &c = scans[i];
        const int st = la_call(c.q, c.k, c.v, DRS_F32, c.g, c.mode, c.state_in, nullptr, c.y, c.state_out, nullptr, B,
                               H, T, c.Dk, c.Dv, la_norm_bwd_chunk(chunk, c.Dv), c.flags, workspace, workspace_bytes, s,
                               false, false, c.accumulate);
        if (st != DRS_OK) return st;
        if (i == 1 && drs::norm_terms_launch(dy, na, d16, c16, rows, Dv, s) != hipSuccess) return DRS_ERR_DEVICE;
    }
    // dz0 before the first factor (row 0 of Gz), then both initial-state gradients scaled
    float *dz0 = gz ? (decays ? F(L.dz0) : dcum_k_in) : nullptr;
    if (gz) ok = ok && drs::row0_launch(gz, dz0, units, Dk, s) == hipSuccess;
    if (decays && dstate_in)
        ok = ok && drs::scale_state_launch(ds0, decay, mode, dstate_in, units, H, T, Dk * Dv, rev ? 1 : 0, s) ==
                       hipSuccess;
    if (decays && dcum_k_in)
        ok = ok && drs::scale_state_launch(dz0, decay, mode, dcum_k_in, units, H, T, Dk, rev ? 1 : 0, s) == hipSuccess;
    ok = ok && drs::cast_down_launch(dv32, dv, (size_t)rows * Dv, s) == hipSuccess;
    if (dg) {
        // c_t = q . dq - k . dk (fp32 dq, dk, also rounded into the outputs), and the
        // final states' term <dS_T, S_T> + dz_T . z_T as one dot over Dk Dv + Dk values
        float *c = F(L.c), *dsz = fin ? F(L.dsz) : nullptr, *sz = fin ? F(L.sz) : nullptr;
        ok = ok && drs::decay_terms_cast_launch(q, dq32, k, dk32, c, dq, dk, rows, Dk, s) == hipSuccess;
        if (fin)
            ok = ok && drs::concat_state_launch(dstate_out, dcum_k_out, 1, dsz, units, Dk * Dv, Dk, s) == hipSuccess &&
                 drs::concat_state_launch(sT, zT, 16, sz, units, Dk * Dv, Dk, s) == hipSuccess;
        // counter word 8 of the workspace's first 256 bytes (the scans use words 0..3)
        ok = ok && drs::decay_grad_launch(c, decay, mode, dsz, sz, Dk * Dv + Dk, ddecay, F(L.partial), B, H, T,
                                          rev ? 1 : 0, nullptr, nullptr, reinterpret_cast<unsigned *>(ws) + 8, s) ==
                       hipSuccess;
    } else {
        ok = ok && drs::cast_down_launch(dq32, dq, (size_t)rows * Dk, s) == hipSuccess &&
             drs::cast_down_launch(dk32, dk, (size_t)rows * Dk, s) == hipSuccess;
    }
    return ok ? DRS_OK : DRS_ERR_DEVICE;
}

// The step-by-step backward takes the normalised form, one factor per key channel
// and forced calls; the chunked gradient scans take the rest.  (Splitting the
// normalised form into two unnormalised problems for the chunked scans -- the
// numerator with output gradient dy / d, the denominator with -(dy . y) / d -- lost
// too much: dq and dk are differences of the two problems' parts, which can be tens
// of times larger than the result.  With those gradients rounded to bf16 before the
// scans it missed the 2e-2 bar on a few hundred elements in 100 K, and in fp32 the
// per-step factor gradient, a suffix sum over both problems, missed 1e-5 at T = 2000.)
static bool la_bwd_recurrent(int mode, unsigned flags) {
    return (flags & DRS_NORMALIZE) || mode == DRS_DECAY_ELEM || (flags & DRS_FORCE_RECURRENT);
}

DRS_API size_t la_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv, int dt, int chunk,
                                           unsigned flags) {
    LABwdLayout L;
    if (!la_bwd_layout(B, H, T, Dk, Dv, dt, chunk, flags, &L)) return 0;
    // the decay mode is not an argument: room for either path
    size_t need = 256 + drs::la_rec_bwd_ws_bytes(B, H, T, Dk, Dv, DRS_DECAY_ELEM, (flags & DRS_NORMALIZE) != 0,
                                                 true, true);
    if (L.total > need) need = L.total;
    LANormBwdLayout N;
    if (la_norm_bwd_chunked(dt, DRS_DECAY_NONE, T, flags) &&
        la_norm_bwd_layout(B, H, T, Dk, Dv, chunk, flags & kLaForce, &N) && N.total > need)
        need = N.total;
    return need;
}

DRS_API int la_backward(const void *q, const void *k, const void *v, int dt, const float *decay,
                        int mode, const float *state_in, const float *cum_k_in, const float *state_out,
                        const void *dy, const float *dstate_out, const float *dcum_k_out, void *dq, void *dk,
                        void *dv, float *ddecay, float *dstate_in, float *dcum_k_in, int B, int H, int T, int Dk,
                        int Dv, int chunk, unsigned flags, void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !k || !v || !dy || !dq || !dk || !dv) return DRS_ERR_INVALID;
    if (B < 1 || H < 1 || T < 1) return DRS_ERR_INVALID;
    if (dt != DRS_F32 && dt != DRS_BF16) return DRS_ERR_INVALID;
    if (mode != DRS_DECAY_NONE && mode != DRS_DECAY_HEAD && mode != DRS_DECAY_STEP && mode != DRS_DECAY_ELEM)
        return DRS_ERR_INVALID;
    if ((decay == nullptr) != (mode == DRS_DECAY_NONE)) return DRS_ERR_INVALID;
    if (mode == DRS_DECAY_NONE && ddecay) return DRS_ERR_INVALID;
    if (flags & ~(DRS_REVERSE | DRS_NORMALIZE | kLaForce)) return DRS_ERR_INVALID;
    if ((flags & kLaForce) == kLaForce) return DRS_ERR_INVALID;
    const bool normalize = (flags & DRS_NORMALIZE) != 0;
    if (!normalize && (cum_k_in || dcum_k_out || dcum_k_in)) return DRS_ERR_INVALID;
    const bool rec = la_bwd_recurrent(mode, flags);
    // <dS_final, S_final> needs S_final (the step-by-step path recomputes it)
    if (!rec && ddecay && dstate_out && !state_out) return DRS_ERR_INVALID;
    const void *outs[] = {dq, dk, dv, ddecay, dstate_in, dcum_k_in};
    const void *ins[] = {q, k, v, dy, decay, state_in, cum_k_in, state_out, dstate_out, dcum_k_out};
    for (const void *o : outs)
        for (const void *i : ins)
            if (o && o == i) return DRS_ERR_INVALID;
    if (dq == dk || dq == dv || dk == dv) return DRS_ERR_INVALID;
    if (dstate_in && (dstate_in == ddecay || dstate_in == dcum_k_in)) return DRS_ERR_INVALID;
    if (ddecay && ddecay == dcum_k_in) return DRS_ERR_INVALID;
    const void *big[] = {q, k, v, dy, dq, dk, dv};
    for (const void *pp : big)
        if (!aligned16(pp)) return DRS_ERR_INVALID;
    const void *small[] = {decay, state_in, cum_k_in, state_out, dstate_out, dcum_k_out, ddecay, dstate_in, dcum_k_in};
    for (const void *pp : small)
        if (pp && !aligned4(pp)) return DRS_ERR_INVALID;
    if (workspace && !aligned16(workspace)) return DRS_ERR_INVALID;
    if (la_norm_bwd_chunked(dt, mode, T, flags)) {
        if (!supported_dim(Dk) || !supported_dim(Dv)) return DRS_ERR_UNSUPPORTED;
        if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64) return DRS_ERR_UNSUPPORTED;
        return la_norm_bwd_scans(q, k, v, decay, mode, state_in, cum_k_in, dy, dstate_out, dcum_k_out, dq, dk, dv,
                                 ddecay, dstate_in, dcum_k_in, B, H, T, Dk, Dv, chunk, flags, workspace,
                                 workspace_bytes, static_cast<hipStream_t>(stream));
    }
    if (rec) {
        if (!supported_dim(Dk) || !supported_dim(Dv)) return DRS_ERR_UNSUPPORTED;
        if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64) return DRS_ERR_UNSUPPORTED;
        if ((long)B * H > 0x7fffffffL) return DRS_ERR_UNSUPPORTED;
        const bool fin = dstate_out || dcum_k_out;
        // after the 256 bytes of look-back counters, which other calls sharing the
        // workspace rely on (this path never touches them)
        const size_t scratch = drs::la_rec_bwd_ws_bytes(B, H, T, Dk, Dv, mode, normalize, ddecay != nullptr, fin);
        const size_t need = scratch ? 256 + scratch : 0;
        if (need && (!workspace || workspace_bytes < need)) return DRS_ERR_WORKSPACE;
        drs::LARecBwdParams p = {};
        p.q = q; p.k = k; p.v = v; p.dy = dy;
        p.decay = decay;
        p.state_in = state_in; p.cum_k_in = cum_k_in;
        p.dstate_out = dstate_out; p.dcum_k_out = dcum_k_out;
        p.dq = dq; p.dk = dk; p.dv = dv;
        p.ddecay = ddecay; p.dstate_in = dstate_in; p.dcum_k_in = dcum_k_in;
        p.B = B; p.H = H; p.T = T; p.Dk = Dk; p.Dv = Dv;
        p.mode = (int)mode;
        p.reverse = (flags & DRS_REVERSE) ? 1 : 0;
        p.normalize = normalize ? 1 : 0;
        drs::la_rec_bwd_layout(need ? static_cast<char *>(workspace) + 256 : nullptr, p, fin);
        p.tb = T < 16 ? T : 16;
        (void)hipGetLastError();
        return drs::la_rec_bwd_launch(p, dt == DRS_BF16, static_cast<hipStream_t>(stream)) == hipSuccess
                   ? DRS_OK : DRS_ERR_DEVICE;
    }
    return la_bwd_scans(q, k, v, dt, decay, mode, state_in, state_out, dy, dstate_out, dq, dk, dv, ddecay, dstate_in,
                        B, H, T, Dk, Dv, chunk, flags, workspace, workspace_bytes, static_cast<hipStream_t>(stream),
                        false);
}

DRS_API size_t wkv_workspace_bytes(int B, int T, int C, unsigned flags) {
    if (B < 1 || T < 1 || C < 1) return 0;
    if (flags & ~(kWkvForce | DRS_WKV_OWN_AGGREGATES)) return 0;
    const WkvPath path = wkv_choose(B, T, C, flags);
    if (path == WkvPath::kChain && !drs::wkv_chain_supported(B, T, C)) return 0;
    if (path == WkvPath::kRows && !drs::wkv_rows_supported(B, T, C)) return 0;
    return wkv_ws_bytes(B, T, C, path);
}

DRS_API int wkv_forward(const float *w, const float *u, const float *k, const float *v, const float *state_in,
                        float *y, float *state_out, int B, int T, int C, unsigned flags, void *workspace,
                        size_t workspace_bytes, void *stream) {
    if (!w || !u || !k || !v || !y) return DRS_ERR_INVALID;
    if (B < 1 || T < 1 || C < 1) return DRS_ERR_INVALID;
    if (flags & ~(kWkvForce | DRS_WKV_OWN_AGGREGATES)) return DRS_ERR_INVALID;
    const unsigned force = flags & kWkvForce;
    if (force & (force - 1)) return DRS_ERR_INVALID;   // more than one FORCE flag
    if (y == k || y == v) return DRS_ERR_INVALID;
    const void *ptrs[] = {w, u, k, v, y, state_in, state_out, workspace};
    for (const void *pp : ptrs)
        if (pp && !aligned4(pp)) return DRS_ERR_INVALID;
    if (workspace && !aligned16(workspace)) return DRS_ERR_INVALID;
    if (B > 65535) return DRS_ERR_UNSUPPORTED;

    const WkvPath path = wkv_choose(B, T, C, flags);
    if (path == WkvPath::kChain && !drs::wkv_chain_supported(B, T, C)) return DRS_ERR_UNSUPPORTED;
    if (path == WkvPath::kRows) {   // 16-byte pieces of k, v, y; no state updated in place
        if (!drs::wkv_rows_supported(B, T, C) || !aligned16(k) || !aligned16(v) || !aligned16(y) ||
            (state_out && state_out == state_in))
            return DRS_ERR_UNSUPPORTED;
    }
    const size_t need = wkv_ws_bytes(B, T, C, path);
    if (need && (!workspace || workspace_bytes < need)) return DRS_ERR_WORKSPACE;

    drs::WKVParams p = {};
    p.w = w; p.u = u; p.k = k; p.v = v; p.state_in = state_in;
    p.y = y; p.state_out = state_out;
    p.B = B; p.T = T; p.C = C;
    p.seg_len = T; p.nseg = 1;
    char *ws = static_cast<char *>(workspace);
    if (path == WkvPath::kScan) {
        drs::wkv_scan_plan(B, T, C, &p.seg_len, &p.nseg);
        if (p.nseg > 65535) return DRS_ERR_UNSUPPORTED;
        p.ws = reinterpret_cast<float *>(ws + drs::kWkvCtrBytes);
    } else if (path == WkvPath::kChain) {
        p.ncblk = (C + 63) / 64;
        p.nblk = (T + drs::kWkvChainBlock - 1) / drs::kWkvChainBlock;
        const size_t nslots = (size_t)B * p.ncblk * p.nblk;
        p.ws_ctr = reinterpret_cast<unsigned *>(ws);
        p.ws_flags = reinterpret_cast<unsigned long long *>(ws + drs::kWkvCtrBytes);
        p.ws_agg = reinterpret_cast<float *>(ws + drs::kWkvCtrBytes + round256(nslots * 8));
        p.spin_limit = kSpinLimit;
        p.walk = (long)B * p.ncblk >= drs::kWkvWalkUnits ? 1 : 0;
        // start-order ids only where the final state overwrites the initial one
        p.ticket = (state_out != nullptr && state_out == state_in) ? 1 : 0;
        p.own_aggs = ((flags & DRS_WKV_OWN_AGGREGATES) && !p.ticket) ? 1 : 0;   // in place: always waits
    } else if (path == WkvPath::kRows) {
        drs::wkv_rows_layout(ws, p);
        p.spin_limit = kSpinLimit;
        p.own_aggs = (flags & DRS_WKV_OWN_AGGREGATES) ? 1 : 0;
    }
    (void)hipGetLastError();
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (path) {
        case WkvPath::kChain: e = drs::wkv_launch_chain(p, s); break;
        case WkvPath::kRows: e = drs::wkv_launch_rows(p, s); break;
        case WkvPath::kScan: e = drs::wkv_launch_scan(p, s); break;
        default: e = drs::wkv_launch_seq(p, s); break;
    }
    return e == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
}

DRS_API size_t wkv_backward_workspace_bytes(int B, int T, int C, unsigned flags) {
    if (B < 1 || T < 1 || C < 1 || flags) return 0;
    return drs::wkv_bwd_ws_bytes(B, T, C);
}

DRS_API int wkv_backward(const float *w, const float *u, const float *k, const float *v, const float *state_in,
                         const float *dy, float *dw, float *du, float *dk, float *dv, float *dstate_in, int B, int T,
                         int C, unsigned flags, void *workspace, size_t workspace_bytes, void *stream) {
    if (!w || !u || !k || !v || !dy || !dk || !dv) return DRS_ERR_INVALID;
    if (B < 1 || T < 1 || C < 1) return DRS_ERR_INVALID;
    if (flags) return DRS_ERR_INVALID;
    const void *outs[] = {dw, du, dk, dv, dstate_in};
    const void *ins[] = {w, u, k, v, state_in, dy};
    for (const void *o : outs)
        for (const void *i : ins)
            if (o && o == i) return DRS_ERR_INVALID;
    if (dk == dv || (dw && dw == du)) return DRS_ERR_INVALID;
    if (dstate_in && (dstate_in == dk || dstate_in == dv || dstate_in == dw || dstate_in == du))
        return DRS_ERR_INVALID;
    const void *ptrs[] = {w, u, k, v, state_in, dy, dw, du, dk, dv, dstate_in};
    for (const void *pp : ptrs)
        if (pp && !aligned4(pp)) return DRS_ERR_INVALID;
    if (workspace && !aligned16(workspace)) return DRS_ERR_INVALID;
    if (B > 65535 || (size_t)T * C * 4 >= ((size_t)1 << 31)) return DRS_ERR_UNSUPPORTED;
    const size_t need = drs::wkv_bwd_ws_bytes(B, T, C);
    if (!workspace || workspace_bytes < need) return DRS_ERR_WORKSPACE;
    drs::WKVBwdParams p = {};
    p.w = w; p.u = u; p.k = k; p.v = v; p.state_in = state_in; p.dy = dy;
    p.dk = dk; p.dv = dv; p.dw = dw; p.du = du; p.dstate_in = dstate_in;
    p.B = B; p.T = T; p.C = C;
    drs::wkv_bwd_layout(B, T, C, static_cast<char *>(workspace), p);
    (void)hipGetLastError();
    return drs::wkv_launch_bwd(p, static_cast<hipStream_t>(stream)) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
}

DRS_API size_t ema_workspace_bytes(int B, int T, int C, int dt, unsigned flags) {
    if (flags & ~DRS_REVERSE) return 0;
    return ema_ws_bytes_checked(B, T, C, dt);
}

DRS_API int ema_forward(const void *x, const void *f, int dt, const float *state_in, void *y,
                        float *state_out, int B, int T, int C, unsigned flags, void *workspace,
                        size_t workspace_bytes, void *stream) {
    return ema_call(x, f, dt, state_in, y, state_out, B, T, C, flags, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream), false);
}

// Enough channels to fill the GPU: one fused kernel (x, f read twice, y written
// once); otherwise the forward and reverse calls and an add.
bool ema_bidir_fused(int B, int T, int C) { return drs::ema_walk(B, T, C); }

DRS_API size_t ema_bidirectional_workspace_bytes(int B, int T, int C, int dt, unsigned flags) {
    if (flags) return 0;
    if (B < 1 || T < 1 || C < 1 || (dt != DRS_F32 && dt != DRS_BF16)) return 0;
    if (!drs::ema_supported(B, T, C, dt == DRS_BF16 ? 2 : 4)) return 0;
    if (ema_bidir_fused(B, T, C)) return drs::ema_bidir_ws_bytes(B, T, C);
    const size_t esize = dt == DRS_BF16 ? 2 : 4;
    return tail_offset(ema_ws_bytes_checked(B, T, C, dt)) + (size_t)B * T * C * esize;
}

DRS_API int ema_bidirectional(const void *x, const void *f, int dt, void *y, int B, int T, int C,
                              unsigned flags, void *workspace, size_t workspace_bytes, void *stream) {
    if (flags) return DRS_ERR_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int st = ema_call(x, f, dt, nullptr, y, nullptr, B, T, C, 0, workspace, workspace_bytes, s, true);
    if (st != DRS_OK) return st;
    const size_t need = ema_bidirectional_workspace_bytes(B, T, C, dt, 0);
    if (!workspace || need == 0 || workspace_bytes < need) return DRS_ERR_WORKSPACE;
    if (ema_bidir_fused(B, T, C)) {
        drs::EmaParams p = {};
        p.x = x; p.f = f; p.y = y;
        p.B = B; p.T = T; p.C = C;
        p.ncblk = (C + 63) / 64;
        p.nblk = (T + drs::kEmaBlock - 1) / drs::kEmaBlock;
        p.ws_agg = reinterpret_cast<float *>(static_cast<char *>(workspace) + drs::kEmaCtrBytes);
        (void)hipGetLastError();
        return drs::ema_bidir_launch(p, dt == DRS_BF16, s) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
    }
    void *tmp = static_cast<char *>(workspace) + tail_offset(ema_ws_bytes_checked(B, T, C, dt));
    st = ema_call(x, f, dt, nullptr, y, nullptr, B, T, C, 0, workspace, workspace_bytes, s, false);
    if (st != DRS_OK) return st;
    st = ema_call(x, f, dt, nullptr, tmp, nullptr, B, T, C, DRS_REVERSE, workspace, workspace_bytes, s, false);
    if (st != DRS_OK) return st;
    const size_t n = (size_t)B * T * C;
    const bool vec = aligned16(y);
    return drs::add_into_launch(y, tmp, n, dt == DRS_BF16, vec, s) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
}

DRS_API const char *drs_status_string(int status) {
    switch (status) {
        case DRS_OK: return "ok";
        case DRS_ERR_INVALID: return "invalid argument";
        case DRS_ERR_UNSUPPORTED: return "unsupported size or option";
        case DRS_ERR_WORKSPACE: return "workspace missing or too small";
        case DRS_ERR_DEVICE: return "HIP launch failed";
        case DRS_ERR_SCRATCH: return "the call needs more scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

DRS_API int drs_version(void) { return 10300; }

}  // extern "C"
