// api.hip -- the C ABI of libdrs: argument validation, kernel selection, launch.
//
// Every check happens on the host before anything is enqueued, so a non-zero
// return leaves all outputs untouched.  No exception crosses the boundary.
#include <stdint.h>

#include "combine.h"
#include "drs.h"
#include "ema.h"
#include "la_bwd.h"
#include "la_elem.h"
#include "la_fwd_launch.h"
#include "la_rec.h"
#include "wkv.h"


namespace {

constexpr int kTargetWaves = 2048;        // eight per compute unit of an MI355X
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

int la_default_chunk(drs_dtype dt, int Dk) {
    if (dt == DRS_BF16) return 64;
    if (Dk <= 32) return 64;
    return Dk == 64 ? 32 : 16;
}

// Returns false for sizes the kernels do not cover.
bool la_make_plan(drs_dtype dt, int B, int H, int T, int Dk, int Dv, int chunk, LAPlan *pl) {
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
    pl->off_agg = pl->off_flags + round256(nslots * 8);
    pl->ws_bytes = pl->off_agg + round256(nslots * pl->slot_floats * 4);
    return true;
}

enum class WkvPath { kSeq, kScan, kChain };

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
    if (drs::wkv_chain_supported(B, T, C) && T > drs::kWkvChainSub) {
        const long units = (long)B * ((C + 63) / 64), nblk = (T + drs::kWkvChainBlock - 1) / drs::kWkvChainBlock;
        if (units >= drs::kWkvWalkUnits || units * nblk <= kWkvChainOneRound) return WkvPath::kChain;
    }
    return drs::wkv_use_scan(B, T, C) ? WkvPath::kScan : WkvPath::kSeq;
}

size_t wkv_ws_bytes(int B, int T, int C, WkvPath path) {
    if (path == WkvPath::kChain) return drs::wkv_chain_ws_bytes(B, T, C);
    if (path == WkvPath::kScan) {
        int L, n;
        drs::wkv_scan_plan(B, T, C, &L, &n);
        return drs::kWkvCtrBytes + (size_t)(n + 1) * 3 * (size_t)B * (size_t)C * sizeof(float);
    }
    return 0;
}

constexpr unsigned kWkvForce = DRS_FORCE_SEQ | DRS_FORCE_SCAN | DRS_FORCE_CHAIN;

hipError_t la_launch(drs_dtype dt, const drs::LAParams &p, int Dk, int Dv, int C, hipStream_t s, bool dry) {
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

constexpr unsigned kLaForce = DRS_FORCE_RECURRENT | DRS_FORCE_CHUNKED;

// The step-by-step kernel takes short sequences (decode steps), forced calls and
// the per-key-channel decay mode where the chunked one for it does not apply
// (fp32 inputs, normalization, factors not 16-byte aligned); the chunked kernels
// take the rest.
bool la_use_recurrent(int T, drs_decay mode, const float *decay, unsigned flags, drs_dtype dt) {
    if (flags & DRS_FORCE_RECURRENT) return true;
    if (flags & DRS_FORCE_CHUNKED) return false;
    if (T <= drs::kLaRecMaxT) return true;
    return mode == DRS_DECAY_ELEM && (dt != DRS_BF16 || (flags & DRS_NORMALIZE) || !aligned16(decay));
}

// The decay mode is not an argument here: a chunked call gets room for either
// chunked kernel (scalar factors, or one per key channel).
size_t la_ws_bytes(int B, int H, int T, int Dk, int Dv, drs_dtype dt, int chunk, unsigned flags) {
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
int la_call(const void *q, const void *k, const void *v, drs_dtype dt, const float *decay, drs_decay mode,
            const float *state_in, const float *cum_k_in, void *y, float *state_out, float *cum_k_out, int B,
            int H, int T, int Dk, int Dv, int chunk, unsigned flags, void *workspace, size_t workspace_bytes,
            hipStream_t s, bool dry, bool y_f32 = false, bool accumulate = false) {
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

    if (la_launch(dt, p, Dk, Dv, pl.C, s, true) != hipSuccess) return DRS_ERR_UNSUPPORTED;   // no HIP call yet
    if (dry) return DRS_OK;
    (void)hipGetLastError();
    return la_launch(dt, p, Dk, Dv, pl.C, s, false) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
}

size_t ema_ws_bytes_checked(int B, int T, int C, drs_dtype dt) {
    if (B < 1 || T < 1 || C < 1 || (dt != DRS_F32 && dt != DRS_BF16)) return 0;
    if (!drs::ema_supported(B, T, C, dt == DRS_BF16 ? 2 : 4)) return 0;
    return drs::ema_ws_bytes(B, T, C);
}

int ema_call(const void *x, const void *f, drs_dtype dt, const float *state_in, void *y, float *state_out, int B,
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

DRS_API size_t la_workspace_bytes(int B, int H, int T, int Dk, int Dv, drs_dtype dt, int chunk, unsigned flags) {
    return la_ws_bytes(B, H, T, Dk, Dv, dt, chunk, flags);
}

DRS_API int la_forward(const void *q, const void *k, const void *v, drs_dtype dt, const float *decay,
                       drs_decay mode, const float *state_in, const float *cum_k_in, void *y,
                       float *state_out, float *cum_k_out, int B, int H, int T, int Dk, int Dv, int chunk,
                       unsigned flags, void *workspace, size_t workspace_bytes, void *stream) {
    return la_call(q, k, v, dt, decay, mode, state_in, cum_k_in, y, state_out, cum_k_out, B, H, T, Dk, Dv, chunk,
                   flags, workspace, workspace_bytes, static_cast<hipStream_t>(stream), false);
}

DRS_API size_t la_bidirectional_workspace_bytes(int B, int H, int T, int Dk, int Dv, drs_dtype dt, int chunk,
                                                unsigned flags) {
    if (B < 1 || H < 1 || T < 1 || (dt != DRS_F32 && dt != DRS_BF16)) return 0;
    if (!supported_dim(Dk) || !supported_dim(Dv)) return 0;
    const size_t esize = dt == DRS_BF16 ? 2 : 4;
    return tail_offset(la_ws_bytes(B, H, T, Dk, Dv, dt, chunk, flags)) + (size_t)B * H * T * Dv * esize;
}

DRS_API int la_bidirectional(const void *q, const void *k, const void *v, drs_dtype dt, const float *decay,
                             drs_decay mode, void *y, int B, int H, int T, int Dk, int Dv, int chunk,
                             unsigned flags, void *workspace, size_t workspace_bytes, void *stream) {
    if (flags & DRS_REVERSE) return DRS_ERR_INVALID;
    const size_t need = la_bidirectional_workspace_bytes(B, H, T, Dk, Dv, dt, chunk, flags);
    hipStream_t s = static_cast<hipStream_t>(stream);
    int st = la_call(q, k, v, dt, decay, mode, nullptr, nullptr, y, nullptr, nullptr, B, H, T, Dk, Dv, chunk,
                     flags, workspace, workspace_bytes, s, true);
    if (st != DRS_OK) return st;
    if (!workspace || need == 0 || workspace_bytes < need) return DRS_ERR_WORKSPACE;
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

bool la_bwd_layout(int B, int H, int T, int Dk, int Dv, drs_dtype dt, int chunk, unsigned flags, LABwdLayout *L) {
    if (B < 1 || H < 1 || T < 1 || (dt != DRS_F32 && dt != DRS_BF16)) return false;
    if (!supported_dim(Dk) || !supported_dim(Dv)) return false;
    const unsigned f = flags & kLaForce;
    const size_t a = la_ws_bytes(B, H, T, Dv, Dk, dt, chunk, f), b = la_ws_bytes(B, H, T, Dk, Dv, dt, chunk, f);
    const size_t units = (size_t)B * H, st = round256(units * Dk * Dv * 4), tt = round256(units * T * 4);
    L->scan = 0;
    L->s0t = round256(a > b ? a : b);
    if (L->s0t < 256) L->s0t = 256;      // keep the counters even when no scan needs them
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

DRS_API size_t la_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv, drs_dtype dt, int chunk,
                                           unsigned flags) {
    LABwdLayout L;
    return la_bwd_layout(B, H, T, Dk, Dv, dt, chunk, flags, &L) ? L.total : 0;
}

DRS_API int la_backward(const void *q, const void *k, const void *v, drs_dtype dt, const float *decay,
                        drs_decay mode, const float *state_in, const float *state_out, const void *dy,
                        const float *dstate_out, void *dq, void *dk, void *dv, float *ddecay, float *dstate_in,
                        int B, int H, int T, int Dk, int Dv, int chunk, unsigned flags, void *workspace,
                        size_t workspace_bytes, void *stream) {
    if (!q || !k || !v || !dy || !dq || !dk || !dv) return DRS_ERR_INVALID;
    if (B < 1 || H < 1 || T < 1) return DRS_ERR_INVALID;
    if (dt != DRS_F32 && dt != DRS_BF16) return DRS_ERR_INVALID;
    if (mode != DRS_DECAY_NONE && mode != DRS_DECAY_HEAD && mode != DRS_DECAY_STEP && mode != DRS_DECAY_ELEM)
        return DRS_ERR_INVALID;
    if ((decay == nullptr) != (mode == DRS_DECAY_NONE)) return DRS_ERR_INVALID;
    if (mode == DRS_DECAY_NONE && ddecay) return DRS_ERR_INVALID;
    if (flags & ~(DRS_REVERSE | DRS_NORMALIZE | kLaForce)) return DRS_ERR_INVALID;
    if ((flags & kLaForce) == kLaForce) return DRS_ERR_INVALID;
    if (ddecay && dstate_out && !state_out) return DRS_ERR_INVALID;   // <dS_final, S_final> needs S_final
    const void *outs[] = {dq, dk, dv, ddecay, dstate_in};
    const void *ins[] = {q, k, v, dy, decay, state_in, state_out, dstate_out};
    for (const void *o : outs)
        for (const void *i : ins)
            if (o && o == i) return DRS_ERR_INVALID;
    if (dq == dk || dq == dv || dk == dv) return DRS_ERR_INVALID;
    const void *big[] = {q, k, v, dy, dq, dk, dv};
    for (const void *pp : big)
        if (!aligned16(pp)) return DRS_ERR_INVALID;
    const void *small[] = {decay, state_in, state_out, dstate_out, ddecay, dstate_in};
    for (const void *pp : small)
        if (pp && !aligned4(pp)) return DRS_ERR_INVALID;
    if (workspace && !aligned16(workspace)) return DRS_ERR_INVALID;
    if (flags & DRS_NORMALIZE) return DRS_ERR_UNSUPPORTED;          // the normalised form has no backward here
    if (mode == DRS_DECAY_ELEM) return DRS_ERR_UNSUPPORTED;         // per-channel factors: forward only
    LABwdLayout Lw;
    if (!la_bwd_layout(B, H, T, Dk, Dv, dt, chunk, flags, &Lw)) return DRS_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < Lw.total) return DRS_ERR_WORKSPACE;

    hipStream_t s = static_cast<hipStream_t>(stream);
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
    const drs_decay mback = shifted ? DRS_DECAY_STEP : mode;
    float *ds0 = dstate_in ? (mode == DRS_DECAY_NONE ? dstate_in : reinterpret_cast<float *>(ws + Lw.ds0)) : nullptr;
    const unsigned fwd = (rev ? DRS_REVERSE : 0u) | force, bwd = (rev ? 0u : DRS_REVERSE) | force;
    const bool via32 = ddecay && dt == DRS_BF16;
    void *dq_s = via32 ? static_cast<void *>(ws + Lw.dq32) : dq;
    void *dk_s = via32 ? static_cast<void *>(ws + Lw.dk32) : dk;

    // every check of the three scans first, so that an error leaves nothing enqueued
    int st = la_call(dy, v, k, dt, decay, mode, s0t, nullptr, dq_s, nullptr, nullptr, B, H, T, Dv, Dk, chunk, fwd,
                     workspace, workspace_bytes, s, true, via32);
    if (st == DRS_OK)
        st = la_call(v, dy, q, dt, gback, mback, dsft, nullptr, dk_s, nullptr, nullptr, B, H, T, Dv, Dk, chunk, bwd,
                     workspace, workspace_bytes, s, true, via32);
    if (st == DRS_OK)
        st = la_call(k, q, dy, dt, gback, mback, dstate_out, nullptr, dv, ds0, nullptr, B, H, T, Dk, Dv, chunk, bwd,
                     workspace, workspace_bytes, s, true);
    if (st != DRS_OK) return st;

    (void)hipGetLastError();
    bool ok = true;
    if (s0t) ok = ok && drs::transpose_units_launch(state_in, s0t, units, Dk, Dv, s) == hipSuccess;
    if (dsft) ok = ok && drs::transpose_units_launch(dstate_out, dsft, units, Dk, Dv, s) == hipSuccess;
    if (shifted)
        ok = ok && drs::shift_decay_launch(decay, (int)mode, const_cast<float *>(gback), units, H, T, rev ? 1 : 0, s) ==
                       hipSuccess;
    if (!ok) return DRS_ERR_DEVICE;
    // dq_t = S_t dy_t: the forward scan of v k^T, read by dy
    st = la_call(dy, v, k, dt, decay, mode, s0t, nullptr, dq_s, nullptr, nullptr, B, H, T, Dv, Dk, chunk, fwd,
                 workspace, workspace_bytes, s, false, via32);
    // dk_t = G_t v_t: the opposite-order scan of dy q^T, read by v
    if (st == DRS_OK)
        st = la_call(v, dy, q, dt, gback, mback, dsft, nullptr, dk_s, nullptr, nullptr, B, H, T, Dv, Dk, chunk, bwd,
                     workspace, workspace_bytes, s, false, via32);
    // dv_t = G_t^T k_t: the opposite-order scan of q dy^T, read by k; its final
    // state is the gradient reaching the first visited step
    if (st == DRS_OK)
        st = la_call(k, q, dy, dt, gback, mback, dstate_out, nullptr, dv, ds0, nullptr, B, H, T, Dk, Dv, chunk, bwd,
                     workspace, workspace_bytes, s, false);
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
        // counter 16 of the workspace's first 256 bytes (the scans use 0..3)
        ok = ok && drs::decay_grad_launch(c, decay, (int)mode, dstate_out, state_out, Dk * Dv, ddecay,
                                          reinterpret_cast<float *>(ws + Lw.partial), B, H, T, rev ? 1 : 0,
                                          scale ? ds0 : nullptr, scale ? dstate_in : nullptr,
                                          reinterpret_cast<unsigned *>(ws) + 16, s) == hipSuccess;
    }
    return ok ? DRS_OK : DRS_ERR_DEVICE;
}

DRS_API size_t wkv_workspace_bytes(int B, int T, int C, unsigned flags) {
    if (B < 1 || T < 1 || C < 1) return 0;
    if (flags & ~(kWkvForce | DRS_WKV_OWN_AGGREGATES)) return 0;
    const WkvPath path = wkv_choose(B, T, C, flags);
    if (path == WkvPath::kChain && !drs::wkv_chain_supported(B, T, C)) return 0;
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
    }
    (void)hipGetLastError();
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (path) {
        case WkvPath::kChain: e = drs::wkv_launch_chain(p, s); break;
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
                         const float *dy, float *dw, float *du, float *dk, float *dv, int B, int T, int C,
                         unsigned flags, void *workspace, size_t workspace_bytes, void *stream) {
    if (!w || !u || !k || !v || !dy || !dk || !dv) return DRS_ERR_INVALID;
    if (B < 1 || T < 1 || C < 1) return DRS_ERR_INVALID;
    if (flags) return DRS_ERR_INVALID;
    const void *outs[] = {dw, du, dk, dv};
    const void *ins[] = {w, u, k, v, state_in, dy};
    for (const void *o : outs)
        for (const void *i : ins)
            if (o && o == i) return DRS_ERR_INVALID;
    if (dk == dv || (dw && dw == du)) return DRS_ERR_INVALID;
    const void *ptrs[] = {w, u, k, v, state_in, dy, dw, du, dk, dv};
    for (const void *pp : ptrs)
        if (pp && !aligned4(pp)) return DRS_ERR_INVALID;
    if (workspace && !aligned16(workspace)) return DRS_ERR_INVALID;
    if (B > 65535 || (size_t)T * C * 4 >= ((size_t)1 << 31)) return DRS_ERR_UNSUPPORTED;
    const size_t need = drs::wkv_bwd_ws_bytes(B, T, C);
    if (!workspace || workspace_bytes < need) return DRS_ERR_WORKSPACE;
    drs::WKVBwdParams p = {};
    p.w = w; p.u = u; p.k = k; p.v = v; p.state_in = state_in; p.dy = dy;
    p.dk = dk; p.dv = dv; p.dw = dw; p.du = du;
    p.B = B; p.T = T; p.C = C;
    drs::wkv_bwd_layout(B, T, C, static_cast<char *>(workspace), p);
    (void)hipGetLastError();
    return drs::wkv_launch_bwd(p, static_cast<hipStream_t>(stream)) == hipSuccess ? DRS_OK : DRS_ERR_DEVICE;
}

DRS_API size_t ema_workspace_bytes(int B, int T, int C, drs_dtype dt, unsigned flags) {
    if (flags & ~DRS_REVERSE) return 0;
    return ema_ws_bytes_checked(B, T, C, dt);
}

DRS_API int ema_forward(const void *x, const void *f, drs_dtype dt, const float *state_in, void *y,
                        float *state_out, int B, int T, int C, unsigned flags, void *workspace,
                        size_t workspace_bytes, void *stream) {
    return ema_call(x, f, dt, state_in, y, state_out, B, T, C, flags, workspace, workspace_bytes,
                    static_cast<hipStream_t>(stream), false);
}

// Enough channels to fill the GPU: one fused kernel (x, f read twice, y written
// once); otherwise the forward and reverse calls and an add.
bool ema_bidir_fused(int B, int T, int C) { return drs::ema_walk(B, T, C); }

DRS_API size_t ema_bidirectional_workspace_bytes(int B, int T, int C, drs_dtype dt, unsigned flags) {
    if (flags) return 0;
    if (B < 1 || T < 1 || C < 1 || (dt != DRS_F32 && dt != DRS_BF16)) return 0;
    if (!drs::ema_supported(B, T, C, dt == DRS_BF16 ? 2 : 4)) return 0;
    if (ema_bidir_fused(B, T, C)) return drs::ema_bidir_ws_bytes(B, T, C);
    const size_t esize = dt == DRS_BF16 ? 2 : 4;
    return tail_offset(ema_ws_bytes_checked(B, T, C, dt)) + (size_t)B * T * C * esize;
}

DRS_API int ema_bidirectional(const void *x, const void *f, drs_dtype dt, void *y, int B, int T, int C,
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
        default: return "unknown status";
    }
}

DRS_API int drs_version(void) { return 10200; }

}  // extern "C"
