// wkv.hip -- RWKV-4 WKV forward on gfx950: sequential and time-parallel paths.
//
// Definition (RWKV-LM issue #167, the att_seq recurrence; RWKV-LM discussion
// #189, the exponentially weighted (value, log-scale) pairs): per channel the
// state (aa, bb, pp) stands for the sums aa e^pp (values) and bb e^pp
// (weights).  Token t with key k and value v is read out against the state
// with the bonus u, then absorbed after one step of decay w:
//     m = max(pp, u + k):   y = (aa e^{pp-m} + v e^{u+k-m}) / (bb e^{pp-m} + e^{u+k-m})
//     m'= max(pp + w, k):   aa <- aa e^{pp+w-m'} + v e^{k-m'},  bb likewise,  pp <- m'
// In each max one of the two exponentials is e^0 = 1, so a step costs two
// exp2 and one reciprocal.
//
// Log-scales are kept in log2 units, and pp is held as an anchor plus a step
// count: pp = anchor + n w with one rounding (fma) instead of one rounding
// per step, so a large key that stays the running maximum for many steps
// does not drift.  The value is the same in exact arithmetic.
//
// Sequential path: one lane per (b, c), coalesced [T, C] streaming, the next
// block of PF steps of k and v loaded while the current block is computed.
// Time-parallel path (few channels, long T): T is cut into segments; pass 1
// summarises every segment from the empty state, pass 2 folds the summaries
// of the earlier segments with the segment combine
//     (aa1,bb1,pp1) then (aa2,bb2,pp2) over n2 steps:
//     q = pp1 + n2 w, m = max(q, pp2), aa = aa1 2^{q-m} + aa2 2^{pp2-m}, ...
// and then re-runs its own segment from that carry, writing y.
#include "common.h"
#include "wkv.h"

namespace drs {

struct WKVState {
    float aa, bb, anc, n;   // pp (log2 units) = anc + n * w2
};

__device__ __forceinline__ WKVState wkv_empty() { return WKVState{0.f, 0.f, -1e38f * kLog2e, 0.f}; }

// One token: optional read-out, then absorb.  Branch-free: of the two terms
// in each max-shifted sum the larger keeps weight 1 and the other gets
// 2^-|difference|, picked with selects.
template <bool OUT>
__device__ __forceinline__ float wkv_step(WKVState &s, float w2, float u2, float k, float v) {
    const float k2 = k * kLog2e;
    float y = 0.f;
    if (OUT) {
        const float pp2 = fmaf(s.n, w2, s.anc);
        const float d = pp2 - (u2 + k2);
        const float ex = exp2_fast(-fabsf(d));
        const bool past = d > 0.f;                  // the absorbed sums dominate
        const float num = fmaf(ex, past ? v : s.aa, past ? s.aa : v);
        const float den = fmaf(ex, past ? 1.f : s.bb, past ? s.bb : 1.f);
        y = num * rcp_fast(den);
    }
    const float cand = fmaf(s.n + 1.f, w2, s.anc);   // pp + w, one rounding
    const float d2 = cand - k2;
    const float ex2 = exp2_fast(-fabsf(d2));
    const bool keep = d2 >= 0.f;                      // decayed past stays the scale
    const float aa = fmaf(ex2, keep ? v : s.aa, keep ? s.aa : v);
    const float bb = fmaf(ex2, keep ? 1.f : s.bb, keep ? s.bb : 1.f);
    s.aa = aa;
    s.bb = bb;
    s.anc = keep ? s.anc : k2;
    s.n = keep ? s.n + 1.f : 0.f;
    return y;
}

// Run steps [t0, t1) of one channel; k, v, y point at element (b, 0, c), stride C.
// Whole blocks of PF steps stream without predicates, the next block's loads
// in flight while the current block is computed; the tail runs step by step.
template <bool OUT, int PF>
__device__ __forceinline__ void wkv_run(WKVState &s, float w2, float u2, const float *__restrict__ k,
                                        const float *__restrict__ v, float *__restrict__ y, int t0, int t1,
                                        int C) {
    const int nfull = (t1 - t0) / PF;
    float kc[PF], vc[PF];
    auto load = [&](int tb, float *kd, float *vd) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            kd[i] = __builtin_nontemporal_load(k + (size_t)(tb + i) * C);
            vd[i] = __builtin_nontemporal_load(v + (size_t)(tb + i) * C);
        }
    };
    if (nfull > 0) load(t0, kc, vc);
    for (int blk = 0; blk < nfull; ++blk) {
        const int tb = t0 + blk * PF;
        float kn[PF], vn[PF];
        if (blk + 1 < nfull) load(tb + PF, kn, vn);
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const float yy = wkv_step<OUT>(s, w2, u2, kc[i], vc[i]);
            if (OUT) __builtin_nontemporal_store(yy, y + (size_t)(tb + i) * C);
        }
#pragma unroll
        for (int i = 0; i < PF; ++i) { kc[i] = kn[i]; vc[i] = vn[i]; }
    }
    for (int t = t0 + nfull * PF; t < t1; ++t) {
        const float yy = wkv_step<OUT>(s, w2, u2, k[(size_t)t * C], v[(size_t)t * C]);
        if (OUT) y[(size_t)t * C] = yy;
    }
}

__device__ __forceinline__ WKVState wkv_load_state(const float *st, int B, int C, int b, int c) {
    if (!st) return wkv_empty();
    const size_t i = (size_t)b * C + c, plane = (size_t)B * C;
    return WKVState{st[i], st[plane + i], st[2 * plane + i] * kLog2e, 0.f};
}

__device__ __forceinline__ void wkv_store_state(float *st, const WKVState &s, float w2, int B, int C, int b,
                                                int c) {
    const size_t i = (size_t)b * C + c, plane = (size_t)B * C;
    st[i] = s.aa;
    st[plane + i] = s.bb;
    st[2 * plane + i] = fmaf(s.n, w2, s.anc) * kLn2;
}

constexpr int kWkvBlock = 256;
constexpr int kWkvPF = 32;

__global__ __launch_bounds__(kWkvBlock) void wkv_seq_fwd(WKVParams p) {
    const int c = blockIdx.x * kWkvBlock + threadIdx.x, b = blockIdx.y;
    if (c >= p.C) return;
    const float w2 = p.w[c] * kLog2e, u2 = p.u[c] * kLog2e;
    WKVState s = wkv_load_state(p.state_in, p.B, p.C, b, c);
    const size_t base = (size_t)b * p.T * p.C + c;
    wkv_run<true, kWkvPF>(s, w2, u2, p.k + base, p.v + base, p.y + base, 0, p.T, p.C);
    if (p.state_out) wkv_store_state(p.state_out, s, w2, p.B, p.C, b, c);
}

// Workspace: plane-major [nseg + 1][3][B][C]; slot 0 holds the initial state
// (log2 scale, n = 0), slot 1 + j the summary of segment j (log2 scale).
__device__ __forceinline__ float *ws_slot(const WKVParams &p, int slot) {
    return p.ws + (size_t)slot * 3 * p.B * p.C;
}

__global__ __launch_bounds__(kWkvBlock) void wkv_seg_summary(WKVParams p) {
    const int c = blockIdx.x * kWkvBlock + threadIdx.x, b = blockIdx.y, j = blockIdx.z;
    if (c >= p.C) return;
    const float w2 = p.w[c] * kLog2e, u2 = p.u[c] * kLog2e;
    const size_t i = (size_t)b * p.C + c, plane = (size_t)p.B * p.C;
    if (j == 0) {   // snapshot the carried state, so state_out may alias state_in
        const WKVState s0 = wkv_load_state(p.state_in, p.B, p.C, b, c);
        float *d = ws_slot(p, 0);
        d[i] = s0.aa;
        d[plane + i] = s0.bb;
        d[2 * plane + i] = s0.anc;
    }
    if (j == p.nseg - 1) return;   // the last summary is never needed
    const int t0 = j * p.seg_len, t1 = min(p.T, t0 + p.seg_len);
    WKVState s = wkv_empty();
    const size_t base = (size_t)b * p.T * p.C + c;
    wkv_run<false, kWkvPF>(s, w2, u2, p.k + base, p.v + base, nullptr, t0, t1, p.C);
    float *d = ws_slot(p, 1 + j);
    d[i] = s.aa;
    d[plane + i] = s.bb;
    d[2 * plane + i] = fmaf(s.n, w2, s.anc);
}

__global__ __launch_bounds__(kWkvBlock) void wkv_seg_output(WKVParams p) {
    const int c = blockIdx.x * kWkvBlock + threadIdx.x, b = blockIdx.y, j = blockIdx.z;
    if (c >= p.C) return;
    const float w2 = p.w[c] * kLog2e, u2 = p.u[c] * kLog2e;
    const size_t i = (size_t)b * p.C + c, plane = (size_t)p.B * p.C;
    const float *s0 = ws_slot(p, 0);
    float aa = s0[i], bb = s0[plane + i], pp = s0[2 * plane + i];
    const float span_w = (float)p.seg_len * w2;
    for (int jj = 0; jj < j; ++jj) {   // fold the summaries of the earlier segments
        const float *sm = ws_slot(p, 1 + jj);
        const float a2 = sm[i], b2 = sm[plane + i], p2 = sm[2 * plane + i];
        const float q = pp + span_w;
        const float m = fmaxf(q, p2);
        const float e1 = exp2_fast(q - m), e2 = exp2_fast(p2 - m);
        aa = fmaf(aa, e1, a2 * e2);
        bb = fmaf(bb, e1, b2 * e2);
        pp = m;
    }
    WKVState s{aa, bb, pp, 0.f};
    const int t0 = j * p.seg_len, t1 = min(p.T, t0 + p.seg_len);
    const size_t base = (size_t)b * p.T * p.C + c;
    wkv_run<true, kWkvPF>(s, w2, u2, p.k + base, p.v + base, p.y + base, t0, t1, p.C);
    if (j == p.nseg - 1 && p.state_out) wkv_store_state(p.state_out, s, w2, p.B, p.C, b, c);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

// Segment plan of the time-parallel path: enough (segment, channel) lanes to
// give every SIMD of the chip a few waves, segments of at least 64 steps.
void wkv_scan_plan(int B, int T, int C, int *seg_len, int *nseg) {
    const long lanes = (long)B * C;
    const long target = 1L << 17;   // ~2048 waves
    long s = (target + lanes - 1) / lanes;
    const long smax = (T + 63) / 64;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    long L = (T + s - 1) / s;
    L = (L + 15) / 16 * 16;
    if ((T + L - 1) / L > 65535) L = (T + 65534) / 65535;   // grid z limit
    *seg_len = (int)L;
    *nseg = (int)((T + L - 1) / L);
}

bool wkv_use_scan(int B, int T, int C) {
    // the sequential kernel already has >= ~1024 waves of independent channels
    return (long)B * C < 32768L && T >= 256;
}

hipError_t wkv_launch_seq(const WKVParams &p, hipStream_t stream) {
    dim3 grid((p.C + kWkvBlock - 1) / kWkvBlock, p.B);
    hipLaunchKernelGGL(wkv_seq_fwd, grid, dim3(kWkvBlock), 0, stream, p);
    return hipGetLastError();
}

hipError_t wkv_launch_scan(const WKVParams &p, hipStream_t stream) {
    dim3 grid((p.C + kWkvBlock - 1) / kWkvBlock, p.B, p.nseg);
    hipLaunchKernelGGL(wkv_seg_summary, grid, dim3(kWkvBlock), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(wkv_seg_output, grid, dim3(kWkvBlock), 0, stream, p);
    return hipGetLastError();
}

}  // namespace drs
