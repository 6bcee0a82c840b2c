// wkv_bwd.hip -- backward of the RWKV-4 WKV recurrence on gfx950.
//
// RWKV-LM discussion #189 remarks that the gradient of the WKV sums is itself
// a set of cumulative sums.  In the linear form of the recurrence (the sums
// A_t, B_t of the earlier tokens that the log-scale state stands for),
//     y_t = (A_t + e^{u+k_t} v_t) / D_t,   D_t = B_t + e^{u+k_t},
// the gradients reaching A_t and B_t obey the reverse recurrences
//     Abar_t = dy_t / D_t + e^w Abar_{t+1},   Bbar_t = -dy_t y_t / D_t + e^w Bbar_{t+1},
// and
//     dk_t = e^{u+k_t} dy_t (v_t - y_t) / D_t + e^{k_t} (v_t Abar_{t+1} + Bbar_{t+1})
//     dv_t = e^{u+k_t} dy_t / D_t + e^{k_t} Abar_{t+1}
//     du   = sum_t e^{u+k_t} dy_t (v_t - y_t) / D_t
//     dw   = sum_t dy_t (A'_t - y_t B'_t) / D_t,  with A'_{t+1} = e^w (A_t + A'_t)
// (A' = dA/dw, likewise B').  These are first-order linear recurrences, so a
// span of steps has a summary (its sums from the empty state, the scale as an
// anchor plus a step count, and for A', B' the w-derivative of those sums), and
// consecutive spans combine exactly as the forward kernel's spans do; decaying
// (A, A') over n steps turns A' into e^{nw} (A' + n A).
//
// Two kernels, one lane per channel, 4 waves per 64 channels of a batch row, each
// wave owning 16 steps of every 64-step block:
//   wkv_bwd_ckpt (forward sweep): every wave summarises its steps (state, A',
//     B') from the empty state; one wave per block (rotating) folds the block's
//     summaries into the carried state and stores it as the checkpoint of the next
//     block.  k and v are read once.
//   wkv_bwd_rev (blocks from the end): each wave gets its entering state from the
//     block checkpoint and the summaries of the waves before it, rebuilds its
//     outputs and log2 denominators in registers (adding its terms of du and dw),
//     summarises its reverse sums (Abar, Bbar) from the empty state, gets the
//     reverse sums entering from the right (the later block's, then the summaries
//     of the later waves), and runs its steps backward writing dk and dv.  The
//     reverse sums are kept on an anchored log2-scale like the state, so that every
//     exponential formed has a non-positive argument up to rounding: e^{u+k}/D <= 1
//     and e^{k} Abar is bounded because D_{t'} contains the decayed term of token t.
// The per-row sums of du and dw go to the workspace and are added over the
// batch in a fixed order.
#include <type_traits>

#include "common.h"
#include "wkv.h"

namespace drs {

namespace {

// Precision: the log2-scales reach ~90 with keys of +-60, where one fp32
// rounding already costs ~4e-6 relative in the exponential formed from a
// difference of two of them, and the gradients subtract nearly equal sums
// (A' - y B', v Abar + Bbar), which fp32 copies of y would spoil.  So the
// scales, the sums, the checkpoints and the rebuilt outputs and denominators are
// fp64; each exponential is the fp32 exp2 of a difference already formed in
// fp64 (an argument <= 0 of modest size).

struct Fwd {
    double aa, bb, anc, ap, bp, du, dw;   // state (log2-scale anc + n w2), A', B', gradient sums
    float n;
};

// One step forward: returns y_t and writes log2 D_t.  With DERIV it also carries
// A', B' and adds the step's terms of du and dw; without, it only rebuilds y and D.
template <bool DERIV>
__device__ __forceinline__ double fwd_step(Fwd &s, double w2, double u2, float k, float v, float dy, double &lden) {
    const double k2 = (double)k * (double)kLog2e;
    const double pp2 = fma((double)s.n, w2, s.anc);
    const double d = pp2 - (u2 + k2);
    const double ex = (double)exp2_fast(-(float)fabs(d));
    const bool past = d > 0.0;
    const double e_pp = past ? 1.0 : ex, e_cur = past ? ex : 1.0;   // 2^{pp-m}, 2^{u+k-m}
    const double den = fma(e_pp, s.bb, e_cur);                      // D / 2^m
    const double num = fma(e_pp, s.aa, e_cur * (double)v);
    // 1/den: the fp32 reciprocal (~2^-23) refined by two Newton steps in fp64
    // (~2^-46, then full precision), far shorter than an IEEE fp64 division
    double inv = (double)rcp_fast((float)den);
    inv = inv * fma(-den, inv, 2.0);
    inv = inv * fma(-den, inv, 2.0);
    const double y = num * inv;
    if constexpr (DERIV) {
        const double g = (double)dy * inv;
        s.du = fma(e_cur * g, (double)v - y, s.du);
        s.dw = fma(e_pp * g, fma(-y, s.bp, s.ap), s.dw);
    }
    lden = (past ? pp2 : u2 + k2) + (double)__log2f((float)den);
    // absorb the token after one step of decay
    const double cand = fma((double)s.n + 1.0, w2, s.anc);
    const double d2 = cand - k2;
    const double ex2 = (double)exp2_fast(-(float)fabs(d2));
    const bool keep = d2 >= 0.0;
    const double f1 = keep ? 1.0 : ex2, f2 = keep ? ex2 : 1.0;
    if constexpr (DERIV) {
        s.ap = f1 * (s.aa + s.ap);
        s.bp = f1 * (s.bb + s.bp);
    }
    s.aa = fma(f1, s.aa, f2 * (double)v);
    s.bb = fma(f1, s.bb, f2);
    s.anc = keep ? s.anc : k2;
    s.n = keep ? s.n + 1.f : 0.f;
    return y;
}

struct Bwd {
    double ab, bb, anc;    // Abar, Bbar scaled by 2^{anc + n w2}
    float n;
};

__device__ __forceinline__ void bwd_step(Bwd &s, double w2, double u2, float k, float v, double y, float dy,
                                         double lden, float &dk, float &dv) {
    const double k2 = (double)k * (double)kLog2e;
    const double z2 = fma((double)s.n, w2, s.anc);
    const double ec = (double)exp2_fast((float)(u2 + k2 - lden));   // e^{u+k} / D
    const double ez = (double)exp2_fast((float)(k2 + z2));          // e^{k} times the scale of (Abar, Bbar)_{t+1}
    const double vv = v, yy = y, gg = dy;
    dk = (float)fma(ec * gg, vv - yy, ez * fma(vv, s.ab, s.bb));
    dv = (float)fma(ec, gg, ez * s.ab);
    // (Abar, Bbar)_t = (dy, -dy y) / D + e^w (Abar, Bbar)_{t+1}
    const double cand = fma((double)s.n + 1.0, w2, s.anc);
    const double d3 = cand + lden;                                  // log2 of the decayed part over 1/D
    const double ex3 = (double)exp2_fast(-(float)fabs(d3));
    const bool keep = d3 >= 0.0;
    const double g1 = keep ? 1.0 : ex3, g2 = keep ? ex3 : 1.0;
    s.ab = fma(g1, s.ab, g2 * gg);
    s.bb = fma(g1, s.bb, -g2 * gg * yy);
    s.anc = keep ? s.anc : -lden;
    s.n = keep ? s.n + 1.f : 0.f;
}

// Summaries and combines.  A forward summary is a Fwd state (du, dw unused) run
// from the empty state; a reverse summary a Bwd state run backward from empty.
__device__ __forceinline__ Fwd fwd_empty() { return Fwd{0.0, 0.0, -1e38 * (double)kLog2e, 0.0, 0.0, 0.0, 0.0, 0.f}; }
__device__ __forceinline__ Bwd bwd_empty() { return Bwd{0.0, 0.0, -1e38 * (double)kLog2e, 0.f}; }

// Absorb one token into a forward summary (the absorbing half of fwd_step).
__device__ __forceinline__ void fwd_absorb(Fwd &s, double w2, float k, float v) {
    const double k2 = (double)k * (double)kLog2e;
    const double cand = fma((double)s.n + 1.0, w2, s.anc);
    const double d2 = cand - k2;
    const double ex2 = (double)exp2_fast(-(float)fabs(d2));
    const bool keep = d2 >= 0.0;
    const double f1 = keep ? 1.0 : ex2, f2 = keep ? ex2 : 1.0;
    s.ap = f1 * (s.aa + s.ap);
    s.bp = f1 * (s.bb + s.bp);
    s.aa = fma(f1, s.aa, f2 * (double)v);
    s.bb = fma(f1, s.bb, f2);
    s.anc = keep ? s.anc : k2;
    s.n = keep ? s.n + 1.f : 0.f;
}

// One step of the reverse sums without the outputs (the update half of bwd_step).
__device__ __forceinline__ void bwd_absorb(Bwd &s, double w2, double y, float dy, double lden) {
    const double cand = fma((double)s.n + 1.0, w2, s.anc);
    const double d3 = cand + lden;
    const double ex3 = (double)exp2_fast(-(float)fabs(d3));
    const bool keep = d3 >= 0.0;
    const double g1 = keep ? 1.0 : ex3, g2 = keep ? ex3 : 1.0, gg = dy;
    s.ab = fma(g1, s.ab, g2 * gg);
    s.bb = fma(g1, s.bb, -g2 * gg * y);
    s.anc = keep ? s.anc : -lden;
    s.n = keep ? s.n + 1.f : 0.f;
}

// x, then a span y of n2 steps (in the recurrence's own direction).  The larger
// decayed scale keeps its anchor and count exactly; the derivative of the decayed
// x part gains n2 times its sums.
__device__ __forceinline__ Fwd fwd_combine(const Fwd &x, const Fwd &y, float n2, double w2) {
    const float xn = x.n + n2;
    const double d = fma((double)(xn - y.n), w2, x.anc - y.anc);
    const bool xbig = d >= 0.0;
    const double ex = (double)exp2_fast(-(float)fabs(d));
    const double e1 = xbig ? 1.0 : ex, e2 = xbig ? ex : 1.0, m = (double)n2;
    Fwd r;
    r.aa = fma(x.aa, e1, y.aa * e2);
    r.bb = fma(x.bb, e1, y.bb * e2);
    r.ap = fma(fma(m, x.aa, x.ap), e1, y.ap * e2);
    r.bp = fma(fma(m, x.bb, x.bp), e1, y.bp * e2);
    r.anc = xbig ? x.anc : y.anc;
    r.n = xbig ? xn : y.n;
    r.du = 0.0;
    r.dw = 0.0;
    return r;
}
__device__ __forceinline__ Bwd bwd_combine(const Bwd &x, const Bwd &y, float n2, double w2) {
    const float xn = x.n + n2;
    const double d = fma((double)(xn - y.n), w2, x.anc - y.anc);
    const bool xbig = d >= 0.0;
    const double ex = (double)exp2_fast(-(float)fabs(d));
    const double e1 = xbig ? 1.0 : ex, e2 = xbig ? ex : 1.0;
    return Bwd{fma(x.ab, e1, y.ab * e2), fma(x.bb, e1, y.bb * e2), xbig ? x.anc : y.anc, xbig ? xn : y.n};
}

// Fixed-reference form of a span (the fast path of the reverse walk).  Within a
// span of at most kBwdSub steps, every sum is measured against one reference line
// 2^(p0 + t w2) (t counted from the span start): token i then has the height
// h_i = k2_i - (i + 1) w2, and
//     A_t = 2^(p0 + t w2) alpha_t,  alpha_t = alpha_0 + sum_{i<t} 2^(h_i - p0) v_i,
//     A'_t = 2^(p0 + t w2) (t alpha_t + alpha'_t),  alpha'_t = alpha'_0 - sum_{i<t} (i+1) 2^(h_i - p0) v_i,
//     e^{u+k_t} = 2^(p0 + t w2) c_t,  c_t = 2^(h_t - p0) 2^(w2 + u2),
// so y_t and D_t / 2^(p0 + t w2) = beta_t + c_t need no rescaling, and the reverse
// sums on the line 2^-(p0 + t w2) are plain sums from the right of dy_t / den_t.
// With p0 at least the largest height, every term is at most 1; the path is taken
// when the heights of a wave's span (and w2 + u2) spread over less than
// kFastSpread, which keeps every term that matters a normal fp64 number.
constexpr double kFastSpread = 900.0;

// 2^x for fp64 x: the fraction on the fp32 unit (relative error ~1e-7), the
// integer part exact; arguments below -1100 give 0.
__device__ __forceinline__ double exp2_d(double x) {
    x = fmax(x, -1100.0);
    const double fl = floor(x);
    return ldexp((double)exp2_fast((float)(x - fl)), (int)fl);
}

// Reverse sums of the fixed-reference form (plain sums of dy / den) are not
// normalised: they reach ~2^100 where a span's early denominators are tiny next to
// its reference line.  The combines weight the smaller-scale side by an fp32
// exp2 of the scale difference, which assumes the larger scale also carries the
// larger value; so such a state is rescaled by a power of two (exactly) to
// max(|Abar|, |Bbar|) in [0.5, 1) before it is exchanged.
__device__ __forceinline__ Bwd bwd_norm(Bwd r) {
    const double m = fmax(fabs(r.ab), fabs(r.bb));
    if (m > 0.0) {
        const int e = __builtin_amdgcn_frexp_exp(m);
        r.ab = ldexp(r.ab, -e);
        r.bb = ldexp(r.bb, -e);
        r.anc += (double)e;
    }
    return r;
}

// 1/x: the fp64 reciprocal estimate refined by two Newton steps.
__device__ __forceinline__ double rcp_d(double x) {
    double r = __builtin_amdgcn_rcp(x);
    r = r * fma(-x, r, 2.0);
    return r * fma(-x, r, 2.0);
}

constexpr int kBwdWaves = 4;
constexpr int kBwdSub = 16;                           // steps per wave per block
constexpr int kBwdBlock = kBwdWaves * kBwdSub;        // checkpoint spacing
constexpr int kCkptFields = 6;                        // aa, bb, anchor, A', B', count

// Checkpoints [b][block][field][c] (doubles): the state entering every block.
struct Ckpt {
    double *base;
    int nblk, C;
    __device__ double *at(int b, int blk, int field, int c) const {
        return base + (((size_t)b * nblk + blk) * kCkptFields + field) * C + c;
    }
};
// Block-indexed planes of doubles [b][block][field][c] (split mode: summaries, carries).
struct Planes {
    double *base;
    int nblk, C, fields;
    __device__ double *at(int b, int blk, int field, int c) const {
        return base + (((size_t)b * nblk + blk) * fields + field) * C + c;
    }
};
__device__ __forceinline__ void fwd_store(const Planes &pl, int b, int blk, int c, const Fwd &s) {
    *pl.at(b, blk, 0, c) = s.aa;
    *pl.at(b, blk, 1, c) = s.bb;
    *pl.at(b, blk, 2, c) = s.anc;
    *pl.at(b, blk, 3, c) = s.ap;
    *pl.at(b, blk, 4, c) = s.bp;
    *pl.at(b, blk, 5, c) = (double)s.n;
}
__device__ __forceinline__ Fwd fwd_load(const Planes &pl, int b, int blk, int c) {
    return Fwd{*pl.at(b, blk, 0, c), *pl.at(b, blk, 1, c), *pl.at(b, blk, 2, c), *pl.at(b, blk, 3, c),
               *pl.at(b, blk, 4, c), 0.0, 0.0, (float)*pl.at(b, blk, 5, c)};
}
__device__ __forceinline__ void bwd_store(const Planes &pl, int b, int blk, int c, const Bwd &r) {
    *pl.at(b, blk, 0, c) = r.ab;
    *pl.at(b, blk, 1, c) = r.bb;
    *pl.at(b, blk, 2, c) = r.anc;
    *pl.at(b, blk, 3, c) = (double)r.n;
}
__device__ __forceinline__ Bwd bwd_load(const Planes &pl, int b, int blk, int c) {
    return Bwd{*pl.at(b, blk, 0, c), *pl.at(b, blk, 1, c), *pl.at(b, blk, 2, c), (float)*pl.at(b, blk, 3, c)};
}

__device__ __forceinline__ void ckpt_store(const Ckpt &ck, int b, int blk, int c, const Fwd &s) {
    *ck.at(b, blk, 0, c) = s.aa;
    *ck.at(b, blk, 1, c) = s.bb;
    *ck.at(b, blk, 2, c) = s.anc;
    *ck.at(b, blk, 3, c) = s.ap;
    *ck.at(b, blk, 4, c) = s.bp;
    *ck.at(b, blk, 5, c) = (double)s.n;
}

// Forward sweep: checkpoints.  Wave j summarises steps 16j..16j+15 of each block;
// the fold of block blk is done by wave blk % 4, after the block's barrier, into the
// carried state in LDS (summaries double-buffered by block parity).
__global__ __launch_bounds__(64 * kBwdWaves, kBwdWaves / 2) void wkv_bwd_ckpt(WKVBwdParams p) {
    __shared__ Fwd sums[2][kBwdWaves][64];
    __shared__ Fwd carry[64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ncblk = (p.C + 63) / 64, units = p.B * ncblk;
    const int unit = p.split ? (int)(blockIdx.x % (unsigned)units) : (int)blockIdx.x;
    const int b = unit / ncblk, c = (unit - b * ncblk) * 64 + lane;
    const int T = p.T, C = p.C, cc = min(c, C - 1);
    const int nblk = (T + kBwdBlock - 1) / kBwdBlock;
    const double w2 = (double)p.w[cc] * (double)kLog2e;
    const Ckpt ck{p.ckpt, nblk, C};
    const size_t row0 = (size_t)b * T * C;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + row0, T * C * 4);
    const unsigned voff = c < C ? (unsigned)(c * 4) : kOutOfRange;
    auto soff = [&](int t) { return (unsigned)(min(t, T - 1) * C * 4); };
    if (p.split) {
        // a segment of blocks, each block's summary from the empty state (the
        // checkpoints follow from a per-channel scan of these summaries)
        const int seg = (int)(blockIdx.x / (unsigned)units), j0 = seg * p.per, j1 = min(nblk, j0 + p.per);
        float kr[kBwdSub], vr[kBwdSub];
#pragma unroll
        for (int i = 0; i < kBwdSub; ++i) {
            kr[i] = buffer_load4s<kNonTemporal>(rk, voff, soff(j0 * kBwdBlock + wv * kBwdSub + i));
            vr[i] = buffer_load4s<kNonTemporal>(rv, voff, soff(j0 * kBwdBlock + wv * kBwdSub + i));
        }
        for (int blk = j0; blk < j1; ++blk) {
            auto span = [&](int j) { return min(max(T - (blk * kBwdBlock + j * kBwdSub), 0), kBwdSub); };
            const int t0 = blk * kBwdBlock + wv * kBwdSub, n = span(wv);
            const unsigned vn = blk + 1 < j1 ? voff : kOutOfRange;
            Fwd s = fwd_empty();
#pragma unroll
            for (int i = 0; i < kBwdSub; ++i) {
                if (i < n) fwd_absorb(s, w2, kr[i], vr[i]);
                kr[i] = buffer_load4s<kNonTemporal>(rk, vn, soff(t0 + kBwdBlock + i));
                vr[i] = buffer_load4s<kNonTemporal>(rv, vn, soff(t0 + kBwdBlock + i));
            }
            sums[blk & 1][wv][lane] = s;
            __syncthreads();
            if (wv == blk % kBwdWaves && c < C) {
                Fwd f = fwd_empty();
#pragma unroll
                for (int j = 0; j < kBwdWaves; ++j) f = fwd_combine(f, sums[blk & 1][j][lane], (float)span(j), w2);
                fwd_store(Planes{p.bsum, nblk, C, kCkptFields}, b, blk, c, f);
            }
        }
        return;
    }
    if (wv == 0) {
        Fwd s0 = fwd_empty();
        if (p.state_in) {
            const size_t i = (size_t)b * C + cc, plane = (size_t)p.B * C;
            s0.aa = p.state_in[i];
            s0.bb = p.state_in[plane + i];
            s0.anc = (double)p.state_in[2 * plane + i] * (double)kLog2e;
        }
        carry[lane] = s0;
        if (c < C) ckpt_store(ck, b, 0, c, s0);
    }
    float kr[kBwdSub], vr[kBwdSub];
#pragma unroll
    for (int i = 0; i < kBwdSub; ++i) {
        kr[i] = buffer_load4s<kNonTemporal>(rk, voff, soff(wv * kBwdSub + i));
        vr[i] = buffer_load4s<kNonTemporal>(rv, voff, soff(wv * kBwdSub + i));
    }
    for (int blk = 0; blk < nblk; ++blk) {
        const int t0 = blk * kBwdBlock + wv * kBwdSub, n = min(max(T - t0, 0), kBwdSub);
        const unsigned vn = blk + 1 < nblk ? voff : kOutOfRange;
        Fwd s = fwd_empty();
#pragma unroll
        for (int i = 0; i < kBwdSub; ++i) {
            if (i < n) fwd_absorb(s, w2, kr[i], vr[i]);
            kr[i] = buffer_load4s<kNonTemporal>(rk, vn, soff(t0 + kBwdBlock + i));
            vr[i] = buffer_load4s<kNonTemporal>(rv, vn, soff(t0 + kBwdBlock + i));
        }
        sums[blk & 1][wv][lane] = s;
        __syncthreads();
        if (wv == blk % kBwdWaves && blk + 1 < nblk) {   // the next block's entering state
            Fwd f = carry[lane];
#pragma unroll
            for (int j = 0; j < kBwdWaves; ++j) f = fwd_combine(f, sums[blk & 1][j][lane], (float)kBwdSub, w2);
            carry[lane] = f;
            if (c < C) ckpt_store(ck, b, blk + 1, c, f);
        }
    }
}

// Split mode: per channel, the checkpoints from the block summaries (blocks in
// order from the initial state), and the reverse sums entering every block from
// the reverse block summaries (blocks from the end).
__global__ __launch_bounds__(256) void wkv_bwd_fscan(WKVBwdParams p) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)p.B * p.C) return;
    const int b = (int)(i / p.C), c = (int)(i - (long)b * p.C), T = p.T, C = p.C;
    const int nblk = (T + kBwdBlock - 1) / kBwdBlock;
    const double w2 = (double)p.w[c] * (double)kLog2e;
    const Ckpt ck{p.ckpt, nblk, C};
    const Planes sm{p.bsum, nblk, C, kCkptFields};
    Fwd f = fwd_empty();
    if (p.state_in) {
        const size_t j = (size_t)b * C + c, plane = (size_t)p.B * C;
        f.aa = p.state_in[j];
        f.bb = p.state_in[plane + j];
        f.anc = (double)p.state_in[2 * plane + j] * (double)kLog2e;
    }
    for (int blk = 0; blk < nblk; ++blk) {
        ckpt_store(ck, b, blk, c, f);
        if (blk + 1 < nblk) f = fwd_combine(f, fwd_load(sm, b, blk, c), (float)kBwdBlock, w2);
    }
}

__global__ __launch_bounds__(256) void wkv_bwd_rscan(WKVBwdParams p) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)p.B * p.C) return;
    const int b = (int)(i / p.C), c = (int)(i - (long)b * p.C), T = p.T, C = p.C;
    const int nblk = (T + kBwdBlock - 1) / kBwdBlock;
    const double w2 = (double)p.w[c] * (double)kLog2e;
    const Planes sm{p.bsum, nblk, C, 4}, car{p.rcar, nblk, C, 4};
    Bwd r = bwd_empty();
    for (int blk = nblk - 1; blk >= 0; --blk) {
        bwd_store(car, b, blk, c, r);
        if (blk > 0) r = bwd_combine(r, bwd_load(sm, b, blk, c), (float)min(kBwdBlock, T - blk * kBwdBlock), w2);
    }
}

// Reverse walk.  Registers hold the block's k, v, dy with step i in slot i (REV =
// false) or in slot 15 - i (REV = true); each slot is reloaded with the previous
// block's step as soon as the backward run has used it, in the slot order of the
// other parity, so the loads complete in the order the next block's forward run
// needs them.
__global__ __launch_bounds__(64 * kBwdWaves, kBwdWaves / 2) void wkv_bwd_rev(WKVBwdParams p) {
    __shared__ Fwd fsum[kBwdWaves - 1][64];
    __shared__ Bwd rsum[kBwdWaves][64];
    __shared__ Bwd rcarry[2][64];
    __shared__ double red[2][kBwdWaves][64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // walks: one workgroup per 64 channels; split mode: one per (64 channels, block),
    // pass 1 storing the block's reverse summary, pass 2 its gradients
    const int ncblk = (p.C + 63) / 64, units = p.B * ncblk;
    const int unit = p.split ? (int)(blockIdx.x % (unsigned)units) : (int)blockIdx.x;
    const int b = unit / ncblk, c = (unit - b * ncblk) * 64 + lane;
    const int T = p.T, C = p.C, cc = min(c, C - 1);
    const int nblk = (T + kBwdBlock - 1) / kBwdBlock;
    // blocks visited: [last, first], from the end
    const int seg = p.split ? (int)(blockIdx.x / (unsigned)units) : 0;
    const int last = p.split ? seg * p.per : 0, myblk = p.split ? min(nblk, last + p.per) - 1 : nblk - 1;
    const double w2 = (double)p.w[cc] * (double)kLog2e, u2 = (double)p.u[cc] * (double)kLog2e;
    const double wu2 = w2 + u2, cwu = exp2_d(wu2);   // 2^(w2 + u2): c_t over 2^(h_t - p0)
    const Ckpt ck{p.ckpt, nblk, C};
    const size_t row0 = (size_t)b * T * C;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dy + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rdk = make_rsrc(p.dk + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rdv = make_rsrc(p.dv + row0, T * C * 4);
    const unsigned voff = c < C ? (unsigned)(c * 4) : kOutOfRange;
    auto soff = [&](int t) { return (unsigned)(min(t, T - 1) * C * 4); };
    auto span = [&](int blk, int j) { return min(max(T - (blk * kBwdBlock + j * kBwdSub), 0), kBwdSub); };

    float kr[kBwdSub], vr[kBwdSub], gr[kBwdSub];
    double du = 0.0, dw = 0.0;
    Bwd rfirst = bwd_empty();
    if (wv == 0)
        rcarry[myblk & 1][lane] = p.split == 2 ? bwd_load(Planes{p.rcar, nblk, C, 4}, b, myblk, cc) : bwd_empty();
    // the first block visited, in the memory-operation order of the reloads (two
    // stores, dropped as out of range, then three loads per step)
    {
        const int t0 = myblk * kBwdBlock + wv * kBwdSub;
#pragma unroll
        for (int i = 0; i < kBwdSub; ++i) {
            buffer_store4s(rdk, kOutOfRange, (unsigned)(i * 4), 0.f);
            buffer_store4s(rdv, kOutOfRange, (unsigned)(i * 4), 0.f);
            kr[i] = buffer_load4s(rk, voff, soff(t0 + i));
            vr[i] = buffer_load4s(rv, voff, soff(t0 + i));
            gr[i] = buffer_load4s(rd, voff, soff(t0 + i));
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    auto block = [&](int blk, auto rev_tag) {
        constexpr bool REV = decltype(rev_tag)::value;
        auto slot = [](int i) { return REV ? kBwdSub - 1 - i : i; };
        const int t0 = blk * kBwdBlock + wv * kBwdSub, n = span(blk, wv);
        // the block's entering state (checkpoint)
        Fwd e{*ck.at(b, blk, 0, cc), *ck.at(b, blk, 1, cc), *ck.at(b, blk, 2, cc), *ck.at(b, blk, 3, cc),
              *ck.at(b, blk, 4, cc), 0.0, 0.0, (float)*ck.at(b, blk, 5, cc)};
        // heights of this wave's tokens over its reference line; the fixed-reference
        // form when they (and w2 + u2) stay within kFastSpread for every lane
        auto height = [&](int i) { return fma(-(double)(i + 1), w2, (double)kr[slot(i)] * (double)kLog2e); };
        double hmax = -1e300, hmin = 1e300;
#pragma unroll
        for (int i = 0; i < kBwdSub; ++i)
            if (i < n) {
                const double h = height(i);
                hmax = fmax(hmax, h);
                hmin = fmin(hmin, h);
            }
        const bool fast = __all(n == 0 || hmax - hmin + fabs(wu2) < kFastSpread);
        // forward summaries of this wave's steps, for the later waves
        if (wv < kBwdWaves - 1) {
            Fwd s = fwd_empty();
            if (fast) {
                if (n > 0) {
                    double al = 0.0, be = 0.0, alp = 0.0, bep = 0.0;
#pragma unroll
                    for (int i = 0; i < kBwdSub; ++i)
                        if (i < n) {
                            const double ee = exp2_d(height(i) - hmax), ev = ee * (double)vr[slot(i)];
                            al += ev;
                            be += ee;
                            alp = fma(-(double)(i + 1), ev, alp);
                            bep = fma(-(double)(i + 1), ee, bep);
                        }
                    // at the span end t = n: scale 2^(hmax + n w2), derivative n alpha + alpha'
                    s = Fwd{al, be, fma((double)n, w2, hmax), fma((double)n, al, alp), fma((double)n, be, bep),
                            0.0, 0.0, 0.f};
                }
            } else {
#pragma unroll
                for (int i = 0; i < kBwdSub; ++i)
                    if (i < n) fwd_absorb(s, w2, kr[slot(i)], vr[slot(i)]);
            }
            fsum[wv][lane] = s;
        }
        __syncthreads();
        for (int j = 0; j < wv; ++j) e = fwd_combine(e, fsum[j][lane], (float)kBwdSub, w2);
        // outputs of this wave's steps with, fixed-reference form: 1/den (den = D over
        // the reference line), else log2 D; and their du, dw terms
        double yb[kBwdSub], lb[kBwdSub];
        double p0 = 0.0, rl = 0.0, rs = 0.0;   // fixed-reference form: the line, reverse local sums
        if (fast) {
            const double ppe = fma((double)e.n, w2, e.anc);
            p0 = fmax(hmax, ppe);
            const double s0 = exp2_d(ppe - p0);
            double al = e.aa * s0, be = e.bb * s0, alp = e.ap * s0, bep = e.bp * s0;
#pragma unroll
            for (int i = 0; i < kBwdSub; ++i) {
                yb[i] = 0.0;
                lb[i] = 0.0;
                if (i < n) {
                    const double vv = vr[slot(i)], gg = gr[slot(i)];
                    const double ee = exp2_d(height(i) - p0), ct = ee * cwu;
                    // y = (alpha + c v) / (beta + c), written as v minus a correction so that
                    // y = v exactly when the sums are empty
                    const double inv = rcp_d(be + ct), vmy = fma(be, vv, -al) * inv, y = vv - vmy, g = gg * inv;
                    du = fma(ct * g, vmy, du);
                    dw = fma(g, fma(-y, fma((double)i, be, bep), fma((double)i, al, alp)), dw);
                    yb[i] = y;
                    lb[i] = inv;
                    rl += g;
                    rs = fma(-g, y, rs);
                    const double ev = ee * vv;
                    al += ev;
                    be += ee;
                    alp = fma(-(double)(i + 1), ev, alp);
                    bep = fma(-(double)(i + 1), ee, bep);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < kBwdSub; ++i) {
                yb[i] = 0.0;
                lb[i] = 0.0;
                if (i < n) yb[i] = fwd_step<true>(e, w2, u2, kr[slot(i)], vr[slot(i)], gr[slot(i)], lb[i]);
            }
            du += e.du;
            dw += e.dw;
        }
        // reverse summary of this wave's steps, for the earlier waves (split pass 1: all
        // waves, folded into the block's summary)
        if (wv > 0 || p.split == 1) {
            Bwd r = bwd_empty();
            if (fast) {
                if (n > 0) r = bwd_norm(Bwd{rl, rs, -p0, 0.f});   // at the span start: scale 2^-p0
            } else {
#pragma unroll
                for (int i = kBwdSub - 1; i >= 0; --i)
                    if (i < n) bwd_absorb(r, w2, yb[i], gr[slot(i)], lb[i]);
            }
            rsum[wv][lane] = r;
        }
        __syncthreads();
        if (p.split == 1 && wv == 0 && c < C) {
            Bwd rb = bwd_empty();
            for (int j = kBwdWaves - 1; j >= 0; --j) rb = bwd_combine(rb, rsum[j][lane], (float)span(blk, j), w2);
            bwd_store(Planes{p.bsum, nblk, C, 4}, b, blk, c, rb);
        }
        Bwd r = rcarry[blk & 1][lane];
        for (int j = kBwdWaves - 1; j > wv; --j) r = bwd_combine(r, rsum[j][lane], (float)span(blk, j), w2);
        // backward run: dk, dv; each slot then takes the previous block's step
        const unsigned vn = blk > last ? voff : kOutOfRange;
        const int tp = t0 - kBwdBlock;
        // fixed-reference form: the reverse sums entering from the right, on the line at t = n
        double rho = 0.0, sig = 0.0;
        if (fast && n > 0) {
            const double sc = exp2_d(fma((double)r.n, w2, r.anc) + fma((double)n, w2, p0));
            rho = r.ab * sc;
            sig = r.bb * sc;
        }
#pragma unroll
        for (int i = kBwdSub - 1; i >= 0; --i) {
            const int sl = slot(i);
            if (i < n && p.split != 1) {
                float a, g;
                if (fast) {
                    const double vv = vr[sl], gg = gr[sl], y = yb[i], inv = lb[i];
                    const double ee = exp2_d(height(i) - p0), cg = ee * cwu * inv * gg;
                    g = (float)fma(ee, rho, cg);
                    a = (float)fma(cg, vv - y, ee * fma(vv, rho, sig));
                    const double gi = gg * inv;
                    rho += gi;
                    sig = fma(-gi, y, sig);
                } else {
                    bwd_step(r, w2, u2, kr[sl], vr[sl], yb[i], gr[sl], lb[i], a, g);
                }
                buffer_store4s(rdk, voff, (unsigned)((t0 + i) * C * 4), a);
                buffer_store4s(rdv, voff, (unsigned)((t0 + i) * C * 4), g);
            }
            // the previous block's step that the other parity keeps in this slot
            const int sp = REV ? sl : kBwdSub - 1 - sl;
            kr[sl] = buffer_load4s(rk, vn, soff(max(tp, 0) + sp));
            vr[sl] = buffer_load4s(rv, vn, soff(max(tp, 0) + sp));
            gr[sl] = buffer_load4s(rd, vn, soff(max(tp, 0) + sp));
        }
        if (fast && n > 0) r = bwd_norm(Bwd{rho, sig, -p0, 0.f});   // at the span start
        if (wv == 0 && blk > last) rcarry[(blk - 1) & 1][lane] = r;
        if (wv == 0 && blk == 0) rfirst = r;   // (Abar, Bbar) reaching the sums of the carried state
    };
    {
        int blk = myblk;
        for (; blk >= last + 1; blk -= 2) {
            block(blk, std::false_type{});
            block(blk - 1, std::true_type{});
        }
        if (blk == last) block(last, std::false_type{});
    }
    if (p.split == 1) return;
    // the carried state's gradient: it enters through A_0 = aa e^pp and B_0 = bb e^pp,
    // so d aa = Abar_0 e^pp, d bb = Bbar_0 e^pp, d pp = aa d aa + bb d bb (zeros for
    // the empty state)
    if (p.dstate_in && wv == 0 && last == 0 && c < C) {
        const size_t i = (size_t)b * C + c, plane = (size_t)p.B * C;
        double da = 0.0, db = 0.0, dp = 0.0;
        if (p.state_in) {
            const double aa0 = p.state_in[i], bb0 = p.state_in[plane + i];
            const double sc = exp2_d(fma((double)rfirst.n, w2, rfirst.anc) +
                                     (double)p.state_in[2 * plane + i] * (double)kLog2e);
            da = rfirst.ab * sc;
            db = rfirst.bb * sc;
            dp = fma(aa0, da, bb0 * db);
        }
        p.dstate_in[i] = (float)da;
        p.dstate_in[plane + i] = (float)db;
        p.dstate_in[2 * plane + i] = (float)dp;
    }
    // per-row sums of du and dw: the waves' partial sums added in wave order
    red[0][wv][lane] = du;
    red[1][wv][lane] = dw;
    __syncthreads();
    if (wv == 0 && c < C) {
        double su = 0.0, sw = 0.0;
        for (int j = 0; j < kBwdWaves; ++j) {
            su += red[0][j][lane];
            sw += red[1][j][lane];
        }
        const int nparts = p.split ? p.nseg : 1, part = seg;
        const size_t j = ((size_t)b * nparts + part) * C + c, plane = (size_t)p.B * nparts * C;
        p.part[j] = (float)su;
        p.part[plane + j] = (float)sw;
    }
}

// du[c], dw[c] = sums of the partials [2][B][nparts][C], b then part ascending.
__global__ __launch_bounds__(256) void wkv_bwd_reduce(const float *part, float *du, float *dw, int B, int nparts,
                                                      int C) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    const size_t rows = (size_t)B * nparts;
    float su = 0.f, sw = 0.f;
    for (size_t r = 0; r < rows; ++r) {
        su += part[r * C + c];
        sw += part[rows * C + r * C + c];
    }
    if (du) du[c] = su;
    if (dw) dw[c] = sw;
}

}  // namespace

// Split mode below this many 64-channel groups (the walks then leave most SIMDs
// idle): every (group, block) runs at once, joined by per-channel scans of the
// block summaries, at the cost of reading k, v and dy once more.
constexpr long kBwdSplitUnits = 256;

bool wkv_bwd_split(int B, int T, int C) {
    const long units = (long)B * (((long)C + 63) / 64), nblk = ((long)T + kBwdBlock - 1) / kBwdBlock;
    return units < kBwdSplitUnits && nblk > 1;
}

// Split mode: segments of `per` blocks, enough of them that the workgroups fill
// one resident round (two per CU) without exceeding it.
namespace {
void split_plan(int B, int T, int C, int *nseg, int *per) {
    const long units = (long)B * (((long)C + 63) / 64), nblk = ((long)T + kBwdBlock - 1) / kBwdBlock;
    long s = 512 / units;
    if (s < 1) s = 1;
    if (s > nblk) s = nblk;
    const long pb = (nblk + s - 1) / s;
    *per = (int)pb;
    *nseg = (int)((nblk + pb - 1) / pb);
}
}  // namespace

// Workspace: the first kWkvCtrBytes are left alone (other calls sharing it keep
// their counters there); then the block checkpoints (six doubles per channel and
// block), in split mode the block summaries (six) and reverse carries (four), and
// the partial sums of du and dw (per row, or per row and block in split mode).
namespace {
size_t r256(size_t x) { return (x + 255) / 256 * 256; }
}

size_t wkv_bwd_ws_bytes(int B, int T, int C) {
    const size_t nblk = ((size_t)T + kBwdBlock - 1) / kBwdBlock, plane = (size_t)B * nblk * C * 8;
    const bool sp = wkv_bwd_split(B, T, C);
    int nseg = 1, per = 1;
    if (sp) split_plan(B, T, C, &nseg, &per);
    const size_t nparts = (size_t)nseg;
    return kWkvCtrBytes + r256(plane * kCkptFields) + (sp ? r256(plane * kCkptFields) + r256(plane * 4) : 0) +
           r256((size_t)2 * B * nparts * C * 4);
}

void wkv_bwd_layout(int B, int T, int C, char *ws, WKVBwdParams &p) {
    const size_t nblk = ((size_t)T + kBwdBlock - 1) / kBwdBlock, plane = (size_t)B * nblk * C * 8;
    const bool sp = wkv_bwd_split(B, T, C);
    char *q = ws + kWkvCtrBytes;
    p.ckpt = reinterpret_cast<double *>(q);
    q += r256(plane * kCkptFields);
    p.bsum = p.rcar = nullptr;
    if (sp) {
        p.bsum = reinterpret_cast<double *>(q);
        q += r256(plane * kCkptFields);
        p.rcar = reinterpret_cast<double *>(q);
        q += r256(plane * 4);
    }
    p.part = reinterpret_cast<float *>(q);
    p.split = 0;
    p.nseg = p.per = 1;
    if (sp) split_plan(B, T, C, &p.nseg, &p.per);
}

hipError_t wkv_launch_bwd(const WKVBwdParams &p, hipStream_t stream) {
    const unsigned groups = (unsigned)(p.B * ((p.C + 63) / 64));
    const bool sp = wkv_bwd_split(p.B, p.T, p.C);
    hipError_t e;
    if (sp) {
        WKVBwdParams q = p;
        const unsigned lanes = (unsigned)(((long)p.B * p.C + 255) / 256);
        const unsigned grid = groups * (unsigned)p.nseg;
        q.split = 1;
        hipLaunchKernelGGL(wkv_bwd_ckpt, dim3(grid), dim3(64 * kBwdWaves), 0, stream, q);
        hipLaunchKernelGGL(wkv_bwd_fscan, dim3(lanes), dim3(256), 0, stream, q);
        hipLaunchKernelGGL(wkv_bwd_rev, dim3(grid), dim3(64 * kBwdWaves), 0, stream, q);
        hipLaunchKernelGGL(wkv_bwd_rscan, dim3(lanes), dim3(256), 0, stream, q);
        q.split = 2;
        hipLaunchKernelGGL(wkv_bwd_rev, dim3(grid), dim3(64 * kBwdWaves), 0, stream, q);
    } else {
        hipLaunchKernelGGL(wkv_bwd_ckpt, dim3(groups), dim3(64 * kBwdWaves), 0, stream, p);
        hipLaunchKernelGGL(wkv_bwd_rev, dim3(groups), dim3(64 * kBwdWaves), 0, stream, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess || (!p.du && !p.dw)) return e;
    hipLaunchKernelGGL(wkv_bwd_reduce, dim3((unsigned)((p.C + 255) / 256)), dim3(256), 0, stream, p.part, p.du,
                       p.dw, p.B, sp ? p.nseg : 1, p.C);
    return hipGetLastError();
}

}  // namespace drs
