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
// (A' = dA/dw, likewise B').  One lane per (b, c) makes two passes:
//   forward:  the state as in the forward kernel (log2-scaled, the log-scale as
//             anchor + n w), A' and B' on the same scale, du and dw; it stores
//             log2 D_t and the recomputed y_t for the second pass;
//   backward: Abar, Bbar on a shared log2-scale, again an anchor plus a step
//             count, so that every exponential formed has a non-positive
//             argument up to rounding: e^{u+k}/D <= 1 and e^{k} Abar is bounded
//             because D_{t'} contains the decayed term of token t.
// The per-row sums of du and dw go to the workspace and are added over the
// batch in a fixed order.
#include "common.h"
#include "wkv.h"

namespace drs {

namespace {

constexpr int kBwdThreads = 64;
constexpr int kBwdPF = 16;   // steps of every input in flight per lane

// Precision: the log2-scales reach ~90 with keys of +-60, where one fp32
// rounding already costs ~4e-6 relative in the exponential formed from a
// difference of two of them, and the gradients subtract nearly equal sums
// (A' - y B', v Abar + Bbar), which fp32 copies of y would spoil.  So the
// scales, the sums, the stored log2 denominators and the stored outputs are
// fp64; each exponential is the fp32 exp2 of a difference already formed in
// fp64 (an argument <= 0 of modest size).

struct Fwd {
    double aa, bb, anc, ap, bp, du, dw;   // state (log2-scale anc + n w2), A', B', gradient sums
    float n;
};

// One step forward: returns y_t; writes log2 D_t.
__device__ __forceinline__ double fwd_step(Fwd &s, double w2, double u2, float k, float v, float dy, double &lden) {
    const double k2 = (double)k * (double)kLog2e;
    const double pp2 = fma((double)s.n, w2, s.anc);
    const double d = pp2 - (u2 + k2);
    const double ex = (double)exp2_fast(-(float)fabs(d));
    const bool past = d > 0.0;
    const double e_pp = past ? 1.0 : ex, e_cur = past ? ex : 1.0;   // 2^{pp-m}, 2^{u+k-m}
    const double den = fma(e_pp, s.bb, e_cur);                      // D / 2^m
    const double num = fma(e_pp, s.aa, e_cur * (double)v);
    const double inv = 1.0 / den;
    const double y = num * inv;
    const double g = (double)dy * inv;
    s.du = fma(e_cur * g, (double)v - y, s.du);
    s.dw = fma(e_pp * g, fma(-y, s.bp, s.ap), s.dw);
    lden = (past ? pp2 : u2 + k2) + (double)__log2f((float)den);
    // absorb the token after one step of decay
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

__global__ __launch_bounds__(kBwdThreads) void wkv_bwd(WKVBwdParams p) {
    const int c = blockIdx.x * kBwdThreads + threadIdx.x, b = blockIdx.y;
    if (c >= p.C) return;
    const int T = p.T, C = p.C;
    const double w2 = (double)p.w[c] * (double)kLog2e, u2 = (double)p.u[c] * (double)kLog2e;
    const size_t base = (size_t)b * T * C + c;
    const float *k = p.k + base, *v = p.v + base, *dy = p.dy + base;
    double *lden = p.lden + base;
    double *yr = p.yrec + base;

    Fwd f;
    if (p.state_in) {
        const size_t i = (size_t)b * C + c, plane = (size_t)p.B * C;
        f = Fwd{p.state_in[i], p.state_in[plane + i], (double)p.state_in[2 * plane + i] * (double)kLog2e,
                0.0, 0.0, 0.0, 0.0, 0.f};
    } else {
        f = Fwd{0.0, 0.0, -1e38 * (double)kLog2e, 0.0, 0.0, 0.0, 0.0, 0.f};
    }

    // ---- forward pass: blocks of PF steps, the next block's loads in flight ----
    const int nfull = T / kBwdPF;
    float kc[kBwdPF], vc[kBwdPF], gc[kBwdPF];
    auto load = [&](int tb, float *kd, float *vd, float *gd) {
#pragma unroll
        for (int i = 0; i < kBwdPF; ++i) {
            const size_t o = (size_t)(tb + i) * C;
            kd[i] = __builtin_nontemporal_load(k + o);
            vd[i] = __builtin_nontemporal_load(v + o);
            gd[i] = __builtin_nontemporal_load(dy + o);
        }
    };
    if (nfull > 0) load(0, kc, vc, gc);
    for (int blk = 0; blk < nfull; ++blk) {
        const int tb = blk * kBwdPF;
        float kn[kBwdPF], vn[kBwdPF], gn[kBwdPF];
        if (blk + 1 < nfull) load(tb + kBwdPF, kn, vn, gn);
#pragma unroll
        for (int i = 0; i < kBwdPF; ++i) {
            double ld;
            const double y = fwd_step(f, w2, u2, kc[i], vc[i], gc[i], ld);
            lden[(size_t)(tb + i) * C] = ld;
            yr[(size_t)(tb + i) * C] = y;
        }
#pragma unroll
        for (int i = 0; i < kBwdPF; ++i) { kc[i] = kn[i]; vc[i] = vn[i]; gc[i] = gn[i]; }
    }
    for (int t = nfull * kBwdPF; t < T; ++t) {
        const size_t o = (size_t)t * C;
        double ld;
        const double y = fwd_step(f, w2, u2, k[o], v[o], dy[o], ld);
        lden[o] = ld;
        yr[o] = y;
    }
    p.part[(size_t)b * C + c] = (float)f.du;
    p.part[(size_t)p.B * C + (size_t)b * C + c] = (float)f.dw;

    // ---- backward pass: the ragged tail first (it ends the sequence), then
    // whole blocks from the end, each block's predecessor loading meanwhile -----
    Bwd r{0.0, 0.0, -1e38 * (double)kLog2e, 0.f};
    float *dk = p.dk + base, *dv = p.dv + base;
    for (int t = T - 1; t >= nfull * kBwdPF; --t) {
        const size_t o = (size_t)t * C;
        float a, e;
        bwd_step(r, w2, u2, k[o], v[o], yr[o], dy[o], lden[o], a, e);
        dk[o] = a;
        dv[o] = e;
    }
    double yc[kBwdPF], lc[kBwdPF];
    auto loadb = [&](int tb, float *kd, float *vd, float *gd, double *yd, double *ld) {
        load(tb, kd, vd, gd);
#pragma unroll
        for (int i = 0; i < kBwdPF; ++i) {
            yd[i] = yr[(size_t)(tb + i) * C];
            ld[i] = lden[(size_t)(tb + i) * C];
        }
    };
    if (nfull > 0) loadb((nfull - 1) * kBwdPF, kc, vc, gc, yc, lc);
    for (int blk = nfull - 1; blk >= 0; --blk) {
        const int tb = blk * kBwdPF;
        float kn[kBwdPF], vn[kBwdPF], gn[kBwdPF];
        double yn[kBwdPF], ln[kBwdPF];
        if (blk > 0) loadb(tb - kBwdPF, kn, vn, gn, yn, ln);
#pragma unroll
        for (int i = kBwdPF - 1; i >= 0; --i) {
            float a, e;
            bwd_step(r, w2, u2, kc[i], vc[i], yc[i], gc[i], lc[i], a, e);
            __builtin_nontemporal_store(a, dk + (size_t)(tb + i) * C);
            __builtin_nontemporal_store(e, dv + (size_t)(tb + i) * C);
        }
#pragma unroll
        for (int i = 0; i < kBwdPF; ++i) { kc[i] = kn[i]; vc[i] = vn[i]; gc[i] = gn[i]; yc[i] = yn[i]; lc[i] = ln[i]; }
    }
}

// du[c], dw[c] = sums over b of the per-row partials, b ascending.
__global__ __launch_bounds__(256) void wkv_bwd_reduce(const float *part, float *du, float *dw, int B, int C) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    float su = 0.f, sw = 0.f;
    for (int b = 0; b < B; ++b) {
        su += part[(size_t)b * C + c];
        sw += part[(size_t)B * C + (size_t)b * C + c];
    }
    if (du) du[c] = su;
    if (dw) dw[c] = sw;
}

}  // namespace

// The first kWkvCtrBytes are left alone (other calls sharing the workspace keep
// their counters there); then the fp64 log2 denominators, the recomputed
// outputs, and the per-row partials.
size_t wkv_bwd_ws_bytes(int B, int T, int C) {
    const size_t n = (size_t)B * T * C;
    return kWkvCtrBytes + (n * 8 + 255) / 256 * 256 + (n * 8 + 255) / 256 * 256 +
           ((size_t)2 * B * C * 4 + 255) / 256 * 256;
}

hipError_t wkv_launch_bwd(const WKVBwdParams &p, hipStream_t stream) {
    hipLaunchKernelGGL(wkv_bwd, dim3((unsigned)((p.C + kBwdThreads - 1) / kBwdThreads), (unsigned)p.B),
                       dim3(kBwdThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || (!p.du && !p.dw)) return e;
    hipLaunchKernelGGL(wkv_bwd_reduce, dim3((unsigned)((p.C + 255) / 256)), dim3(256), 0, stream, p.part, p.du,
                       p.dw, p.B, p.C);
    return hipGetLastError();
}

}  // namespace drs
