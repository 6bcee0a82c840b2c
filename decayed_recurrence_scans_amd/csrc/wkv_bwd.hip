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
//             the state entering every block of 16 steps (a checkpoint);
//   backward: per block from the end, the block's outputs and log2 denominators
//             are rebuilt from its checkpoint in registers, then
//             Abar, Bbar run on a shared log2-scale, again an anchor plus a step
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
// scales, the sums, the checkpoints and the rebuilt outputs and denominators are
// fp64; each exponential is the fp32 exp2 of a difference already formed in
// fp64 (an argument <= 0 of modest size).

struct Fwd {
    double aa, bb, anc, ap, bp, du, dw;   // state (log2-scale anc + n w2), A', B', gradient sums
    float n;
};

// One step forward: returns y_t and writes log2 D_t.  With DERIV it also carries
// A', B' and adds the step's terms of du and dw (the first pass); without, it only
// rebuilds y and D (the block recomputation of the second pass).
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

// Steps of a block: the forward pass stores the state (aa, bb, anchor, count)
// entering every block; the reverse pass rebuilds the block's outputs and
// denominators from it in registers.
constexpr int kBwdBlock = kBwdPF;

__global__ __launch_bounds__(kBwdThreads) void wkv_bwd(WKVBwdParams p) {
    const int c = blockIdx.x * kBwdThreads + threadIdx.x, b = blockIdx.y;
    if (c >= p.C) return;
    const int T = p.T, C = p.C;
    const int nblk = (T + kBwdBlock - 1) / kBwdBlock;
    const double w2 = (double)p.w[c] * (double)kLog2e, u2 = (double)p.u[c] * (double)kLog2e;
    const size_t row0 = (size_t)b * T * C;
    // checkpoints [b][block][field][c], fields aa, bb, anchor, count
    double *ck = p.ckpt + (size_t)b * nblk * 4 * C + c;
    auto ckf = [&](int blk, int field) -> double & { return ck[((size_t)blk * 4 + field) * C]; };

    // rows past T are out of range: loads give 0 (those steps are never used)
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dy + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rdk = make_rsrc(p.dk + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rdv = make_rsrc(p.dv + row0, T * C * 4);
    auto off = [&](int t) { return t < T ? (unsigned)(((size_t)t * C + c) * 4) : kOutOfRange; };

    Fwd f;
    if (p.state_in) {
        const size_t i = (size_t)b * C + c, plane = (size_t)p.B * C;
        f = Fwd{p.state_in[i], p.state_in[plane + i], (double)p.state_in[2 * plane + i] * (double)kLog2e,
                0.0, 0.0, 0.0, 0.0, 0.f};
    } else {
        f = Fwd{0.0, 0.0, -1e38 * (double)kLog2e, 0.0, 0.0, 0.0, 0.0, 0.f};
    }

    struct Blk {
        float k[kBwdBlock], v[kBwdBlock], g[kBwdBlock];
    };
    auto load = [&](int blk, Blk &B) {
#pragma unroll
        for (int i = 0; i < kBwdBlock; ++i) {
            const unsigned o = off(blk * kBwdBlock + i);
            B.k[i] = buffer_load4(rk, o);
            B.v[i] = buffer_load4(rv, o);
            B.g[i] = buffer_load4(rd, o);
        }
    };

    // ---- forward pass: checkpoints, du, dw -----------------------------------------
    Blk cur, nxt;
    load(0, cur);
    for (int blk = 0; blk < nblk; ++blk) {
        if (blk + 1 < nblk) load(blk + 1, nxt);
        ckf(blk, 0) = f.aa;
        ckf(blk, 1) = f.bb;
        ckf(blk, 2) = f.anc;
        ckf(blk, 3) = (double)f.n;
        const int n = min(kBwdBlock, T - blk * kBwdBlock);
#pragma unroll
        for (int i = 0; i < kBwdBlock; ++i) {
            if (i < n) {
                double ld;
                fwd_step<true>(f, w2, u2, cur.k[i], cur.v[i], cur.g[i], ld);
            }
        }
        if (blk + 1 < nblk) cur = nxt;
    }
    p.part[(size_t)b * C + c] = (float)f.du;
    p.part[(size_t)p.B * C + (size_t)b * C + c] = (float)f.dw;

    // ---- reverse pass: per block from the end, rebuild (y, log2 D) from the
    // checkpoint, then run the gradients backward; the previous block loads meanwhile
    Bwd r{0.0, 0.0, -1e38 * (double)kLog2e, 0.f};
    load(nblk - 1, cur);
    for (int blk = nblk - 1; blk >= 0; --blk) {
        if (blk > 0) load(blk - 1, nxt);
        Fwd s{ckf(blk, 0), ckf(blk, 1), ckf(blk, 2), 0.0, 0.0, 0.0, 0.0, (float)ckf(blk, 3)};
        const int n = min(kBwdBlock, T - blk * kBwdBlock);
        double yb[kBwdBlock], lb[kBwdBlock];
#pragma unroll
        for (int i = 0; i < kBwdBlock; ++i) yb[i] = fwd_step<false>(s, w2, u2, cur.k[i], cur.v[i], 0.f, lb[i]);
#pragma unroll
        for (int i = kBwdBlock - 1; i >= 0; --i) {
            if (i < n) {
                float a, e;
                bwd_step(r, w2, u2, cur.k[i], cur.v[i], yb[i], cur.g[i], lb[i], a, e);
                const unsigned o = off(blk * kBwdBlock + i);
                buffer_store4(rdk, o, a);
                buffer_store4(rdv, o, e);
            }
        }
        if (blk > 0) cur = nxt;
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
// their counters there); then the block checkpoints (4 doubles per channel and
// block of kBwdBlock steps) and the per-row partials.
size_t wkv_bwd_ws_bytes(int B, int T, int C) {
    const size_t nblk = (T + kBwdBlock - 1) / kBwdBlock;
    return kWkvCtrBytes + ((size_t)B * nblk * 4 * C * 8 + 255) / 256 * 256 +
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
