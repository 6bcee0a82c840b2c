// la_rec_bwd.hip -- the backward of linear attention, one step at a time.
//
// The gradients of L = sum_t dy_t . y_t + <dS_final, S_final> (+ <dz_final,
// z_final> with the normaliser) for the recurrence S_t = g_t S_{t-1} + k_t v_t^T,
// z_t = g_t z_{t-1} + k_t, y_t = q_t^T S_t (or q_t^T S_t / q_t^T z_t): the decay of
// RetNet issue #21 (cumulative_ema: the factor of step t multiplies the state
// carried in; one factor per head, per step or per key channel), the QKV / QK1
// normaliser with a carried key sum of flash-linear-attention issue #268.  The pages
// say only that the gradient is again a set of cumulative sums (RWKV-LM discussion
// #189); here it is the chain rule through the recurrence, in two sweeps:
//
//   forward sweep, visiting order: recompute S_t and z_t; the read-out passes on
//     a_t = dy_t / d_t  to the numerator n_t = q_t^T S_t  and
//     c_t = -(dy_t . y_t) / d_t  to the denominator d_t = q_t^T z_t
//     (a_t = dy_t, c_t = 0 without the normaliser);  dq_t = S_t a_t + z_t c_t.
//   reverse sweep, opposite order, with G = dL/dS and Gz = dL/dz of the state
//     leaving the step:  G += q_t a_t^T,  Gz += q_t c_t;  dk_t = G v_t + Gz,
//     dv_t = G^T k_t;  then G, Gz scale by g_t (per key row i in per-channel mode);
//     what is left at the end is the initial state's and key sum's gradient.
//
// The factor gradient without the states of every step: scaling g_t[i] by lambda
// has the same effect on L as scaling q_s[i] by lambda and k_s[i] by 1/lambda for
// every step s visited at or after t, plus row i of the final state and key sum by
// lambda.  So  g_t[i] dL/dg_t[i] = sum_{s visited at or after t} (q_s[i] dq_s[i] -
// k_s[i] dk_s[i]) + <dS_final[i,:], S_final[i,:]> + dz_final[i] z_final[i], a
// running sum of the reverse sweep (summed over i for scalar factors).  Its terms
// partly cancel, so they are formed and summed in fp64 (fp32 sums over a few
// hundred steps missed a 1e-5 bar).
//
// Layout as the forward step-by-step kernel: one workgroup per (b, h); thread (rg,
// quad) holds columns 4 quad .. 4 quad + 3 of rows rg + RG i of the state (and of
// its gradient), i < RPT.  Sums over a row's columns are lane exchanges; sums over
// rows go through lane exchanges inside a wave and LDS across waves (two buffers
// alternating by step, one barrier per step).
#include "common.h"
#include "la_rec.h"
#include "la_rec_bwd.h"

namespace drs {

namespace {

template <typename TI> __device__ __forceinline__ float load_in(const TI *p, size_t i);
template <> __device__ __forceinline__ float load_in<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_in<uint16_t>(const uint16_t *p, size_t i) {
    return bf16_bits_to_f32(p[i]);
}
__device__ __forceinline__ void store_out(float *p, size_t i, float x) { p[i] = x; }
__device__ __forceinline__ void store_out(uint16_t *p, size_t i, float x) { p[i] = f32_to_bf16_bits(x); }

constexpr int kThreads = 256;

// factor of key row d at staged step n
template <int MODE>
__device__ __forceinline__ float factor_of(const float *sg, float gh, int n, int d, int Dk) {
    if constexpr (MODE == 0) return 1.f;
    else if constexpr (MODE == 1) return gh;
    else if constexpr (MODE == 2) return sg[n];
    else return sg[n * Dk + d];
}

// ---- forward sweep: dq, and a_t / c_t for the reverse sweep ------------------------
template <typename TI, int RPT, int MODE, bool NORM>
__global__ __launch_bounds__(kThreads) void la_rbwd_fwd(LARecBwdParams p) {
    extern __shared__ f32x4 smem4[];
    const int Dk = p.Dk, Dv = p.Dv, T = p.T, TB = p.tb;
    const int NT = blockDim.x, QPR = Dv >> 2, RG = NT / QPR;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = NT >> 6;
    const int quad = tid % QPR, rg = tid / QPR;
    const int bh = blockIdx.x;

    f32x4 *red = smem4;                                              // [2][nw][QPR]
    float *rden = reinterpret_cast<float *>(red + 2 * nw * QPR);     // [2][4]
    float *sv = rden + 8;                                            // [TB][Dv]
    float *sdy = sv + TB * Dv;                                       // [TB][Dv]
    float *sq = sdy + TB * Dv;                                       // [TB][Dk]
    float *sk = sq + TB * Dk;                                        // [TB][Dk]
    float *sg = sk + TB * Dk;                                        // [TB][Dk] | [TB]

    f32x4 S[RPT];
    float z[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int d = rg + RG * i;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[i][r] = p.state_in ? p.state_in[((size_t)bh * Dk + d) * Dv + 4 * quad + r] : 0.f;
        z[i] = (NORM && p.cum_k_in) ? p.cum_k_in[(size_t)bh * Dk + d] : 0.f;
    }
    const float gh = MODE == 1 ? p.decay[bh % p.H] : 1.f;
    const TI *qg = static_cast<const TI *>(p.q) + (size_t)bh * T * Dk;
    const TI *kg = static_cast<const TI *>(p.k) + (size_t)bh * T * Dk;
    const TI *vg = static_cast<const TI *>(p.v) + (size_t)bh * T * Dv;
    const TI *dyg = static_cast<const TI *>(p.dy) + (size_t)bh * T * Dv;
    TI *dqg = static_cast<TI *>(p.dq) + (size_t)bh * T * Dk;
    const int dk_shift = __builtin_ctz(Dk), dv_shift = __builtin_ctz(Dv);

    int par = 0;
    for (int n0 = 0; n0 < T; n0 += TB) {
        const int nb = T - n0 < TB ? T - n0 : TB;
        for (int e = tid; e < nb * Dk; e += NT) {
            const int n = e >> dk_shift, d = e & (Dk - 1);
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            sq[e] = load_in<TI>(qg, (size_t)t * Dk + d);
            sk[e] = load_in<TI>(kg, (size_t)t * Dk + d);
            if constexpr (MODE == 3) sg[e] = p.decay[((size_t)bh * T + t) * Dk + d];
        }
        for (int e = tid; e < nb * Dv; e += NT) {
            const int n = e >> dv_shift, j = e & (Dv - 1);
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            sv[e] = load_in<TI>(vg, (size_t)t * Dv + j);
            sdy[e] = load_in<TI>(dyg, (size_t)t * Dv + j);
        }
        if constexpr (MODE == 2) {
            for (int n = tid; n < nb; n += NT) {
                const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
                sg[n] = p.decay[(size_t)bh * T + t];
            }
        }
        __syncthreads();

        for (int n = 0; n < nb; ++n) {
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            const float *qn = sq + n * Dk, *kn = sk + n * Dk;
            const f32x4 vq = *reinterpret_cast<const f32x4 *>(sv + n * Dv + 4 * quad);
            const f32x4 dy4 = *reinterpret_cast<const f32x4 *>(sdy + n * Dv + 4 * quad);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            float dacc = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int d = rg + RG * i;
                const float g = factor_of<MODE>(sg, gh, n, d, Dk);
                const float kd = kn[d], qd = qn[d];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    S[i][r] = fmaf(kd, vq[r], g * S[i][r]);
                    if constexpr (NORM) acc[r] = fmaf(qd, S[i][r], acc[r]);
                }
                if constexpr (NORM) {
                    z[i] = fmaf(g, z[i], kd);
                    dacc = fmaf(qd, z[i], dacc);
                }
            }
            f32x4 a4 = dy4;
            float c = 0.f;
            if constexpr (NORM) {
                // n_t (this thread's four columns) and d_t, summed over every row
                for (int m = QPR; m < 64; m <<= 1) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] += __shfl_xor(acc[r], m, 64);
                    dacc += __shfl_xor(dacc, m, 64);
                }
                if (lane < QPR) red[(par * nw + wv) * QPR + quad] = acc;
                if (lane == 0) rden[par * 4 + wv] = dacc;
                __syncthreads();
                f32x4 num = red[(par * nw) * QPR + quad];
                float den = rden[par * 4];
                for (int w2 = 1; w2 < nw; ++w2) {
                    num += red[(par * nw + w2) * QPR + quad];
                    den += rden[par * 4 + w2];
                }
                float dyy = 0.f;   // dy_t . y_t
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    a4[r] = dy4[r] / den;
                    dyy = fmaf(dy4[r], num[r] / den, dyy);
                }
                for (int m = 1; m < QPR; m <<= 1) dyy += __shfl_xor(dyy, m, 64);
                c = -dyy / den;
                if (wv == 0 && lane < QPR) {
                    *reinterpret_cast<f32x4 *>(p.a32 + ((size_t)bh * T + t) * Dv + 4 * quad) = a4;
                    if (quad == 0) p.c32[(size_t)bh * T + t] = c;
                }
            }
            // dq_t = S_t a_t + z_t c_t, row by row
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int d = rg + RG * i;
                float part = S[i][0] * a4[0];
#pragma unroll
                for (int r = 1; r < 4; ++r) part = fmaf(S[i][r], a4[r], part);
                for (int m = 1; m < QPR; m <<= 1) part += __shfl_xor(part, m, 64);
                if constexpr (NORM) part = fmaf(z[i], c, part);
                if (quad == 0) {
                    store_out(dqg, (size_t)t * Dk + d, part);
                    if (p.dq32) p.dq32[((size_t)bh * T + t) * Dk + d] = part;
                }
            }
            par ^= 1;
        }
        __syncthreads();   // every wave is done with the staged block before it is replaced
    }
    if (p.sfin) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int d = rg + RG * i;
            *reinterpret_cast<f32x4 *>(p.sfin + ((size_t)bh * Dk + d) * Dv + 4 * quad) = S[i];
        }
    }
    if (NORM && p.zfin && quad == 0) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) p.zfin[(size_t)bh * Dk + rg + RG * i] = z[i];
    }
}

// ---- reverse sweep: dk, dv, the factor gradient, the initial gradients -------------
template <typename TI, int RPT, int MODE, bool NORM, bool DG>
__global__ __launch_bounds__(kThreads) void la_rbwd_rev(LARecBwdParams p) {
    extern __shared__ f32x4 smem4[];
    const int Dk = p.Dk, Dv = p.Dv, T = p.T, TB = p.tb;
    const int NT = blockDim.x, QPR = Dv >> 2, RG = NT / QPR;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = NT >> 6;
    const int quad = tid % QPR, rg = tid / QPR;
    const int bh = blockIdx.x;
    constexpr bool SCALAR = MODE == 1 || MODE == 2;   // one factor for every key row

    f32x4 *red = smem4;                                              // [2][nw][QPR]
    double *rsum = reinterpret_cast<double *>(red + 2 * nw * QPR);   // [2][4]
    float *sv = reinterpret_cast<float *>(rsum + 8);                 // [TB][Dv]
    float *sa = sv + TB * Dv;                                        // [TB][Dv] a_t (dy_t)
    float *sq = sa + TB * Dv;                                        // [TB][Dk]
    float *sk = sq + TB * Dk;                                        // [TB][Dk]
    float *sdq = sk + TB * Dk;                                       // [TB][Dk] (DG)
    float *sc = sdq + (DG ? TB * Dk : 0);                            // [TB] (NORM)
    float *sg = sc + (NORM ? TB : 0);                                // [TB][Dk] | [TB]

    f32x4 G[RPT];
    float Gz[RPT];
    double R[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int d = rg + RG * i;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            G[i][r] = p.dstate_out ? p.dstate_out[((size_t)bh * Dk + d) * Dv + 4 * quad + r] : 0.f;
        Gz[i] = (NORM && p.dcum_k_out) ? p.dcum_k_out[(size_t)bh * Dk + d] : 0.f;
        R[i] = 0.0;
    }
    double Rtot = 0.0;
    float hsum = 0.f;
    if constexpr (DG) {
        // the final-state terms <dS_final[i,:], S_final[i,:]> + dz_final[i] z_final[i]
        double rows = 0.0;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int d = rg + RG * i;
            double part = 0.0;
            if (p.dstate_out) {
                const f32x4 s = *reinterpret_cast<const f32x4 *>(p.sfin + ((size_t)bh * Dk + d) * Dv + 4 * quad);
#pragma unroll
                for (int r = 0; r < 4; ++r) part += (double)G[i][r] * (double)s[r];
            }
            for (int m = 1; m < QPR; m <<= 1) part += __shfl_xor(part, m, 64);
            if (NORM && p.dcum_k_out) part += (double)Gz[i] * (double)p.zfin[(size_t)bh * Dk + d];
            R[i] = part;
            rows += quad == 0 ? part : 0.0;
        }
        if constexpr (SCALAR) {
            for (int m = 1; m < 64; m <<= 1) rows += __shfl_xor(rows, m, 64);
            if (lane == 0) rsum[4 + wv] = rows;   // parity 1: the first step writes parity 0
            __syncthreads();
            if (tid == 0)
                for (int w2 = 0; w2 < nw; ++w2) Rtot += rsum[4 + w2];
        }
    }
    const float gh = MODE == 1 ? p.decay[bh % p.H] : 1.f;
    const TI *qg = static_cast<const TI *>(p.q) + (size_t)bh * T * Dk;
    const TI *kg = static_cast<const TI *>(p.k) + (size_t)bh * T * Dk;
    const TI *vg = static_cast<const TI *>(p.v) + (size_t)bh * T * Dv;
    const TI *dyg = static_cast<const TI *>(p.dy) + (size_t)bh * T * Dv;
    TI *dkg = static_cast<TI *>(p.dk) + (size_t)bh * T * Dk;
    TI *dvg = static_cast<TI *>(p.dv) + (size_t)bh * T * Dv;
    const int dk_shift = __builtin_ctz(Dk), dv_shift = __builtin_ctz(Dv);

    int par = 0;
    const int nblk = (T + TB - 1) / TB;
    for (int bi = nblk - 1; bi >= 0; --bi) {
        const int n0 = bi * TB, nb = T - n0 < TB ? T - n0 : TB;
        for (int e = tid; e < nb * Dk; e += NT) {
            const int n = e >> dk_shift, d = e & (Dk - 1);
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            sq[e] = load_in<TI>(qg, (size_t)t * Dk + d);
            sk[e] = load_in<TI>(kg, (size_t)t * Dk + d);
            if constexpr (DG) sdq[e] = p.dq32[((size_t)bh * T + t) * Dk + d];
            if constexpr (MODE == 3) sg[e] = p.decay[((size_t)bh * T + t) * Dk + d];
        }
        for (int e = tid; e < nb * Dv; e += NT) {
            const int n = e >> dv_shift, j = e & (Dv - 1);
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            sv[e] = load_in<TI>(vg, (size_t)t * Dv + j);
            if constexpr (NORM) sa[e] = p.a32[((size_t)bh * T + t) * Dv + j];
            else sa[e] = load_in<TI>(dyg, (size_t)t * Dv + j);
        }
        for (int n = tid; n < nb; n += NT) {
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            if constexpr (NORM) sc[n] = p.c32[(size_t)bh * T + t];
            if constexpr (MODE == 2) sg[n] = p.decay[(size_t)bh * T + t];
        }
        __syncthreads();

        for (int n = nb - 1; n >= 0; --n) {
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            const float *qn = sq + n * Dk, *kn = sk + n * Dk;
            const f32x4 v4 = *reinterpret_cast<const f32x4 *>(sv + n * Dv + 4 * quad);
            const f32x4 a4 = *reinterpret_cast<const f32x4 *>(sa + n * Dv + 4 * quad);
            const float c = NORM ? sc[n] : 0.f;
            f32x4 dv4 = {0.f, 0.f, 0.f, 0.f};
            double epart = 0.0;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int d = rg + RG * i;
                const float qd = qn[d], kd = kn[d];
                float part = 0.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    G[i][r] = fmaf(qd, a4[r], G[i][r]);
                    part = fmaf(G[i][r], v4[r], part);
                    dv4[r] = fmaf(G[i][r], kd, dv4[r]);
                }
                if constexpr (NORM) Gz[i] = fmaf(qd, c, Gz[i]);
                for (int m = 1; m < QPR; m <<= 1) part += __shfl_xor(part, m, 64);
                const float dki = NORM ? part + Gz[i] : part;
                if (quad == 0) store_out(dkg, (size_t)t * Dk + d, dki);
                const float g = factor_of<MODE>(sg, gh, n, d, Dk);
                if constexpr (DG) {
                    const double e = (double)qd * (double)sdq[n * Dk + d] - (double)kd * (double)dki;
                    if constexpr (MODE == 3) {
                        R[i] += e;
                        if (quad == 0) p.ddecay[((size_t)bh * T + t) * Dk + d] = (float)(R[i] / (double)g);
                    } else {
                        epart += quad == 0 ? e : 0.0;
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) G[i][r] *= g;
                if constexpr (NORM) Gz[i] *= g;
            }
            for (int m = QPR; m < 64; m <<= 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r) dv4[r] += __shfl_xor(dv4[r], m, 64);
            }
            if (lane < QPR) red[(par * nw + wv) * QPR + quad] = dv4;
            if constexpr (DG && SCALAR) {
                for (int m = 1; m < 64; m <<= 1) epart += __shfl_xor(epart, m, 64);
                if (lane == 0) rsum[par * 4 + wv] = epart;
            }
            __syncthreads();
            if (wv == 0 && lane < QPR) {
                f32x4 o = red[(par * nw) * QPR + quad];
                for (int w2 = 1; w2 < nw; ++w2) o += red[(par * nw + w2) * QPR + quad];
#pragma unroll
                for (int r = 0; r < 4; ++r) store_out(dvg, (size_t)t * Dv + 4 * quad + r, o[r]);
            }
            if constexpr (DG && SCALAR) {
                if (tid == 0) {
                    double e = rsum[par * 4];
                    for (int w2 = 1; w2 < nw; ++w2) e += rsum[par * 4 + w2];
                    Rtot += e;
                    const float dg = (float)(Rtot / (double)factor_of<MODE>(sg, gh, n, 0, Dk));
                    if constexpr (MODE == 2) p.ddecay[(size_t)bh * T + t] = dg;
                    else hsum += dg;
                }
            }
            par ^= 1;
        }
        __syncthreads();
    }
    if (p.dstate_in) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int d = rg + RG * i;
#pragma unroll
            for (int r = 0; r < 4; ++r) p.dstate_in[((size_t)bh * Dk + d) * Dv + 4 * quad + r] = G[i][r];
        }
    }
    if (NORM && p.dcum_k_in && quad == 0) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) p.dcum_k_in[(size_t)bh * Dk + rg + RG * i] = Gz[i];
    }
    if (DG && MODE == 1 && tid == 0) p.hpart[bh] = hsum;
}

// ddecay[h] = sum over b of the per-unit sums, b ascending
__global__ void sum_over_batch(const float *part, float *out, int B, int H) {
    const int h = blockIdx.x * blockDim.x + threadIdx.x;
    if (h >= H) return;
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += part[(size_t)b * H + h];
    out[h] = s;
}

size_t fwd_lds(const LARecBwdParams &p, int nt) {
    const int nw = nt / 64, qpr = p.Dv / 4;
    const int gcols = p.mode == 3 ? p.Dk : (p.mode == 2 ? 1 : 0);
    return (size_t)2 * nw * qpr * 16 + 8 * 4 + (size_t)p.tb * (2 * p.Dk + 2 * p.Dv + gcols) * 4;
}
size_t rev_lds(const LARecBwdParams &p, int nt, bool dg) {
    const int nw = nt / 64, qpr = p.Dv / 4;
    const int gcols = p.mode == 3 ? p.Dk : (p.mode == 2 ? 1 : 0);
    return (size_t)2 * nw * qpr * 16 + 8 * 8 +
           (size_t)p.tb * (2 * p.Dk + (dg ? p.Dk : 0) + 2 * p.Dv + (p.normalize ? 1 : 0) + gcols) * 4;
}

template <typename TI, int RPT, int MODE, bool NORM>
hipError_t launch_sweeps(const LARecBwdParams &p, int nt, hipStream_t s) {
    const dim3 grid((unsigned)(p.B * p.H)), block((unsigned)nt);
    hipLaunchKernelGGL((la_rbwd_fwd<TI, RPT, MODE, NORM>), grid, block, fwd_lds(p, nt), s, p);
    if (p.ddecay && MODE != 0)
        hipLaunchKernelGGL((la_rbwd_rev<TI, RPT, MODE, NORM, MODE != 0>), grid, block, rev_lds(p, nt, true), s, p);
    else
        hipLaunchKernelGGL((la_rbwd_rev<TI, RPT, MODE, NORM, false>), grid, block, rev_lds(p, nt, false), s, p);
    if (p.ddecay && MODE == 1)
        hipLaunchKernelGGL(sum_over_batch, dim3((unsigned)((p.H + 255) / 256)), dim3(256), 0, s, p.hpart, p.ddecay,
                           p.B, p.H);
    return hipGetLastError();
}

template <typename TI, int MODE, bool NORM>
hipError_t launch_rpt(const LARecBwdParams &p, int rpt, int nt, hipStream_t s) {
    switch (rpt) {
        case 1: return launch_sweeps<TI, 1, MODE, NORM>(p, nt, s);
        case 2: return launch_sweeps<TI, 2, MODE, NORM>(p, nt, s);
        case 4: return launch_sweeps<TI, 4, MODE, NORM>(p, nt, s);
        case 8: return launch_sweeps<TI, 8, MODE, NORM>(p, nt, s);
        case 16: return launch_sweeps<TI, 16, MODE, NORM>(p, nt, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename TI, bool NORM>
hipError_t launch_mode(const LARecBwdParams &p, int rpt, int nt, hipStream_t s) {
    switch (p.mode) {
        case 0: return launch_rpt<TI, 0, NORM>(p, rpt, nt, s);
        case 1: return launch_rpt<TI, 1, NORM>(p, rpt, nt, s);
        case 2: return launch_rpt<TI, 2, NORM>(p, rpt, nt, s);
        case 3: return launch_rpt<TI, 3, NORM>(p, rpt, nt, s);
        default: return hipErrorInvalidValue;
    }
}

size_t r256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

size_t la_rec_bwd_ws_bytes(int B, int H, int T, int Dk, int Dv, bool normalize, bool ddecay, bool final_terms) {
    const size_t units = (size_t)B * H;
    size_t n = 0;
    if (ddecay) n += r256(units * T * Dk * 4);                                // dq32
    if (normalize) n += r256(units * T * Dv * 4) + r256(units * T * 4);       // a32, c32
    if (ddecay && final_terms) n += r256(units * Dk * Dv * 4) + r256(units * Dk * 4);   // sfin, zfin
    if (ddecay) n += r256(units * 4);                                         // hpart
    return n;
}

hipError_t la_rec_bwd_launch(const LARecBwdParams &p, bool bf16, hipStream_t s) {
    const int nt = la_rec_threads(p.Dk, p.Dv);
    const int rpt = p.Dk * p.Dv / 4 / nt;
    if (bf16) return p.normalize ? launch_mode<uint16_t, true>(p, rpt, nt, s) : launch_mode<uint16_t, false>(p, rpt, nt, s);
    return p.normalize ? launch_mode<float, true>(p, rpt, nt, s) : launch_mode<float, false>(p, rpt, nt, s);
}

}  // namespace drs
