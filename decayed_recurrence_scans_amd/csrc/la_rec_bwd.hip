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
// running sum of the reverse sweep (summed over i for scalar factors).
//
// Both sweeps compute in fp64 (inputs are fp32 or bf16, exact in fp64): the state,
// key sum and their gradients run over the whole sequence, and dq = S a + z c and
// dk = G v + Gz are differences of parts that can be tens of times larger than the
// result.  In fp32 a 2000-step normalised call used up to 0.66 of the fp32 bar on
// dq and missed it on a per-step factor gradient.  This kernel is bound by its
// per-step chain, not by arithmetic.
//
// Time segments: with few (b, h) units each sweep splits the sequence into nseg
// segments that run in parallel.  Both recurrences are linear in their state, so a
// segment's effect on the state is a summary -- forward: S_out = Gamma S_in + dS,
// z_out = Gamma z_in + dz; reverse: G_in = Gamma G_out + dG, Gz likewise -- with Gamma
// the product of the segment's factors (per key row).  Summary kernels form these
// from a zero state without any reductions (elementwise per step); a sweep
// workgroup folds the summaries of the segments before it (forward) or after it
// (reverse) in a fixed order into its entering state.  The factor gradient's running
// sum restarts at each segment; a last kernel adds the later segments' totals.
//
// Layout as the forward step-by-step kernel: one workgroup per (b, h, segment); thread (rg,
// quad) holds columns 4 quad .. 4 quad + 3 of rows rg + RG i of the state (and of
// its gradient), i < RPT.  Sums over a row's columns are lane exchanges; sums over
// rows go through lane exchanges inside a wave and LDS across waves (two buffers
// alternating by step, one barrier per step).
#include "common.h"
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

// Up to 16 waves per workgroup: at Dk = Dv = 128 each thread then holds 4 rows, a
// quarter of the serial work per step of 256-thread workgroups (16 rows each).
constexpr int kThreads = 1024;
constexpr int kMaxWaves = kThreads / 64;

int bwd_threads(int Dk, int Dv) {
    const int quads = Dk * Dv / 4;
    return quads < kThreads ? quads : kThreads;
}

// factor of key row d at staged step n
template <int MODE>
__device__ __forceinline__ float factor_of(const float *sg, float gh, int n, int d, int Dk) {
    if constexpr (MODE == 0) return 1.f;
    else if constexpr (MODE == 1) return gh;
    else if constexpr (MODE == 2) return sg[n];
    else return sg[n * Dk + d];
}

// Sums of a thread's RPT row values over the QPR lanes that hold the other columns
// of the same rows (lanes differing in the bits below log2 QPR).  A butterfly that
// hands half of the rows to the partner lane at each of the first log2 RPT steps,
// so each lane ends with the full sum of one row, row_of(lane): 2 + log2 QPR - 1
// exchanges for four rows instead of 4 log2 QPR.  RPT <= QPR / 2.
template <int RPT>
__device__ __forceinline__ int row_of(int lane, int QPR) {
    if constexpr (RPT == 4) return ((lane & (QPR >> 1)) ? 2 : 0) + ((lane & (QPR >> 2)) ? 1 : 0);
    else if constexpr (RPT == 2) return (lane & (QPR >> 1)) ? 1 : 0;
    else return 0;
}
template <int RPT>
__device__ __forceinline__ double row_sums(const double (&p)[RPT], int lane, int QPR) {
    double v;
    int m;
    if constexpr (RPT == 4) {
        const bool h1 = lane & (QPR >> 1), h2 = lane & (QPR >> 2);
        // rows {0, 1} stay with the lanes below the half, {2, 3} with those above
        double k0 = h1 ? p[2] : p[0], k1 = h1 ? p[3] : p[1];
        k0 += __shfl_xor(h1 ? p[0] : p[2], QPR >> 1, 64);
        k1 += __shfl_xor(h1 ? p[1] : p[3], QPR >> 1, 64);
        v = h2 ? k1 : k0;
        v += __shfl_xor(h2 ? k0 : k1, QPR >> 2, 64);
        m = QPR >> 3;
    } else if constexpr (RPT == 2) {
        const bool h1 = lane & (QPR >> 1);
        v = h1 ? p[1] : p[0];
        v += __shfl_xor(h1 ? p[0] : p[1], QPR >> 1, 64);
        m = QPR >> 2;
    } else {
        v = p[0];
        m = QPR >> 1;
    }
    for (; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
// a[r] for a lane-dependent r without dynamic register indexing
template <int RPT>
__device__ __forceinline__ double pick(const double (&a)[RPT], int r) {
    double v = a[0];
#pragma unroll
    for (int i = 1; i < RPT; ++i) v = r == i ? a[i] : v;
    return v;
}

// The nw (<= kMaxWaves) wave partials base[0], base[stride], ... added in wave order,
// the loads issued ahead of the adds (a loop bounded by the runtime wave count waited
// for each load in turn: sixteen LDS round trips in a row on every step).
// (Two batches of eight loads: sixteen doubles at once spilled at 1024 threads.)
__device__ __forceinline__ double sum_waves(const double *base, int stride, int nw) {
    constexpr int kBatch = 8;
    double s = 0.0;
#pragma unroll
    for (int w0 = 0; w0 < kMaxWaves; w0 += kBatch) {
        double v[kBatch];
#pragma unroll
        for (int i = 0; i < kBatch; ++i) v[i] = w0 + i < nw ? base[(w0 + i) * stride] : 0.0;
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (w0 + i < nw) s += v[i];
    }
    return s;
}

// doubles per segment summary: forward S, z, factor product; reverse G, Gz
__host__ __device__ __forceinline__ size_t agg_f_len(int Dk, int Dv) { return (size_t)Dk * Dv + 2 * (size_t)Dk; }
__host__ __device__ __forceinline__ size_t agg_r_len(int Dk, int Dv) { return (size_t)Dk * Dv + (size_t)Dk; }

// ---- forward summaries: each segment from a zero state ------------------------------
// S <- g S + k v^T, z <- g z + k and the product of the factors, per key row; no sums
// across threads.  Every segment (the last one's product is the reverse fold's).
template <typename TI, int RPT, int MODE, bool NORM>
__global__ __launch_bounds__(kThreads) void la_rbwd_sumf(LARecBwdParams p) {
    extern __shared__ f32x4 smem4[];
    const int Dk = p.Dk, Dv = p.Dv, T = p.T, TB = p.tb;
    const int NT = blockDim.x, QPR = Dv >> 2, RG = NT / QPR;
    const int tid = threadIdx.x, quad = tid % QPR, rg = tid / QPR;
    const int bh = blockIdx.x / p.nseg, seg = blockIdx.x - bh * p.nseg;
    const int nbeg = seg * p.seg_len, nend = min(T, nbeg + p.seg_len);
    float *sv = reinterpret_cast<float *>(smem4);   // [TB][Dv]
    float *sk = sv + TB * Dv;                        // [TB][Dk]
    float *sg = sk + TB * Dk;                        // [TB][Dk] | [TB]
    double S[RPT][4], z[RPT], gam[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) S[i][r] = 0.0;
        z[i] = 0.0;
        gam[i] = 1.0;
    }
    const float gh = MODE == 1 ? p.decay[bh % p.H] : 1.f;
    const TI *kg = static_cast<const TI *>(p.k) + (size_t)bh * T * Dk;
    const TI *vg = static_cast<const TI *>(p.v) + (size_t)bh * T * Dv;
    const int dk_shift = __builtin_ctz(Dk), dv_shift = __builtin_ctz(Dv);
    for (int n0 = nbeg; n0 < nend; n0 += TB) {
        const int nb = nend - n0 < TB ? nend - n0 : TB;
        for (int e = tid; e < nb * Dk; e += NT) {
            const int n = e >> dk_shift, d = e & (Dk - 1);
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            sk[e] = load_in<TI>(kg, (size_t)t * Dk + d);
            if constexpr (MODE == 3) sg[e] = p.decay[((size_t)bh * T + t) * Dk + d];
        }
        for (int e = tid; e < nb * Dv; e += NT) {
            const int n = e >> dv_shift, j = e & (Dv - 1);
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            sv[e] = load_in<TI>(vg, (size_t)t * Dv + j);
        }
        if constexpr (MODE == 2) {
            for (int n = tid; n < nb; n += NT) {
                const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
                sg[n] = p.decay[(size_t)bh * T + t];
            }
        }
        __syncthreads();
        for (int n = 0; n < nb; ++n) {
            const float *kn = sk + n * Dk;
            const f32x4 v4 = *reinterpret_cast<const f32x4 *>(sv + n * Dv + 4 * quad);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int d = rg + RG * i;
                const double g = factor_of<MODE>(sg, gh, n, d, Dk), kd = kn[d];
#pragma unroll
                for (int r = 0; r < 4; ++r) S[i][r] = fma(kd, (double)v4[r], g * S[i][r]);
                if constexpr (NORM) z[i] = fma(g, z[i], kd);
                if constexpr (MODE != 0) gam[i] *= g;
            }
        }
        __syncthreads();   // the staged block is replaced next
    }
    double *ag = p.aggF + ((size_t)bh * p.nseg + seg) * agg_f_len(Dk, Dv);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int d = rg + RG * i;
#pragma unroll
        for (int r = 0; r < 4; ++r) ag[(size_t)d * Dv + 4 * quad + r] = S[i][r];
        if (quad == 0) {
            ag[Dk * Dv + d] = z[i];
            ag[Dk * Dv + Dk + d] = gam[i];
        }
    }
}

// ---- reverse summaries: each segment but the first from a zero gradient -------------
// Visiting the segment backward: G <- g (G + q a^T), Gz <- g (Gz + q c), with a, c
// from the forward sweep (a = dy, c = 0 without the normaliser).
template <typename TI, int RPT, int MODE, bool NORM>
__global__ __launch_bounds__(kThreads) void la_rbwd_sumr(LARecBwdParams p) {
    extern __shared__ f32x4 smem4[];
    const int Dk = p.Dk, Dv = p.Dv, T = p.T, TB = p.tb;
    const int NT = blockDim.x, QPR = Dv >> 2, RG = NT / QPR;
    const int tid = threadIdx.x, quad = tid % QPR, rg = tid / QPR;
    const int bh = blockIdx.x / (p.nseg - 1), seg = 1 + (int)(blockIdx.x - bh * (p.nseg - 1));
    const int nbeg = seg * p.seg_len, nend = min(T, nbeg + p.seg_len);
    double *sa = reinterpret_cast<double *>(smem4);   // [TB][Dv]
    double *sc = sa + TB * Dv;                         // [TB] (NORM), padded to even
    float *sq = reinterpret_cast<float *>(sc + (NORM ? (TB + 1) / 2 * 2 : 0));   // [TB][Dk]
    float *sg = sq + TB * Dk;                          // [TB][Dk] | [TB]
    double G[RPT][4], Gz[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) G[i][r] = 0.0;
        Gz[i] = 0.0;
    }
    const float gh = MODE == 1 ? p.decay[bh % p.H] : 1.f;
    const TI *qg = static_cast<const TI *>(p.q) + (size_t)bh * T * Dk;
    const TI *dyg = static_cast<const TI *>(p.dy) + (size_t)bh * T * Dv;
    const int dk_shift = __builtin_ctz(Dk), dv_shift = __builtin_ctz(Dv);
    const int nblk = (nend - nbeg + TB - 1) / TB;
    for (int bi = nblk - 1; bi >= 0; --bi) {
        const int n0 = nbeg + bi * TB, nb = nend - n0 < TB ? nend - n0 : TB;
        for (int e = tid; e < nb * Dk; e += NT) {
            const int n = e >> dk_shift, d = e & (Dk - 1);
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            sq[e] = load_in<TI>(qg, (size_t)t * Dk + d);
            if constexpr (MODE == 3) sg[e] = p.decay[((size_t)bh * T + t) * Dk + d];
        }
        for (int e = tid; e < nb * Dv; e += NT) {
            const int n = e >> dv_shift, j = e & (Dv - 1);
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            if constexpr (NORM) sa[e] = p.a64[((size_t)bh * T + t) * Dv + j];
            else sa[e] = load_in<TI>(dyg, (size_t)t * Dv + j);
        }
        for (int n = tid; n < nb; n += NT) {
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            if constexpr (NORM) sc[n] = p.c64[(size_t)bh * T + t];
            if constexpr (MODE == 2) sg[n] = p.decay[(size_t)bh * T + t];
        }
        __syncthreads();
        for (int n = nb - 1; n >= 0; --n) {
            const float *qn = sq + n * Dk;
            const double *a4 = sa + n * Dv + 4 * quad;
            const double c = NORM ? sc[n] : 0.0;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int d = rg + RG * i;
                const double qd = qn[d], g = factor_of<MODE>(sg, gh, n, d, Dk);
#pragma unroll
                for (int r = 0; r < 4; ++r) G[i][r] = g * fma(qd, a4[r], G[i][r]);
                if constexpr (NORM) Gz[i] = g * fma(qd, c, Gz[i]);
            }
        }
        __syncthreads();
    }
    double *ag = p.aggR + ((size_t)bh * p.nseg + seg) * agg_r_len(Dk, Dv);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int d = rg + RG * i;
#pragma unroll
        for (int r = 0; r < 4; ++r) ag[(size_t)d * Dv + 4 * quad + r] = G[i][r];
        if (quad == 0) ag[Dk * Dv + d] = Gz[i];
    }
}

// ---- the factor gradient across segments --------------------------------------------
// g dL/dg at visited step n of segment j = (the running sum inside j) + (the totals of
// the segments after j), divided by the factor; fp64 until the one rounding.
template <int MODE>
__global__ void la_rbwd_fix(LARecBwdParams p) {
    const int T = p.T, Dk = p.Dk, L = p.seg_len, P = p.nseg;
    constexpr bool ELEM = MODE == 3;
    const size_t per = ELEM ? (size_t)Dk : 1;
    const size_t total = (size_t)p.B * p.H * T * per;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (size_t)gridDim.x * blockDim.x) {
        const size_t bt = e / per;
        const int d = (int)(e - bt * per);
        const int bh = (int)(bt / T), n = (int)(bt - (size_t)bh * T);
        const int t = p.reverse ? T - 1 - n : n;
        double tail = 0.0;
        for (int j = P - 1; j > n / L; --j) tail += p.eseg[((size_t)bh * P + j) * Dk + d];
        const size_t mi = ((size_t)bh * T + t) * per + d;
        p.ddecay[mi] = (float)((p.rloc[e] + tail) / (double)p.decay[mi]);
    }
}

// per-head factor: the per-unit sum over the steps, in a fixed order (deterministic)
__global__ __launch_bounds__(256) void la_rbwd_fix_head(LARecBwdParams p) {
    __shared__ double part[256];
    const int T = p.T, Dk = p.Dk, L = p.seg_len, P = p.nseg;
    const int bh = blockIdx.x, tid = threadIdx.x;
    const double g = (double)p.decay[bh % p.H];
    double s = 0.0;
    for (int n = tid; n < T; n += 256) {
        double tail = 0.0;
        for (int j = P - 1; j > n / L; --j) tail += p.eseg[((size_t)bh * P + j) * Dk];
        s += (p.rloc[(size_t)bh * T + n] + tail) / g;
    }
    part[tid] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) part[tid] += part[tid + w];
        __syncthreads();
    }
    if (tid == 0) p.hpart[bh] = (float)part[0];
}

// ---- forward sweep: dq, and a_t / c_t for the reverse sweep ------------------------
template <typename TI, int RPT, int MODE, bool NORM>
__global__ __launch_bounds__(kThreads) void la_rbwd_fwd(LARecBwdParams p) {
    extern __shared__ f32x4 smem4[];
    const int Dk = p.Dk, Dv = p.Dv, T = p.T, TB = p.tb;
    const int NT = blockDim.x, QPR = Dv >> 2, RG = NT / QPR;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = NT >> 6;
    const int quad = tid % QPR, rg = tid / QPR;
    const int ro = row_of<RPT>(lane, QPR);              // the row whose column sums this lane ends with
    const bool owner = (quad & (QPR / RPT - 1)) == 0;   // one lane per (row group, row) stores
    const int bh = blockIdx.x / p.nseg, seg = blockIdx.x - bh * p.nseg;
    const int nbeg = seg * p.seg_len, nend = min(T, nbeg + p.seg_len);

    double *red = reinterpret_cast<double *>(smem4);                 // [2][nw][QPR][4]
    double *rden = red + 2 * nw * QPR * 4;                           // [2][kMaxWaves]
    double *tot = rden + 2 * kMaxWaves;                              // [2][Dv + 2]: n_t, d_t
    float *sv = reinterpret_cast<float *>(tot + 2 * (Dv + 2));       // [TB][Dv]
    float *sdy = sv + TB * Dv;                                       // [TB][Dv]
    float *sq = sdy + TB * Dv;                                       // [TB][Dk]
    float *sk = sq + TB * Dk;                                        // [TB][Dk]
    float *sg = sk + TB * Dk;                                        // [TB][Dk] | [TB]

    double S[RPT][4], z[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int d = rg + RG * i;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[i][r] = p.state_in ? (double)p.state_in[((size_t)bh * Dk + d) * Dv + 4 * quad + r] : 0.0;
        z[i] = (NORM && p.cum_k_in) ? (double)p.cum_k_in[(size_t)bh * Dk + d] : 0.0;
    }
    // the earlier segments' summaries, in order
    for (int j = 0; j < seg; ++j) {
        const double *ag = p.aggF + ((size_t)bh * p.nseg + j) * agg_f_len(Dk, Dv);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int d = rg + RG * i;
            const double gam = ag[Dk * Dv + Dk + d];
#pragma unroll
            for (int r = 0; r < 4; ++r) S[i][r] = fma(gam, S[i][r], ag[(size_t)d * Dv + 4 * quad + r]);
            if constexpr (NORM) z[i] = fma(gam, z[i], ag[Dk * Dv + d]);
        }
    }
    const float gh = MODE == 1 ? p.decay[bh % p.H] : 1.f;
    const TI *qg = static_cast<const TI *>(p.q) + (size_t)bh * T * Dk;
    const TI *kg = static_cast<const TI *>(p.k) + (size_t)bh * T * Dk;
    const TI *vg = static_cast<const TI *>(p.v) + (size_t)bh * T * Dv;
    const TI *dyg = static_cast<const TI *>(p.dy) + (size_t)bh * T * Dv;
    TI *dqg = static_cast<TI *>(p.dq) + (size_t)bh * T * Dk;
    const int dk_shift = __builtin_ctz(Dk), dv_shift = __builtin_ctz(Dv);

    int par = 0;
    for (int n0 = nbeg; n0 < nend; n0 += TB) {
        const int nb = nend - n0 < TB ? nend - n0 : TB;
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
            double acc[4] = {0.0, 0.0, 0.0, 0.0}, dacc = 0.0;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int d = rg + RG * i;
                const double g = factor_of<MODE>(sg, gh, n, d, Dk);
                const double kd = kn[d], qd = qn[d];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    S[i][r] = fma(kd, (double)vq[r], g * S[i][r]);
                    if constexpr (NORM) acc[r] = fma(qd, S[i][r], acc[r]);
                }
                if constexpr (NORM) {
                    z[i] = fma(g, z[i], kd);
                    dacc = fma(qd, z[i], dacc);
                }
            }
            double a4[4] = {dy4[0], dy4[1], dy4[2], dy4[3]}, c = 0.0;
            if constexpr (NORM) {
                // n_t (this thread's four columns) and d_t, summed over every row
                for (int m = QPR; m < 64; m <<= 1) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] += __shfl_xor(acc[r], m, 64);
                    dacc += __shfl_xor(dacc, m, 64);
                }
                if (lane < QPR) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) red[((par * nw + wv) * QPR + quad) * 4 + r] = acc[r];
                }
                if (lane == 0) rden[par * kMaxWaves + wv] = dacc;
                __syncthreads();
                // the waves' partial sums added once per column (and once for d_t), in
                // wave order, instead of by every thread for its own columns
                if (tid <= Dv) {
                    const double sum = tid < Dv ? sum_waves(red + par * nw * QPR * 4 + tid, QPR * 4, nw)
                                                : sum_waves(rden + par * kMaxWaves, 1, nw);
                    tot[par * (Dv + 2) + tid] = sum;
                }
                __syncthreads();
                double num[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) num[r] = tot[par * (Dv + 2) + 4 * quad + r];
                const double inv = 1.0 / tot[par * (Dv + 2) + Dv];   // 1 / d_t
                double dyy = 0.0;   // dy_t . y_t
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    a4[r] = (double)dy4[r] * inv;
                    dyy = fma((double)dy4[r], num[r] * inv, dyy);
                }
                for (int m = 1; m < QPR; m <<= 1) dyy += __shfl_xor(dyy, m, 64);
                c = -dyy * inv;
                if (wv == 0 && lane < QPR) {
                    double *ad = p.a64 + ((size_t)bh * T + t) * Dv + 4 * quad;
#pragma unroll
                    for (int r = 0; r < 4; ++r) ad[r] = a4[r];
                    if (quad == 0) p.c64[(size_t)bh * T + t] = c;
                }
            }
            // dq_t = S_t a_t + z_t c_t: the lane ends with row ro's sum over the columns
            double part[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                part[i] = S[i][0] * a4[0];
#pragma unroll
                for (int r = 1; r < 4; ++r) part[i] = fma(S[i][r], a4[r], part[i]);
            }
            double dqr = row_sums<RPT>(part, lane, QPR);
            if constexpr (NORM) dqr = fma(pick<RPT>(z, ro), c, dqr);
            if (owner) {
                const int d = rg + RG * ro;
                store_out(dqg, (size_t)t * Dk + d, (float)dqr);
                if (p.dq64) p.dq64[((size_t)bh * T + t) * Dk + d] = dqr;
            }
            par ^= 1;
        }
        __syncthreads();   // every wave is done with the staged block before it is replaced
    }
    if (seg != p.nseg - 1) return;
    if (p.sfin) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int d = rg + RG * i;
#pragma unroll
            for (int r = 0; r < 4; ++r) p.sfin[((size_t)bh * Dk + d) * Dv + 4 * quad + r] = S[i][r];
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
    const int ro = row_of<RPT>(lane, QPR);              // the row whose column sums this lane ends with
    const bool owner = (quad & (QPR / RPT - 1)) == 0;   // one lane per (row group, row) stores
    const int bh = blockIdx.x / p.nseg, seg = blockIdx.x - bh * p.nseg;
    const int nbeg = seg * p.seg_len, nend = min(T, nbeg + p.seg_len);
    const bool last = seg == p.nseg - 1;
    constexpr bool SCALAR = MODE == 1 || MODE == 2;   // one factor for every key row

    double *red = reinterpret_cast<double *>(smem4);                 // [2][nw][QPR][4]
    double *rsum = red + 2 * nw * QPR * 4;                           // [2][kMaxWaves]
    double *sa = rsum + 2 * kMaxWaves;                               // [TB][Dv] a_t (dy_t)
    double *sdq = sa + TB * Dv;                                      // [TB][Dk] (DG)
    double *sc = sdq + (DG ? TB * Dk : 0);                           // [TB] (NORM), padded to even
    float *sv = reinterpret_cast<float *>(sc + (NORM ? (TB + 1) / 2 * 2 : 0));   // [TB][Dv], 16-byte aligned
    float *sq = sv + TB * Dv;                                        // [TB][Dk]
    float *sk = sq + TB * Dk;                                        // [TB][Dk]
    float *sg = sk + TB * Dk;                                        // [TB][Dk] | [TB]

    double G[RPT][4], Gz[RPT];
    double Rown = 0.0;   // the factor gradient's running sum of row rg + RG ro (per key channel)
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int d = rg + RG * i;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            G[i][r] = p.dstate_out ? (double)p.dstate_out[((size_t)bh * Dk + d) * Dv + 4 * quad + r] : 0.0;
        Gz[i] = (NORM && p.dcum_k_out) ? (double)p.dcum_k_out[(size_t)bh * Dk + d] : 0.0;
    }
    double Rtot = 0.0, hsum = 0.0;
    if (DG && last) {
        // the final-state terms <dS_final[i,:], S_final[i,:]> + dz_final[i] z_final[i]
        double part[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int d = rg + RG * i;
            part[i] = 0.0;
            if (p.dstate_out) {
#pragma unroll
                for (int r = 0; r < 4; ++r) part[i] += G[i][r] * p.sfin[((size_t)bh * Dk + d) * Dv + 4 * quad + r];
            }
        }
        Rown = row_sums<RPT>(part, lane, QPR);
        if (NORM && p.dcum_k_out) Rown += pick<RPT>(Gz, ro) * p.zfin[(size_t)bh * Dk + rg + RG * ro];
        double rows = owner ? Rown : 0.0;
        if constexpr (SCALAR) {
            for (int m = 1; m < 64; m <<= 1) rows += __shfl_xor(rows, m, 64);
            if (lane == 0) rsum[kMaxWaves + wv] = rows;   // parity 1: the first step writes parity 0
            __syncthreads();
            if (tid == 0)
                for (int w2 = 0; w2 < nw; ++w2) Rtot += rsum[kMaxWaves + w2];
        }
    }
    // the later segments' summaries, nearest last
    for (int j = p.nseg - 1; j > seg; --j) {
        const double *gf = p.aggF + ((size_t)bh * p.nseg + j) * agg_f_len(Dk, Dv);
        const double *gr = p.aggR + ((size_t)bh * p.nseg + j) * agg_r_len(Dk, Dv);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int d = rg + RG * i;
            const double gam = gf[Dk * Dv + Dk + d];
#pragma unroll
            for (int r = 0; r < 4; ++r) G[i][r] = fma(gam, G[i][r], gr[(size_t)d * Dv + 4 * quad + r]);
            if constexpr (NORM) Gz[i] = fma(gam, Gz[i], gr[Dk * Dv + d]);
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
    const int nblk = (nend - nbeg + TB - 1) / TB;
    for (int bi = nblk - 1; bi >= 0; --bi) {
        const int n0 = nbeg + bi * TB, nb = nend - n0 < TB ? nend - n0 : TB;
        for (int e = tid; e < nb * Dk; e += NT) {
            const int n = e >> dk_shift, d = e & (Dk - 1);
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            sq[e] = load_in<TI>(qg, (size_t)t * Dk + d);
            sk[e] = load_in<TI>(kg, (size_t)t * Dk + d);
            if constexpr (DG) sdq[e] = p.dq64[((size_t)bh * T + t) * Dk + d];
            if constexpr (MODE == 3) sg[e] = p.decay[((size_t)bh * T + t) * Dk + d];
        }
        for (int e = tid; e < nb * Dv; e += NT) {
            const int n = e >> dv_shift, j = e & (Dv - 1);
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            sv[e] = load_in<TI>(vg, (size_t)t * Dv + j);
            if constexpr (NORM) sa[e] = p.a64[((size_t)bh * T + t) * Dv + j];
            else sa[e] = load_in<TI>(dyg, (size_t)t * Dv + j);
        }
        for (int n = tid; n < nb; n += NT) {
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            if constexpr (NORM) sc[n] = p.c64[(size_t)bh * T + t];
            if constexpr (MODE == 2) sg[n] = p.decay[(size_t)bh * T + t];
        }
        __syncthreads();

        for (int n = nb - 1; n >= 0; --n) {
            const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
            const float *qn = sq + n * Dk, *kn = sk + n * Dk;
            const f32x4 v4 = *reinterpret_cast<const f32x4 *>(sv + n * Dv + 4 * quad);
            const double *a4 = sa + n * Dv + 4 * quad;
            const double c = NORM ? sc[n] : 0.0;
            double dv4[4] = {0.0, 0.0, 0.0, 0.0}, epart = 0.0, part[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int d = rg + RG * i;
                const double qd = qn[d], kd = kn[d];
                part[i] = 0.0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    G[i][r] = fma(qd, a4[r], G[i][r]);
                    part[i] = fma(G[i][r], (double)v4[r], part[i]);
                    dv4[r] = fma(G[i][r], kd, dv4[r]);
                }
                if constexpr (NORM) Gz[i] = fma(qd, c, Gz[i]);
            }
            {   // dk of row dro = rg + RG ro, whose column sum this lane ends with
                const int dro = rg + RG * ro;
                double dko = row_sums<RPT>(part, lane, QPR);
                if constexpr (NORM) dko += pick<RPT>(Gz, ro);
                if (owner) store_out(dkg, (size_t)t * Dk + dro, (float)dko);
                if constexpr (DG) {
                    const double e = (double)qn[dro] * sdq[n * Dk + dro] - (double)kn[dro] * dko;
                    if constexpr (MODE == 3) {
                        Rown += e;
                        if (owner) {
                            if (p.rloc) p.rloc[((size_t)bh * T + n0 + n) * Dk + dro] = Rown;
                            else p.ddecay[((size_t)bh * T + t) * Dk + dro] =
                                (float)(Rown / (double)factor_of<MODE>(sg, gh, n, dro, Dk));
                        }
                    } else {
                        epart += owner ? e : 0.0;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const double g = factor_of<MODE>(sg, gh, n, rg + RG * i, Dk);
#pragma unroll
                for (int r = 0; r < 4; ++r) G[i][r] *= g;
                if constexpr (NORM) Gz[i] *= g;
            }
            for (int m = QPR; m < 64; m <<= 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r) dv4[r] += __shfl_xor(dv4[r], m, 64);
            }
            if (lane < QPR) {
#pragma unroll
                for (int r = 0; r < 4; ++r) red[((par * nw + wv) * QPR + quad) * 4 + r] = dv4[r];
            }
            if constexpr (DG && SCALAR) {
                for (int m = 1; m < 64; m <<= 1) epart += __shfl_xor(epart, m, 64);
                if (lane == 0) rsum[par * kMaxWaves + wv] = epart;
            }
            __syncthreads();
            // dv: one thread per column (index 4 quad + r of the partials) sums the waves
            if (tid < Dv)
                store_out(dvg, (size_t)t * Dv + tid, (float)sum_waves(red + par * nw * QPR * 4 + tid, QPR * 4, nw));
            if constexpr (DG && SCALAR) {
                if (tid == 0) {
                    const double e = sum_waves(rsum + par * kMaxWaves, 1, nw);
                    Rtot += e;
                    if (p.rloc) {
                        p.rloc[(size_t)bh * T + n0 + n] = Rtot;
                    } else {
                        const double dg = Rtot / (double)factor_of<MODE>(sg, gh, n, 0, Dk);
                        if constexpr (MODE == 2) p.ddecay[(size_t)bh * T + t] = (float)dg;
                        else hsum += dg;
                    }
                }
            }
            par ^= 1;
        }
        __syncthreads();
    }
    if (DG && p.rloc) {   // this segment's totals (the first visited step's running sums)
        double *es = p.eseg + ((size_t)bh * p.nseg + seg) * Dk;
        if constexpr (MODE == 3) {
            if (owner) es[rg + RG * ro] = Rown;
        } else if (tid == 0) {
            es[0] = Rtot;
        }
    }
    if (seg != 0) return;
    if (p.dstate_in) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int d = rg + RG * i;
#pragma unroll
            for (int r = 0; r < 4; ++r) p.dstate_in[((size_t)bh * Dk + d) * Dv + 4 * quad + r] = (float)G[i][r];
        }
    }
    if (NORM && p.dcum_k_in && quad == 0) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) p.dcum_k_in[(size_t)bh * Dk + rg + RG * i] = (float)Gz[i];
    }
    if (DG && MODE == 1 && !p.rloc && tid == 0) p.hpart[bh] = (float)hsum;
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
    return (size_t)2 * nw * qpr * 32 + 2 * kMaxWaves * 8 + (size_t)2 * (p.Dv + 2) * 8 +
           (size_t)p.tb * (2 * p.Dk + 2 * p.Dv + gcols) * 4;
}
size_t rev_lds(const LARecBwdParams &p, int nt, bool dg) {
    const int nw = nt / 64, qpr = p.Dv / 4;
    const int gcols = p.mode == 3 ? p.Dk : (p.mode == 2 ? 1 : 0);
    return (size_t)2 * nw * qpr * 32 + 2 * kMaxWaves * 8 +
           (size_t)p.tb * ((p.Dv + (dg ? p.Dk : 0)) * 8 + (2 * p.Dk + p.Dv + gcols) * 4) +
           (p.normalize ? (size_t)(p.tb + 1) / 2 * 2 * 8 : 0);
}

size_t sumf_lds(const LARecBwdParams &p) {
    const int gcols = p.mode == 3 ? p.Dk : (p.mode == 2 ? 1 : 0);
    return (size_t)p.tb * (p.Dk + p.Dv + gcols) * 4;
}
size_t sumr_lds(const LARecBwdParams &p) {
    const int gcols = p.mode == 3 ? p.Dk : (p.mode == 2 ? 1 : 0);
    return (size_t)p.tb * p.Dv * 8 + (p.normalize ? (size_t)(p.tb + 1) / 2 * 2 * 8 : 0) +
           (size_t)p.tb * (p.Dk + gcols) * 4;
}

template <typename TI, int RPT, int MODE, bool NORM>
hipError_t launch_sweeps(const LARecBwdParams &p, int nt, hipStream_t s) {
    const unsigned units = (unsigned)(p.B * p.H), P = (unsigned)p.nseg;
    const dim3 grid(units * P), block((unsigned)nt);
    if (P > 1) hipLaunchKernelGGL((la_rbwd_sumf<TI, RPT, MODE, NORM>), grid, block, sumf_lds(p), s, p);
    hipLaunchKernelGGL((la_rbwd_fwd<TI, RPT, MODE, NORM>), grid, block, fwd_lds(p, nt), s, p);
    if (P > 1) hipLaunchKernelGGL((la_rbwd_sumr<TI, RPT, MODE, NORM>), dim3(units * (P - 1)), block, sumr_lds(p), s, p);
    if (p.ddecay && MODE != 0)
        hipLaunchKernelGGL((la_rbwd_rev<TI, RPT, MODE, NORM, MODE != 0>), grid, block, rev_lds(p, nt, true), s, p);
    else
        hipLaunchKernelGGL((la_rbwd_rev<TI, RPT, MODE, NORM, false>), grid, block, rev_lds(p, nt, false), s, p);
    if (p.ddecay && MODE != 0 && p.rloc) {
        if constexpr (MODE == 1) {
            hipLaunchKernelGGL(la_rbwd_fix_head, dim3(units), dim3(256), 0, s, p);
        } else {
            const size_t n = (size_t)units * p.T * (MODE == 3 ? p.Dk : 1);
            const size_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
            hipLaunchKernelGGL(la_rbwd_fix<MODE>, dim3((unsigned)blocks), dim3(256), 0, s, p);
        }
    }
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

int la_rec_bwd_nseg(int B, int H, int T) {
    // about one 1024-thread workgroup per compute unit (256), segments of at least 256 steps
    const long units = (long)B * H;
    long P = (256 + units - 1) / units;
    const long pmax = T / 256 > 1 ? T / 256 : 1;
    if (P > pmax) P = pmax;
    if (P > 16) P = 16;
    return (int)(P < 1 ? 1 : P);
}

namespace {
// Walks the workspace layout: with ws == nullptr only counts the bytes.
size_t rec_bwd_layout(char *ws, int B, int H, int T, int Dk, int Dv, int mode, bool normalize, bool ddecay,
                      bool final_terms, LARecBwdParams *p) {
    const size_t units = (size_t)B * H;
    const int P = la_rec_bwd_nseg(B, H, T);
    size_t off = 0;
    auto take = [&](size_t bytes) -> double * {
        double *r = ws ? reinterpret_cast<double *>(ws + off) : nullptr;
        off += r256(bytes);
        return r;
    };
    double *dq64 = ddecay ? take(units * T * Dk * 8) : nullptr;
    double *a64 = normalize ? take(units * T * Dv * 8) : nullptr;
    double *c64 = normalize ? take(units * T * 8) : nullptr;
    double *sfin = ddecay && final_terms ? take(units * Dk * Dv * 8) : nullptr;
    double *zfin = ddecay && final_terms ? take(units * Dk * 8) : nullptr;
    float *hpart = ddecay ? reinterpret_cast<float *>(take(units * 4)) : nullptr;
    double *aggF = P > 1 ? take(units * P * agg_f_len(Dk, Dv) * 8) : nullptr;
    double *aggR = P > 1 ? take(units * P * agg_r_len(Dk, Dv) * 8) : nullptr;
    const bool seg_dg = P > 1 && ddecay && mode != 0;
    double *rloc = seg_dg ? take(units * T * (mode == 3 ? Dk : 1) * 8) : nullptr;
    double *eseg = seg_dg ? take(units * P * Dk * 8) : nullptr;
    if (p) {
        p->dq64 = dq64; p->a64 = a64; p->c64 = c64; p->sfin = sfin; p->zfin = zfin; p->hpart = hpart;
        p->aggF = aggF; p->aggR = aggR; p->rloc = rloc; p->eseg = eseg;
        p->nseg = P;
        p->seg_len = (T + P - 1) / P;
    }
    return off;
}
}  // namespace

size_t la_rec_bwd_ws_bytes(int B, int H, int T, int Dk, int Dv, int mode, bool normalize, bool ddecay,
                           bool final_terms) {
    return rec_bwd_layout(nullptr, B, H, T, Dk, Dv, mode, normalize, ddecay, final_terms, nullptr);
}

void la_rec_bwd_layout(char *ws, LARecBwdParams &p, bool final_terms) {
    rec_bwd_layout(ws, p.B, p.H, p.T, p.Dk, p.Dv, p.mode, p.normalize != 0, p.ddecay != nullptr, final_terms, &p);
}

hipError_t la_rec_bwd_launch(const LARecBwdParams &p_in, bool bf16, hipStream_t s) {
    const int nt = bwd_threads(p_in.Dk, p_in.Dv);
    const int rpt = p_in.Dk * p_in.Dv / 4 / nt;   // 1, 2 or 4
    // fewer staged steps where the sweeps would need more than 64 KB of dynamic LDS
    LARecBwdParams p = p_in;
    const bool dg = p.ddecay && p.mode != 0;
    while (p.tb > 1 && (fwd_lds(p, nt) > 65536 || rev_lds(p, nt, dg) > 65536 || sumr_lds(p) > 65536)) p.tb /= 2;
    if (bf16) return p.normalize ? launch_mode<uint16_t, true>(p, rpt, nt, s) : launch_mode<uint16_t, false>(p, rpt, nt, s);
    return p.normalize ? launch_mode<float, true>(p, rpt, nt, s) : launch_mode<float, false>(p, rpt, nt, s);
}

}  // namespace drs
