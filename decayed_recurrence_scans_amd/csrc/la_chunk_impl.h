// la_chunk_impl.h -- chunked causal decayed linear attention, forward, gfx950.
//
// What is computed (definitions: tensortonic "cs336 linear attention duality"
// exercise for the recurrence; RetNet issue #21 for per-step decay factors,
// the decay-mask (Q K^T * D) V parallel form and reverse = flip/forward/flip;
// flash-linear-attention issue #268 for QKV/QK1 normalisation and the cached
// key sum):
//     S_t = g_t S_{t-1} + k_t v_t^T,  z_t = g_t z_{t-1} + k_t,
//     y_t = q_t^T S_t            (or  q_t^T S_t / q_t^T z_t).
//
// How (one workgroup per (b, h, Dv-slice); one wave per time chunk):
//   Time is cut into chunks of C steps.  Within a chunk, with
//   b_t = sum_{r<=t} log2 g_r (inclusive, chunk-local),
//     intra:  O   = (Q K^T (.) M) V,  M[t,s] = 2^(b_t - b_s) for s <= t else 0
//     inter:  O  += diag(2^b_t) Q S_prev
//     state:  dS  = (K (.) 2^(b_last - b_s))^T V,   S_next = 2^b_last S_prev + dS
//   The W waves of a workgroup hold W consecutive chunks.  Each wave computes
//   its chunk's intra part and dS independently (bf16 MFMA, fp32 accumulate),
//   the chunk states are combined through LDS by the associative decayed
//   prefix (x_a, f_a) o (x_b, f_b) = (x_a f_b + x_b, f_a f_b), and the carry
//   stays in LDS for the next group of W chunks.  Nothing but q, k, v, the
//   decay, y and the boundary states touches global memory.
//
// Precision: the mask is applied before exponentiation (every exponent is
// <= 0), the query-side decay 2^b_t is applied in fp32 after the MFMA, and
// the two fp32 operands of the state products (decayed K and S_prev) enter
// the bf16 MFMA as a hi + lo pair of bf16 values, so the state path keeps
// ~16 mantissa bits.  With fp32 inputs the fp32 MFMA is used throughout.
//
// MFMA register layouts (16x16 outputs): lane l = c16 + 16 g (c16 = l & 15,
// g = l >> 4).  Output register r of a 16x16 tile holds row 4g + r, column
// c16.  An A operand supplies row c16 and a B operand column c16; both supply
// the same contraction indices from lane group g.  The contraction index set
// of each lane group is chosen so that every operand can be used straight
// from the layout it was produced in:
//   * dk contractions (Q K^T, Q S): lane group g holds dk = KB p + E g + e
//     (E = 8 / KB = 32 for bf16, E = 4 / KB = 16 for fp32): one 16-byte load;
//   * s contractions (P V, K^T V): lane group g holds s = 16 st + 4 g + r, the
//     rows an output tile register already has, so the masked scores feed the
//     next MFMA without any shuffle.
#pragma once

#include "common.h"

namespace drs {

struct LAParams {
    const void *q, *k, *v;
    void *y;
    const float *decay;
    const float *state_in, *cum_k_in;
    float *state_out, *cum_k_out;
    int B, H, T, Dv, nslice;
    int mode;       // 0 none, 1 head, 2 step
    int reverse;
    int normalize;
    int nchunks, ngroups;
};

template <typename TI> struct InTraits;
template <> struct InTraits<float> {
    static constexpr int E = 4, KB = 16;
    typedef f32x4 Frag;  // 4 fp32 per lane group
};
template <> struct InTraits<uint16_t> {
    static constexpr int E = 8, KB = 32;
    typedef u16x8 Frag;  // 8 bf16 per lane group
};

__device__ __forceinline__ float in_to_f32(float x) { return x; }
__device__ __forceinline__ float in_to_f32(uint16_t x) { return bf16_bits_to_f32(x); }

template <typename TI>
__device__ __forceinline__ void store_out(TI *p, float x);
template <>
__device__ __forceinline__ void store_out<float>(float *p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t *p, float x) { *p = f32_to_bf16_bits(x); }

template <typename TI, int DK, int DVS, int C, int W>
struct LALayout {
    static constexpr int E = InTraits<TI>::E;
    static constexpr int KB = InTraits<TI>::KB;
    // dk is zero-padded to a whole contraction block (only bf16 with Dk = 16)
    static constexpr int DKP = DK < KB ? KB : DK;
    static constexpr int NT = C / 16;          // 16-row tiles per chunk
    static constexpr int NA = DKP / 16;        // 16-wide dk tiles
    static constexpr int NB = DVS / 16;        // 16-wide dv tiles in the slice
    static constexpr int NKD = DKP / KB;       // dk contraction blocks
    static constexpr int KP = DKP + 4;         // K tile row pitch (elements)
    static constexpr int VP = DVS + 4;         // V tile row pitch (elements)
    static constexpr int SP = DKP + 4;         // state slot pitch (floats), layout [dv][dk]
    static constexpr int KTILE_B = C * KP * (int)sizeof(TI);
    static constexpr int SSLOT_B = DVS * SP * 4;
    static constexpr int REGION_B = ((KTILE_B > SSLOT_B ? KTILE_B : SSLOT_B) + 15) / 16 * 16;
    static constexpr int VTILE_B = (C * VP * (int)sizeof(TI) + 15) / 16 * 16;
    // byte offsets
    static constexpr int OFF_REGION = 0;
    static constexpr int OFF_V = OFF_REGION + W * REGION_B;
    static constexpr int OFF_CARRY = OFF_V + W * VTILE_B;
    static constexpr int OFF_ZCARRY = OFF_CARRY + SSLOT_B;
    static constexpr int OFF_DZ = OFF_ZCARRY + DKP * 4;
    static constexpr int OFF_B2 = OFF_DZ + W * DKP * 4;
    static constexpr int OFF_DEN = OFF_B2 + W * C * 4;
    static constexpr int OFF_GAM = OFF_DEN + W * C * 4;
    static constexpr int TOTAL_B = OFF_GAM + ((W * 4 + 15) / 16) * 16;
    // V tile: 16-byte pieces per row and per lane
    static constexpr int VPIECES_ROW = DVS * (int)sizeof(TI) / 16;
    static constexpr int VPIECES = C * VPIECES_ROW;
    static constexpr int VPIECES_LANE = (VPIECES + 63) / 64;
    static_assert(C == 16 || C == 32 || C == 64, "chunk");
    static_assert(DKP % KB == 0 && DK % 16 == 0 && DVS % 16 == 0, "dims");
};

// ----------------------------------------------------------------------------
// MFMA wrappers
// ----------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mma_dk(const u16x8 &a, const u16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_dk(const f32x4 &a, const f32x4 &b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}

template <typename TI, int DK, int DVS, int C, int W>
__global__ __launch_bounds__(64 * W) void la_chunk_fwd(LAParams p) {
    typedef LALayout<TI, DK, DVS, C, W> L;
    typedef typename InTraits<TI>::Frag Frag;
    constexpr int NT = L::NT, NA = L::NA, NB = L::NB, E = L::E, KB = L::KB, NKD = L::NKD;
    constexpr int DKP = L::DKP;
    constexpr bool BF16 = sizeof(TI) == 2;

    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL_B];

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, c16 = lane & 15, g = lane >> 4;

    // ---- workgroup -> (b*h, slice); siblings of one (b,h) share an XCD ------
    int wg = blockIdx.x;
    const int nwg = gridDim.x;
    if ((p.B * p.H) % 8 == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
    const int bh = wg / p.nslice, slice = wg - bh * p.nslice;
    const int h = bh % p.H;
    const int dv0 = slice * DVS;
    const int T = p.T, Dv = p.Dv;

    const TI *__restrict__ qg = static_cast<const TI *>(p.q) + (size_t)bh * T * DK;
    const TI *__restrict__ kg = static_cast<const TI *>(p.k) + (size_t)bh * T * DK;
    const TI *__restrict__ vg = static_cast<const TI *>(p.v) + (size_t)bh * T * Dv + dv0;
    TI *__restrict__ yg = static_cast<TI *>(p.y) + (size_t)bh * T * Dv + dv0;

    char *region = smem + L::OFF_REGION + w * L::REGION_B;
    TI *ktile = reinterpret_cast<TI *>(region);
    float *myslot = reinterpret_cast<float *>(region);
    TI *vtile = reinterpret_cast<TI *>(smem + L::OFF_V + w * L::VTILE_B);
    float *carry = reinterpret_cast<float *>(smem + L::OFF_CARRY);
    float *zcarry = reinterpret_cast<float *>(smem + L::OFF_ZCARRY);
    float *dzs = reinterpret_cast<float *>(smem + L::OFF_DZ);
    float *b2tab = reinterpret_cast<float *>(smem + L::OFF_B2) + w * C;
    float *dentab = reinterpret_cast<float *>(smem + L::OFF_DEN) + w * C;
    float *gam = reinterpret_cast<float *>(smem + L::OFF_GAM);

    // ---- initial carry: state_in slice -> LDS [dv][dk]; key sum -> LDS -----
    for (int idx = tid; idx < DKP * DVS; idx += 64 * W) {
        const int dk = idx / DVS, dv = idx - dk * DVS;
        carry[dv * L::SP + dk] = (p.state_in && dk < DK)
                                     ? p.state_in[((size_t)bh * DK + dk) * Dv + dv0 + dv] : 0.f;
    }
    for (int idx = tid; idx < DKP; idx += 64 * W)
        zcarry[idx] = (p.normalize && p.cum_k_in && idx < DK) ? p.cum_k_in[(size_t)bh * DK + idx] : 0.f;

    // processing-order row -> memory row
    auto mem_row = [&](int r) { return p.reverse ? (T - 1 - r) : r; };

    // ---- prefetch registers for one chunk ---------------------------------
    Frag Qn[NT][NKD], Kn[NT][NKD];
    uint4 Vn[L::VPIECES_LANE];
    float lgn;

    auto load_chunk = [&](int ch) {
        const int base = ch * C;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            const int r = base + 16 * tt + c16;
            const bool ok = r < T;
            const size_t off = (size_t)(ok ? mem_row(r) : 0) * DK + E * g;
#pragma unroll
            for (int pb = 0; pb < NKD; ++pb) {
                Frag qf = {}, kf = {};
                if (ok && (DK >= KB || E * g < DK)) {
                    qf = *reinterpret_cast<const Frag *>(qg + off + KB * pb);
                    kf = *reinterpret_cast<const Frag *>(kg + off + KB * pb);
                }
                Qn[tt][pb] = qf;
                Kn[tt][pb] = kf;
            }
        }
#pragma unroll
        for (int i = 0; i < L::VPIECES_LANE; ++i) {
            const int piece = lane + 64 * i;
            const int row = piece / L::VPIECES_ROW, col = piece - row * L::VPIECES_ROW;
            const int r = base + row;
            uint4 val = {0u, 0u, 0u, 0u};
            if (piece < L::VPIECES && r < T)
                val = *reinterpret_cast<const uint4 *>(
                    reinterpret_cast<const char *>(vg + (size_t)mem_row(r) * Dv) + 16 * col);
            Vn[i] = val;
        }
        // per-step mode: this lane's row (padding rows decay by 1); head mode:
        // the head's factor on every lane (the prefix is formed by multiplication)
        float lg = 0.f;
        const int r = base + lane;
        if (p.mode == 2 && lane < C && r < T) lg = log2f(p.decay[(size_t)bh * T + mem_row(r)]);
        else if (p.mode == 1) lg = log2f(p.decay[h]);
        lgn = fmaxf(lg, -100.f);   // log2(0) = -inf: clamp (2^-100 acts as zero)
    };

    const int nchunks = p.nchunks;
    load_chunk(w);
    __syncthreads();

    for (int gi = 0; gi < p.ngroups; ++gi) {
        const int ch = gi * W + w;
        Frag Qf[NT][NKD], Kf[NT][NKD];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int pb = 0; pb < NKD; ++pb) { Qf[tt][pb] = Qn[tt][pb]; Kf[tt][pb] = Kn[tt][pb]; }
        uint4 Vc[L::VPIECES_LANE];
#pragma unroll
        for (int i = 0; i < L::VPIECES_LANE; ++i) Vc[i] = Vn[i];
        const float lg = lgn;
        if (gi + 1 < p.ngroups) load_chunk(ch + W);

        // ---- V tile and K tile into this wave's LDS region --------------------
#pragma unroll
        for (int i = 0; i < L::VPIECES_LANE; ++i) {
            const int piece = lane + 64 * i;
            if (piece >= L::VPIECES) break;
            const int row = piece / L::VPIECES_ROW, col = piece - row * L::VPIECES_ROW;
            uint2 *dst = reinterpret_cast<uint2 *>(
                reinterpret_cast<char *>(vtile + row * L::VP) + 16 * col);
            dst[0] = make_uint2(Vc[i].x, Vc[i].y);
            dst[1] = make_uint2(Vc[i].z, Vc[i].w);
        }
#pragma unroll
        for (int st = 0; st < NT; ++st)
#pragma unroll
            for (int pb = 0; pb < NKD; ++pb) {
                uint4 raw = __builtin_bit_cast(uint4, Kf[st][pb]);
                uint2 *dst = reinterpret_cast<uint2 *>(ktile + (16 * st + c16) * L::KP + KB * pb + E * g);
                dst[0] = make_uint2(raw.x, raw.y);
                dst[1] = make_uint2(raw.z, raw.w);
            }

        // ---- chunk-local cumulative log2 decay ---------------------------------
        {
            const int nvalid = min(C, T - ch * C);   // may be <= 0 for a padding chunk
            float b2;
            if (p.mode == 1) {
                b2 = nvalid > 0 ? (float)(min(lane, nvalid - 1) + 1) * lg : 0.f;
            } else {
                b2 = lg;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float o = __shfl_up(b2, off, 64);
                    if (lane >= off) b2 += o;
                }
            }
            if (lane < C) b2tab[lane] = b2;
        }
        wave_lds_sync();

        const float b2last = b2tab[C - 1];
        float b2t[NT];          // b at t = 16 tt + c16   (score-tile columns)
        f32x4 b2s[NT];          // b at 16 x + 4 g + r    (score-tile rows, output rows)
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            b2t[x] = b2tab[16 * x + c16];
            b2s[x] = *reinterpret_cast<const f32x4 *>(b2tab + 16 * x + 4 * g);
        }
        const bool decayed = p.mode != 0;

        // ---- scores A^T[s][t] = K Q^T, masked and decayed --------------------------
        f32x4 P[NT][NT];   // [st][tt], st <= tt used
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int st = 0; st <= tt; ++st) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int pb = 0; pb < NKD; ++pb) acc = mma_dk(Kf[st][pb], Qf[tt][pb], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float val = acc[r];
                    if (st == tt && 4 * g + r > c16) val = 0.f;
                    else if (decayed) val *= exp2_fast(b2t[tt] - b2s[st][r]);
                    acc[r] = val;
                }
                P[st][tt] = acc;
            }

        // ---- V fragments: V[s = 16 st + 4 g + r][16 b + c16] (B operand of P V, K^T V)
        // bf16: 8 values = s-tiles (2 ks, 2 ks + 1); fp32: 4 values = s-tile st.
        constexpr int NVF = BF16 ? (NT + 1) / 2 : NT;
        Frag Vf[NVF][NB];
#pragma unroll
        for (int x = 0; x < NVF; ++x)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int st = BF16 ? 2 * x + (e >> 2) : x;
                    Vf[x][b][e] = st < NT ? vtile[(16 * st + 4 * g + (e & 3)) * L::VP + 16 * b + c16] : TI(0);
                }

        // ---- intra-chunk output O = P V (+ row sums of P for the normaliser) ---------
        f32x4 O[NT][NB];
        float den_in[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
            for (int b = 0; b < NB; ++b) O[tt][b] = f32x4{0.f, 0.f, 0.f, 0.f};
            float rs = 0.f;
            if constexpr (BF16) {
#pragma unroll
                for (int ks = 0; ks < NVF; ++ks) {
                    if (2 * ks > tt) break;
                    u16x8 a;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int st = 2 * ks + (e >> 2);
                        const float val = (st <= tt) ? P[st][tt][e & 3] : 0.f;
                        a[e] = f32_to_bf16_bits(val);
                        rs += bf16_bits_to_f32(a[e]);
                    }
#pragma unroll
                    for (int b = 0; b < NB; ++b) O[tt][b] = mma_dk(a, Vf[ks][b], O[tt][b]);
                }
            } else {
#pragma unroll
                for (int st = 0; st <= tt; ++st) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) rs += P[st][tt][r];
#pragma unroll
                    for (int b = 0; b < NB; ++b) O[tt][b] = mma_dk(P[st][tt], Vf[st][b], O[tt][b]);
                }
            }
            den_in[tt] = rs;
        }

        // ---- chunk state dS = (K * 2^(blast - b_s))^T V and key sum dz ---------------
        f32x4 dS[NA][NB];
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b) dS[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        float dzp[NA];
        f32x4 dfac[NT];
#pragma unroll
        for (int x = 0; x < NT; ++x)
#pragma unroll
            for (int r = 0; r < 4; ++r) dfac[x][r] = decayed ? exp2_fast(b2last - b2s[x][r]) : 1.f;
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            float zs = 0.f;
            if constexpr (BF16) {
#pragma unroll
                for (int ks = 0; ks < NVF; ++ks) {
                    u16x8 hi, lo;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int st = 2 * ks + (e >> 2);
                        float kv = 0.f;
                        if (st < NT)
                            kv = in_to_f32(ktile[(16 * st + 4 * g + (e & 3)) * L::KP + 16 * a + c16]) *
                                 dfac[st][e & 3];
                        zs += kv;
                        hi[e] = f32_to_bf16_bits(kv);
                        lo[e] = f32_to_bf16_bits(kv - bf16_bits_to_f32(hi[e]));
                    }
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        dS[a][b] = mma_dk(hi, Vf[ks][b], dS[a][b]);
                        dS[a][b] = mma_dk(lo, Vf[ks][b], dS[a][b]);
                    }
                }
            } else {
#pragma unroll
                for (int st = 0; st < NT; ++st) {
                    f32x4 kv;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        kv[r] = in_to_f32(ktile[(16 * st + 4 * g + r) * L::KP + 16 * a + c16]) * dfac[st][r];
                        zs += kv[r];
                    }
#pragma unroll
                    for (int b = 0; b < NB; ++b) dS[a][b] = mma_dk(kv, Vf[st][b], dS[a][b]);
                }
            }
            dzp[a] = sum_over_lane_groups(zs);
        }

        // ---- publish dS, dz and the chunk decay to LDS -------------------------------
        wave_lds_sync();   // all K-tile reads of this wave are done before the slot is overwritten
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                *reinterpret_cast<f32x4 *>(myslot + (16 * b + c16) * L::SP + 16 * a + 4 * g) = dS[a][b];
        if (g == 0) {
#pragma unroll
            for (int a = 0; a < NA; ++a) dzs[w * DKP + 16 * a + c16] = dzp[a];
        }
        if (lane == 0) gam[w] = exp2_fast(b2last);
        __syncthreads();

        // ---- S_prev / z_prev of this chunk: carry folded with the earlier waves ----------
        // B-operand layout: dk = KB pb + E g + e, dv = 16 b + c16.
        float Sp[NKD][NB][E];
        float zp[NKD][E];
#pragma unroll
        for (int pb = 0; pb < NKD; ++pb) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int e4 = 0; e4 < E; e4 += 4) {
                    const f32x4 c = *reinterpret_cast<const f32x4 *>(carry + (16 * b + c16) * L::SP + KB * pb + E * g + e4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) Sp[pb][b][e4 + e] = c[e];
                }
#pragma unroll
            for (int e4 = 0; e4 < E; e4 += 4) {
                const f32x4 c = *reinterpret_cast<const f32x4 *>(zcarry + KB * pb + E * g + e4);
#pragma unroll
                for (int e = 0; e < 4; ++e) zp[pb][e4 + e] = c[e];
            }
        }
        for (int j = 0; j < w; ++j) {
            const float gj = gam[j];
            const float *slot = reinterpret_cast<const float *>(smem + L::OFF_REGION + j * L::REGION_B);
#pragma unroll
            for (int pb = 0; pb < NKD; ++pb) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int e4 = 0; e4 < E; e4 += 4) {
                        const f32x4 d = *reinterpret_cast<const f32x4 *>(slot + (16 * b + c16) * L::SP + KB * pb + E * g + e4);
#pragma unroll
                        for (int e = 0; e < 4; ++e) Sp[pb][b][e4 + e] = fmaf(gj, Sp[pb][b][e4 + e], d[e]);
                    }
#pragma unroll
                for (int e4 = 0; e4 < E; e4 += 4) {
                    const f32x4 d = *reinterpret_cast<const f32x4 *>(dzs + j * DKP + KB * pb + E * g + e4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) zp[pb][e4 + e] = fmaf(gj, zp[pb][e4 + e], d[e]);
                }
            }
        }

        // ---- inter-chunk read-out: O += diag(2^b_t) Q S_prev --------------------------
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            Frag shi[NKD], slo[NKD];
#pragma unroll
            for (int pb = 0; pb < NKD; ++pb) {
                if constexpr (BF16) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const uint16_t hb = f32_to_bf16_bits(Sp[pb][b][e]);
                        shi[pb][e] = hb;
                        slo[pb][e] = f32_to_bf16_bits(Sp[pb][b][e] - bf16_bits_to_f32(hb));
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) shi[pb][e] = Sp[pb][b][e];
                }
            }
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x4 ox = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int pb = 0; pb < NKD; ++pb) {
                    ox = mma_dk(Qf[tt][pb], shi[pb], ox);
                    if constexpr (BF16) ox = mma_dk(Qf[tt][pb], slo[pb], ox);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float et = decayed ? exp2_fast(b2s[tt][r]) : 1.f;
                    O[tt][b][r] = fmaf(et, ox[r], O[tt][b][r]);
                }
            }
        }

        // ---- normaliser: den_t = sum_s P[t,s] + 2^b_t q_t . z_prev ------------------------
        if (p.normalize) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                float dx = 0.f;
#pragma unroll
                for (int pb = 0; pb < NKD; ++pb)
#pragma unroll
                    for (int e = 0; e < E; ++e) dx = fmaf(in_to_f32(Qf[tt][pb][e]), zp[pb][e], dx);
                dx = sum_over_lane_groups(dx);
                const float di = sum_over_lane_groups(den_in[tt]);
                const float et = decayed ? exp2_fast(b2t[tt]) : 1.f;
                if (g == 0) dentab[16 * tt + c16] = fmaf(et, dx, di);
            }
            wave_lds_sync();
        }

        // ---- store y ---------------------------------------------------------------
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            f32x4 inv = {1.f, 1.f, 1.f, 1.f};
            if (p.normalize) {
                const f32x4 d = *reinterpret_cast<const f32x4 *>(dentab + 16 * tt + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) inv[r] = 1.f / d[r];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = ch * C + 16 * tt + 4 * g + r;
                if (row < T) {
                    TI *dst = yg + (size_t)mem_row(row) * Dv;
#pragma unroll
                    for (int b = 0; b < NB; ++b) store_out<TI>(dst + 16 * b + c16, O[tt][b][r] * inv[r]);
                }
            }
        }

        // ---- carry for the next group (last wave), after everyone has read it -------------
        __syncthreads();
        if (w == W - 1) {
            const float gw = gam[w];
#pragma unroll
            for (int pb = 0; pb < NKD; ++pb) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int e4 = 0; e4 < E; e4 += 4) {
                        const int o = (16 * b + c16) * L::SP + KB * pb + E * g + e4;
                        const f32x4 d = *reinterpret_cast<const f32x4 *>(myslot + o);
                        f32x4 n;
#pragma unroll
                        for (int e = 0; e < 4; ++e) n[e] = fmaf(gw, Sp[pb][b][e4 + e], d[e]);
                        *reinterpret_cast<f32x4 *>(carry + o) = n;
                    }
                if (c16 == 0) {
#pragma unroll
                    for (int e4 = 0; e4 < E; e4 += 4) {
                        const int o = KB * pb + E * g + e4;
                        const f32x4 d = *reinterpret_cast<const f32x4 *>(dzs + w * DKP + o);
                        f32x4 n;
#pragma unroll
                        for (int e = 0; e < 4; ++e) n[e] = fmaf(gw, zp[pb][e4 + e], d[e]);
                        *reinterpret_cast<f32x4 *>(zcarry + o) = n;
                    }
                }
            }
        }
        (void)nchunks;
    }

    // ---- final state ---------------------------------------------------------------
    __syncthreads();
    if (p.state_out) {
        for (int idx = tid; idx < DK * DVS; idx += 64 * W) {
            const int dk = idx / DVS, dv = idx - dk * DVS;
            p.state_out[((size_t)bh * DK + dk) * Dv + dv0 + dv] = carry[dv * L::SP + dk];
        }
    }
    if (p.normalize && p.cum_k_out && slice == 0) {
        for (int idx = tid; idx < DK; idx += 64 * W) p.cum_k_out[(size_t)bh * DK + idx] = zcarry[idx];
    }
}

}  // namespace drs
