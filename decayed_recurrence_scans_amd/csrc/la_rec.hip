// la_rec.hip -- linear attention one step at a time, the state held in registers.
//
// The recurrence of the tensortonic "cs336 linear attention duality" exercise
// (problem statement), S_t = g_t S_{t-1} + k_t v_t^T, y_t = q_t^T S_t, with the
// decay of RetNet issue #21 (cumulative_ema: the factor of step t multiplies the
// state carried in; factors may have the values' own shape, here one per key
// channel) and the normaliser with a cached key sum of flash-linear-attention
// issue #268 (y_t = q_t^T S_t / q_t^T z_t, z_t = g_t z_{t-1} + k_t).  That issue
// names the case this kernel is for: generation feeds one new token at a time
// together with the carried state and key sum.
//
// One workgroup owns one (b, h) pair.  Its threads tile the fp32 state [Dk, Dv]:
// thread (rg, quad) holds columns 4 quad .. 4 quad + 3 of rows rg + RG i,
// i < RPT, so each wave reads and writes whole contiguous rows.  The state is read
// once, stepped through every token in registers and written once; for a decode
// step the kernel is bound by that state traffic.  Per step, each thread updates
// its rows and forms its share of q_t^T S_t; the shares are summed over the row
// groups with lane exchanges inside a wave and through LDS across waves.  Inputs
// of up to `tb` steps are staged in LDS as fp32 at a time.
#include "common.h"
#include "la_rec.h"

namespace drs {

namespace {

template <typename TI> __device__ __forceinline__ float load_in(const TI *p, size_t i);
template <> __device__ __forceinline__ float load_in<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_in<uint16_t>(const uint16_t *p, size_t i) {
    return bf16_bits_to_f32(p[i]);
}

constexpr int kRecThreads = 256;

template <typename TI, int RPT, int MODE>
__global__ __launch_bounds__(kRecThreads) void la_rec_kernel(LARecParams p) {
    extern __shared__ f32x4 smem4[];
    const int Dk = p.Dk, Dv = p.Dv, T = p.T, TB = p.tb;
    const int NT = blockDim.x;
    const int QPR = Dv >> 2;             // column quads per state row
    const int RG = NT / QPR;             // row groups (RG * RPT == Dk)
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = NT >> 6;
    const int quad = tid % QPR, rg = tid / QPR;
    const int bh = blockIdx.x;
    const bool norm = p.normalize != 0;

    // LDS: partial outputs [2][nw][QPR] (two step parities), partial denominators
    // [2][4], then the staged inputs q, k [TB][Dk], v [TB][Dv], factors.
    f32x4 *red = smem4;
    float *rden = reinterpret_cast<float *>(red + 2 * nw * QPR);
    float *sq = rden + 8;
    float *sk = sq + TB * Dk;
    float *sv = sk + TB * Dk;
    float *sg = sv + TB * Dv;

    // ---- the carried state, through the buffer range check ------------------------
    const size_t st_base = (size_t)bh * Dk * Dv;
    f32x4 S[RPT];
    float z[RPT];
    {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.state_in ? p.state_in + st_base : nullptr,
                                                    p.state_in ? Dk * Dv * 4 : 0);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int d = rg + RG * i;
            const unsigned off = (unsigned)((d * Dv + 4 * quad) * 4);
            if (p.vec_state) {
                S[i] = __builtin_bit_cast(f32x4, buffer_load16(rs, off));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) S[i][r] = buffer_load4(rs, off + 4 * r);
            }
            z[i] = (norm && p.cum_k_in) ? p.cum_k_in[(size_t)bh * Dk + d] : 0.f;
        }
    }
    const float gh = MODE == 1 ? p.decay[bh % p.H] : 1.f;

    const TI *qg = static_cast<const TI *>(p.q) + (size_t)bh * T * Dk;
    const TI *kg = static_cast<const TI *>(p.k) + (size_t)bh * T * Dk;
    const TI *vg = static_cast<const TI *>(p.v) + (size_t)bh * T * Dv;
    const int ysz = (sizeof(TI) == 2 && p.y_f32) ? 4 : (int)sizeof(TI);   // bytes per stored output
    char *yg = static_cast<char *>(p.y) + (size_t)bh * T * Dv * ysz;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(yg, T * Dv * ysz);
    const int dk_shift = __builtin_ctz(Dk), dv_shift = __builtin_ctz(Dv);

    int par = 0;
    for (int n0 = 0; n0 < T; n0 += TB) {
        const int nb = T - n0 < TB ? T - n0 : TB;
        // ---- stage this block of steps (time index of step n: reversed or not) ----
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
        }
        if constexpr (MODE == 2) {
            for (int n = tid; n < nb; n += NT) {
                const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
                sg[n] = p.decay[(size_t)bh * T + t];
            }
        }
        __syncthreads();

        for (int n = 0; n < nb; ++n) {
            const float *qn = sq + n * Dk, *kn = sk + n * Dk;
            const f32x4 vq = *reinterpret_cast<const f32x4 *>(sv + n * Dv + 4 * quad);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            float dacc = 0.f;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int d = rg + RG * i;
                float g;
                if constexpr (MODE == 0) g = 1.f;
                else if constexpr (MODE == 1) g = gh;
                else if constexpr (MODE == 2) g = sg[n];
                else g = sg[n * Dk + d];
                const float kd = kn[d], qd = qn[d];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    S[i][r] = fmaf(kd, vq[r], g * S[i][r]);
                    acc[r] = fmaf(qd, S[i][r], acc[r]);
                }
                z[i] = fmaf(g, z[i], kd);
                dacc = fmaf(qd, z[i], dacc);
            }
            // sum over the row groups of this wave (lanes that share `quad`)
            for (int m = QPR; m < 64; m <<= 1) {
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] += __shfl_xor(acc[r], m, 64);
            }
            if (norm) {
                for (int m = QPR; m < 64; m <<= 1) dacc += __shfl_xor(dacc, m, 64);
            }
            // ... and over the waves; LDS of the two step parities alternates, so one
            // barrier per step orders the writes of step n+2 after the reads of step n
            if (lane < QPR) red[(par * nw + wv) * QPR + quad] = acc;
            if (lane == 0) rden[par * 4 + wv] = dacc;   // quad 0 of this wave's row groups
            __syncthreads();
            if (wv == 0 && lane < QPR) {
                f32x4 o = red[(par * nw) * QPR + quad];
                float den = rden[par * 4];
                for (int w2 = 1; w2 < nw; ++w2) {
                    const f32x4 x = red[(par * nw + w2) * QPR + quad];
                    o += x;
                    den += rden[par * 4 + w2];
                }
                if (norm) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = o[r] / den;
                }
                const int t = p.reverse ? T - 1 - (n0 + n) : n0 + n;
                const unsigned off = (unsigned)(((size_t)t * Dv + 4 * quad) * ysz);
                if constexpr (sizeof(TI) == 2) {
                    if (p.y_f32) buffer_store16(ry, off, __builtin_bit_cast(u32x4, o));
                    else buffer_store8(ry, off, u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])});
                } else {
                    buffer_store16(ry, off, __builtin_bit_cast(u32x4, o));
                }
            }
            par ^= 1;
        }
        __syncthreads();   // the staged block is read by every wave before it is replaced
    }

    // ---- write the state back (in place is fine: every element is read above by
    // the thread that writes it) -------------------------------------------------------
    if (p.state_out) {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.state_out + st_base, Dk * Dv * 4);
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int d = rg + RG * i;
            const unsigned off = (unsigned)((d * Dv + 4 * quad) * 4);
            if (p.vec_state) {
                buffer_store16(rs, off, __builtin_bit_cast(u32x4, S[i]));
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) buffer_store4(rs, off + 4 * r, S[i][r]);
            }
        }
    }
    if (norm && p.cum_k_out && quad == 0) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) p.cum_k_out[(size_t)bh * Dk + rg + RG * i] = z[i];
    }
}

template <typename TI, int MODE>
hipError_t launch_rpt(const LARecParams &p, int rpt, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
    switch (rpt) {
#define DRS_REC_CASE(R) \
        case R: hipLaunchKernelGGL((la_rec_kernel<TI, R, MODE>), grid, block, lds, s, p); break;
        DRS_REC_CASE(1)
        DRS_REC_CASE(2)
        DRS_REC_CASE(4)
        DRS_REC_CASE(8)
        DRS_REC_CASE(16)
#undef DRS_REC_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename TI>
hipError_t launch_mode(const LARecParams &p, int rpt, dim3 grid, dim3 block, size_t lds, hipStream_t s) {
    switch (p.mode) {
        case 0: return launch_rpt<TI, 0>(p, rpt, grid, block, lds, s);
        case 1: return launch_rpt<TI, 1>(p, rpt, grid, block, lds, s);
        case 2: return launch_rpt<TI, 2>(p, rpt, grid, block, lds, s);
        case 3: return launch_rpt<TI, 3>(p, rpt, grid, block, lds, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int la_rec_threads(int Dk, int Dv) {
    const int quads = Dk * Dv / 4;
    return quads < kRecThreads ? quads : kRecThreads;
}

size_t la_rec_lds_bytes(const LARecParams &p) {
    const int nt = la_rec_threads(p.Dk, p.Dv);
    const int nw = nt / 64, qpr = p.Dv / 4;
    const int gcols = p.mode == 3 ? p.Dk : (p.mode == 2 ? 1 : 0);
    return (size_t)2 * nw * qpr * 16 + 8 * 4 + (size_t)p.tb * (2 * p.Dk + p.Dv + gcols) * 4;
}

hipError_t la_rec_launch(const LARecParams &p, bool bf16, hipStream_t stream) {
    const int nt = la_rec_threads(p.Dk, p.Dv);
    const int rpt = p.Dk * p.Dv / 4 / nt;
    const dim3 grid((unsigned)(p.B * p.H)), block((unsigned)nt);
    const size_t lds = la_rec_lds_bytes(p);
    return bf16 ? launch_mode<uint16_t>(p, rpt, grid, block, lds, stream)
                : launch_mode<float>(p, rpt, grid, block, lds, stream);
}

}  // namespace drs
