// la_elem.hip -- chunked linear attention with one decay factor per key channel.
//
// RetNet issue #21: cumulative_ema takes factors of the values' own shape; here
// row i of the state (key channel i) decays by g_t[i] at step t,
//     S_t = diag(g_t) S_{t-1} + k_t v_t^T,   y_t = q_t^T S_t.
// Chunks of 16 rows.  With B_t[i] the chunk-local inclusive sum of log2 g[i],
//     y_t  = (q_t * 2^{B_t})^T S_in + sum_{s<=t} (sum_i q_t[i] k_s[i] 2^{B_t[i]-B_s[i]}) v_s
//     S_out = diag(2^{B_15}) S_in + sum_s (k_s * 2^{B_15 - B_s}) v_s^T.
// Every state-side exponent is <= 0.  The intra-chunk scores factor as
// (q_t 2^{B_t - B_r}) . (k_s 2^{B_r - B_s}) around a reference row r: r = the
// row before the chunk for t in the first eight rows, r = row 7 for the last
// eight.  Query exponents are <= 0; key exponents span at most eight steps, so
// with each step's log2 factor floored at -15 they stay below 2^120 (bf16 and
// fp32 both reach 2^127).  The floor makes a factor below 2^-15 act as 2^-15:
// the old state keeps that share instead of less (a relative error below 3e-5
// of the decayed term).  A zero factor therefore restarts the state up to 2^-15.
//
// Layout of the work (MFMA v_mfma_f32_16x16x16_bf16; a 16x16 accumulator tile
// holds rows 4(l/16)+r, column l%16 in lane l, which is also the A-operand
// layout of its transpose):
//   - a workgroup of Dv/16 waves owns one (b, h, time segment); wave w owns
//     value columns 16w..16w+15 and keeps its Dk x 16 slice of S in registers;
//   - per chunk the workgroup stages the factors (fp32) and, per channel, the
//     prefix B_t; then the scaled operands (bf16) for the scores, the read-out
//     and the state update, and V, all row-major in LDS (operands that are
//     needed across rows come through the gfx950 transpose read);
//   - every wave forms the 16x16 score tile transposed (keys as rows), so the
//     masked tile is directly the B operand of O^T = V^T P^T, adds
//     S^T (q 2^{B_t})^T with S as a hi+lo bf16 pair, stores 8 bytes of y per
//     lane, then updates S with the decayed keys (hi+lo) against V.  The
//     decayed queries of the read-out are a hi+lo pair as well: unlike a scalar
//     decay, a per-channel one cannot be applied after the product.
// Two passes over time segments: pass 1 runs each segment from a zero state and
// stores its summary (the state reached, and the segment's total log2 decay
// per channel); pass 2 folds the summaries of the earlier segments onto the
// initial state in order (deterministic) and produces the outputs.
#include "common.h"
#include "la_elem.h"

namespace drs {

namespace {

typedef short v4i16e __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4i16e, a), __builtin_bit_cast(v4i16e, b), c,
                                                     0, 0, 0);
}

__device__ __forceinline__ u32x2 pack4(float a, float b, float c, float d) {
    return u32x2{pack_bf16x2(a, b), pack_bf16x2(c, d)};
}

// Fragment of a row-major 16-row bf16 LDS tile read across rows: element r of
// lane l is tile[4 (l/16) + r][col0 + l%16].  ds_read_b64_tr_b16 works on
// 16-lane blocks; output lane 4j+e gathers element e of source lanes j, j+4,
// j+8, j+12, so source lane 4m+j addresses row 4 (l/16) + m, column col0 + 4j.
__device__ __forceinline__ u32x2 tr_frag4(const uint16_t *tile, int pitch, int col0, int lane) {
    const int src = lane & 15, g = lane >> 4;
    const uint16_t *pa = tile + (4 * g + (src >> 2)) * pitch + col0 + 4 * (src & 3);
    const v4i16e r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16e *)(pa));
    return __builtin_bit_cast(u32x2, r);
}

// At least 4 waves per SIMD (two workgroups of 8 waves per compute unit at
// Dv = 128, at most 128 VGPRs).  Asking for 6 made the compiler spill (slower).
template <int DK, int DV, bool OUT>
__global__ __launch_bounds__(4 * DV) __attribute__((amdgpu_waves_per_eu(4)))
void la_elem_kernel(LAElemParams p) {
    constexpr int C = kElemChunk;
    constexpr int NT = 4 * DV;            // DV/16 waves
    constexpr int NA = DK / 16;           // channel tiles of the state
    constexpr int PR = DK / 4;            // 4-element pieces per q/k/g row
    constexpr int NP = C * PR;            // pieces per chunk
    constexpr int QP = (NP + NT - 1) / NT;
    constexpr int VR = DV / 4;            // 4-element pieces per v row
    // LDS pitches (u16): a row of DK (DV) elements plus 16, so that the 16 rows a
    // fragment read touches start 8 banks apart (reads of 8 bytes per lane)
    constexpr int RP = DK + 16;
    constexpr int VP = DV + 16;
    static_assert(C * VR == NT, "one v piece per thread");

    __shared__ __align__(16) float sB[C][DK];            // factors, log2 prefix, then partial scores
    __shared__ __align__(16) uint16_t sQr[C][RP];        // q 2^{B_t}, hi       (read-out)
    __shared__ __align__(16) uint16_t sQl[C][RP];        // q 2^{B_t}, lo
    __shared__ __align__(16) uint16_t sQs[C][RP];        // q 2^{B_t - B_r}, hi (scores)
    __shared__ __align__(16) uint16_t sQt[C][RP];        // q 2^{B_t - B_r}, lo
    __shared__ __align__(16) uint16_t sK1[C][RP];        // k 2^{-B_s}, rows 0..7
    __shared__ __align__(16) uint16_t sK2[C][RP];        // k 2^{B_7 - B_s}
    __shared__ __align__(16) uint16_t sKh[C][RP], sKl[C][RP];     // k 2^{B_15-B_s}, hi and lo
    __shared__ __align__(16) uint16_t sV[C][VP];         // v
    __shared__ float sDend[DK];                          // 2^{B_15}

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c16 = lane & 15, g4 = lane >> 4;
    const int unit = blockIdx.x / p.nseg, seg = blockIdx.x - unit * p.nseg;
    const int T = p.T;
    const int ch0 = seg * p.L, ch1 = min(ch0 + p.L, p.nchunks);
    const int dv0 = 16 * w;

    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (size_t)unit * T * DK, T * DK * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (size_t)unit * T * DK, T * DK * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (size_t)unit * T * DV, T * DV * 2);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.decay + (size_t)unit * T * DK, T * DK * 4);
    auto mem_row = [&](int r) { return p.reverse ? T - 1 - r : r; };

    // ---- state: tile a, register r = S[16a + 4 g4 + r][dv0 + c16] ---------------
    f32x4 S[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) S[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    // workspace per unit: the initial state in lane order, then one summary per segment
    const size_t slot_f = (size_t)DK * DV + DK;
    float *init = p.ws + (size_t)unit * ((size_t)DK * DV + p.nseg * slot_f);
    float *slots = init + (size_t)DK * DV;
    auto lane_slot = [&](float *base, int a) { return base + ((size_t)(w * NA + a) * 64 + lane) * 4; };
    if constexpr (!OUT) {
        // Pass 1 copies the initial state for pass 2, so that pass 2 never reads
        // state_in and its last segment may overwrite it (state_out == state_in).
        if (seg == 0) {
#pragma unroll
            for (int a = 0; a < NA; ++a) {
                f32x4 x = {0.f, 0.f, 0.f, 0.f};
                if (p.state_in) {
                    const float *si = p.state_in + (size_t)unit * DK * DV;
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[r] = si[(16 * a + 4 * g4 + r) * DV + dv0 + c16];
                }
                *reinterpret_cast<f32x4 *>(lane_slot(init, a)) = x;
            }
        }
    } else {
        if (p.nseg > 1) {
#pragma unroll
            for (int a = 0; a < NA; ++a) S[a] = *reinterpret_cast<const f32x4 *>(lane_slot(init, a));
        } else if (p.state_in) {   // one segment: each lane reads the elements it writes last
            const float *si = p.state_in + (size_t)unit * DK * DV;
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[a][r] = si[(16 * a + 4 * g4 + r) * DV + dv0 + c16];
        }
        // fold the earlier segments' summaries in order
        for (int j = 0; j < seg; ++j) {
            const float *sl = slots + (size_t)j * slot_f;
#pragma unroll
            for (int a = 0; a < NA; ++a) {
                const f32x4 d = *reinterpret_cast<const f32x4 *>(lane_slot(const_cast<float *>(sl), a));
#pragma unroll
                for (int r = 0; r < 4; ++r) S[a][r] = fmaf(exp2_fast(sl[DK * DV + 16 * a + 4 * g4 + r]), S[a][r], d[r]);
            }
        }
    }
    // per-channel total log2 decay of the segment (pass 1), channels tid, tid + NT, ...
    // the prefix runs on four lanes per channel (rows 4q .. 4q+3 on lane q)
    constexpr int CPT = (4 * DK + NT - 1) / NT;
    float gsum[CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) gsum[c] = 0.f;

    // ---- chunk loads, one chunk ahead in registers --------------------------------
    struct Raw {
        u32x2 q[QP], k[QP], v;
        f32x4 g[QP];
    };
    auto load = [&](int ch, Raw &R) {
#pragma unroll
        for (int n = 0; n < QP; ++n) {
            const int e = tid + n * NT;
            const int t = e / PR, i0 = 4 * (e - (e / PR) * PR);
            const int row = ch * C + t;
            const bool ok = e < NP && row < T;
            const unsigned o2 = ok ? (unsigned)((mem_row(row) * DK + i0) * 2) : kOutOfRange;
            const unsigned o4 = ok ? (unsigned)((mem_row(row) * DK + i0) * 4) : kOutOfRange;
            R.q[n] = __builtin_amdgcn_raw_buffer_load_b64(rq, o2, 0, kNonTemporal);
            R.k[n] = __builtin_amdgcn_raw_buffer_load_b64(rk, o2, 0, kNonTemporal);
            R.g[n] = __builtin_bit_cast(f32x4, buffer_load16(rg, o4));
        }
        const int t = tid / VR, j0 = 4 * (tid - (tid / VR) * VR);
        const int row = ch * C + t;
        const unsigned ov = row < T ? (unsigned)((mem_row(row) * DV + j0) * 2) : kOutOfRange;
        R.v = __builtin_amdgcn_raw_buffer_load_b64(rv, ov, 0, kNonTemporal);
    };

    const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y + (size_t)unit * T * DV, T * DV * 2);
    Raw cur, nxt;
    if (ch0 < ch1) load(ch0, cur);
    for (int ch = ch0; ch < ch1; ++ch) {
        // stage the floored log2 factors (rows past T: factor 1) and v
#pragma unroll
        for (int n = 0; n < QP; ++n) {
            const int e = tid + n * NT;
            if (e < NP) {
                const int t = e / PR, i0 = 4 * (e - (e / PR) * PR);
                const bool live = ch * C + t < T;
                f32x4 lg;
#pragma unroll
                for (int r = 0; r < 4; ++r) lg[r] = live ? fmaxf(__log2f(cur.g[n][r]), kElemLog2Floor) : 0.f;
                *reinterpret_cast<f32x4 *>(&sB[t][i0]) = lg;
            }
        }
        {
            const int t = tid / VR, j0 = 4 * (tid - (tid / VR) * VR);
            *reinterpret_cast<u32x2 *>(&sV[t][j0]) = cur.v;
        }
        if (ch + 1 < ch1) load(ch + 1, nxt);
        __syncthreads();
        // per-channel inclusive prefix over the 16 rows: lane q of a group of four
        // sums rows 4q .. 4q+3, the group scans its four totals with lane exchanges
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int q = tid & 3, i = (tid >> 2) + c * (NT / 4);
            float x[4], run = 0.f;
            if (i < DK) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    run += sB[4 * q + j][i];
                    x[j] = run;
                }
            }
            float inc = run;                                   // inclusive scan of the totals
            const float u1 = __shfl_up(inc, 1, 4);
            if (q >= 1) inc += u1;
            const float u2 = __shfl_up(inc, 2, 4);
            if (q >= 2) inc += u2;
            const float base = inc - run;
            if (i < DK) {
#pragma unroll
                for (int j = 0; j < 4; ++j) sB[4 * q + j][i] = base + x[j];
                if (q == 3) {
                    sDend[i] = exp2_fast(inc);
                    gsum[c] += inc;
                }
            }
        }
        __syncthreads();
        // scaled operands
#pragma unroll
        for (int n = 0; n < QP; ++n) {
            const int e = tid + n * NT;
            if (e < NP) {
                const int t = e / PR, i0 = 4 * (e - (e / PR) * PR);
                float kd[4], qr[4], ql[4], qs[4], qt[4], k1[4], k2[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float b = sB[t][i0 + r], b7 = sB[7][i0 + r], b15 = sB[C - 1][i0 + r];
                    const float qv = (r & 1) ? bf16_hi(cur.q[n][r >> 1]) : bf16_lo(cur.q[n][r >> 1]);
                    const float kv = (r & 1) ? bf16_hi(cur.k[n][r >> 1]) : bf16_lo(cur.k[n][r >> 1]);
                    kd[r] = kv * exp2_fast(b15 - b);
                    if constexpr (OUT) {
                        const float qd = qv * exp2_fast(b);
                        qr[r] = bf16_bits_to_f32(f32_to_bf16_bits(qd));
                        ql[r] = qd - qr[r];
                        const float qe = t < 8 ? qd : qv * exp2_fast(b - b7);
                        qs[r] = bf16_bits_to_f32(f32_to_bf16_bits(qe));
                        qt[r] = qe - qs[r];
                        k1[r] = t < 8 ? kv * exp2_fast(-b) : 0.f;
                        k2[r] = kv * exp2_fast(b7 - b);
                    }
                }
                float kh[4], kl[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    kh[r] = bf16_bits_to_f32(f32_to_bf16_bits(kd[r]));
                    kl[r] = kd[r] - kh[r];
                }
                *reinterpret_cast<u32x2 *>(&sKh[t][i0]) = pack4(kh[0], kh[1], kh[2], kh[3]);
                *reinterpret_cast<u32x2 *>(&sKl[t][i0]) = pack4(kl[0], kl[1], kl[2], kl[3]);
                if constexpr (OUT) {
                    *reinterpret_cast<u32x2 *>(&sQr[t][i0]) = pack4(qr[0], qr[1], qr[2], qr[3]);
                    *reinterpret_cast<u32x2 *>(&sQl[t][i0]) = pack4(ql[0], ql[1], ql[2], ql[3]);
                    *reinterpret_cast<u32x2 *>(&sQs[t][i0]) = pack4(qs[0], qs[1], qs[2], qs[3]);
                    *reinterpret_cast<u32x2 *>(&sQt[t][i0]) = pack4(qt[0], qt[1], qt[2], qt[3]);
                    *reinterpret_cast<u32x2 *>(&sK1[t][i0]) = pack4(k1[0], k1[1], k1[2], k1[3]);
                    *reinterpret_cast<u32x2 *>(&sK2[t][i0]) = pack4(k2[0], k2[1], k2[2], k2[3]);
                }
            }
        }
        __syncthreads();

        // V^T fragment of this wave: value column dv0 + c16, tokens 4 g4 .. 4 g4 + 3
        // (the gfx950 transpose read of the row-major tile)
        const u32x2 vt = tr_frag4(&sV[0][0], VP, dv0, lane);
        if constexpr (OUT) {
            // transposed scores: rows s = 4 g4 + r, column t = c16; the channel tiles
            // are dealt over the waves and the partial tiles summed through LDS
            // (in the prefix array, free once the operands are formed)
            constexpr int NW = DV / 16, NSW = NA < NW ? NA : NW;
            float *part = &sB[0][0];
            const bool lo_half = c16 < 8;
            if (w < NSW) {
                f32x4 sp = {0.f, 0.f, 0.f, 0.f};
                for (int a = w; a < NA; a += NSW) {
                    const int kk = 16 * a + 4 * g4;
                    const u32x2 a1 = *reinterpret_cast<const u32x2 *>(&sK1[c16][kk]);
                    const u32x2 a2 = *reinterpret_cast<const u32x2 *>(&sK2[c16][kk]);
                    const u32x2 bq = *reinterpret_cast<const u32x2 *>(&sQs[c16][kk]);
                    const u32x2 bt = *reinterpret_cast<const u32x2 *>(&sQt[c16][kk]);
                    const u32x2 z = {0u, 0u};
                    // the query side as hi + lo: the key side's rounding is then the only one
                    sp = mma16(a1, lo_half ? bq : z, sp);
                    sp = mma16(a1, lo_half ? bt : z, sp);
                    sp = mma16(a2, lo_half ? z : bq, sp);
                    sp = mma16(a2, lo_half ? z : bt, sp);
                }
                *reinterpret_cast<f32x4 *>(part + (w * 64 + lane) * 4) = sp;
            }
            __syncthreads();
            f32x4 sc = *reinterpret_cast<const f32x4 *>(part + lane * 4);
#pragma unroll
            for (int j = 1; j < NSW; ++j) sc += *reinterpret_cast<const f32x4 *>(part + (j * 64 + lane) * 4);
            float pm[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pm[r] = (4 * g4 + r <= c16) ? sc[r] : 0.f;
            const u32x2 pt = pack4(pm[0], pm[1], pm[2], pm[3]);
            // O^T = V^T P^T + S^T (q 2^B)^T, in three independent accumulation chains
            f32x4 o = mma16(vt, pt, f32x4{0.f, 0.f, 0.f, 0.f});
            f32x4 o2 = {0.f, 0.f, 0.f, 0.f}, o3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int a = 0; a < NA; ++a) {
                u32x2 shi, slo;
                float hi[4], lo[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    hi[r] = bf16_bits_to_f32(f32_to_bf16_bits(S[a][r]));
                    lo[r] = S[a][r] - hi[r];
                }
                shi = pack4(hi[0], hi[1], hi[2], hi[3]);
                slo = pack4(lo[0], lo[1], lo[2], lo[3]);
                // S q as hi*hi + lo*hi + hi*lo: both operands carry ~16 bits
                const u32x2 bq = *reinterpret_cast<const u32x2 *>(&sQr[c16][16 * a + 4 * g4]);
                const u32x2 bl = *reinterpret_cast<const u32x2 *>(&sQl[c16][16 * a + 4 * g4]);
                o = mma16(shi, bq, o);
                o2 = mma16(slo, bq, o2);
                o3 = mma16(shi, bl, o3);
            }
            o += o2 + o3;
            // lane holds y[t = c16][dv0 + 4 g4 .. + 3]
            const int row = ch * C + c16;
            const unsigned off = row < T ? (unsigned)((mem_row(row) * DV + dv0 + 4 * g4) * 2) : kOutOfRange;
            buffer_store8(ry, off, pack4(o[0], o[1], o[2], o[3]));
        }
        // S = diag(2^{B_15}) S + (k 2^{B_15 - B_s})^T v
        const u32x2 vb = vt;   // B operand: column dv0 + c16, tokens 4 g4 .. (the same fragment)
#pragma unroll
        for (int a = 0; a < NA; ++a) {
#pragma unroll
            for (int r = 0; r < 4; ++r) S[a][r] *= sDend[16 * a + 4 * g4 + r];
            const u32x2 ah = tr_frag4(&sKh[0][0], RP, 16 * a, lane);
            const u32x2 al = tr_frag4(&sKl[0][0], RP, 16 * a, lane);
            S[a] = mma16(ah, vb, S[a]);
            S[a] = mma16(al, vb, S[a]);
        }
        __syncthreads();   // LDS of this chunk is read by every wave before the next is staged
        if (ch + 1 < ch1) cur = nxt;
    }

    if constexpr (!OUT) {
        float *sl = slots + (size_t)seg * slot_f;
#pragma unroll
        for (int a = 0; a < NA; ++a)
            *reinterpret_cast<f32x4 *>(lane_slot(sl, a)) = S[a];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int i = (tid >> 2) + c * (NT / 4);
            if ((tid & 3) == 3 && i < DK) sl[DK * DV + i] = gsum[c];
        }
    } else {
        if (seg == p.nseg - 1 && p.state_out) {
            float *so = p.state_out + (size_t)unit * DK * DV;
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int r = 0; r < 4; ++r) so[(16 * a + 4 * g4 + r) * DV + dv0 + c16] = S[a][r];
        }
    }
}

template <int DK, int DV>
hipError_t launch_dims(const LAElemParams &p, hipStream_t s) {
    const dim3 grid((unsigned)(p.B * p.H * p.nseg)), block(4 * DV);
    if (p.nseg > 1) {
        hipLaunchKernelGGL((la_elem_kernel<DK, DV, false>), grid, block, 0, s, p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((la_elem_kernel<DK, DV, true>), grid, block, 0, s, p);
    return hipGetLastError();
}

template <int DK>
hipError_t launch_dv(const LAElemParams &p, int Dv, hipStream_t s) {
    switch (Dv) {
        case 16: return launch_dims<DK, 16>(p, s);
        case 32: return launch_dims<DK, 32>(p, s);
        case 64: return launch_dims<DK, 64>(p, s);
        case 128: return launch_dims<DK, 128>(p, s);
        default: return hipErrorNotSupported;
    }
}

}  // namespace

bool la_elem_plan(int B, int H, int T, int Dk, int Dv, int *nseg, int *L) {
    auto dim_ok = [](int d) { return d == 16 || d == 32 || d == 64 || d == 128; };
    if (!dim_ok(Dk) || !dim_ok(Dv) || B < 1 || H < 1 || T < 1) return false;
    const long units = (long)B * H;
    const long nchunks = (T + (long)kElemChunk - 1) / kElemChunk;
    long ns = (kElemTargetGroups + units - 1) / units;
    if (ns > nchunks) ns = nchunks;
    if (ns < 1) ns = 1;
    const long l = (nchunks + ns - 1) / ns;
    ns = (nchunks + l - 1) / l;
    if (units * ns > 0x7fffffffL) return false;
    *nseg = (int)ns;
    *L = (int)l;
    return true;
}

size_t la_elem_ws_bytes(int B, int H, int T, int Dk, int Dv) {
    int ns, l;
    if (!la_elem_plan(B, H, T, Dk, Dv, &ns, &l)) return 0;
    return 256 + (size_t)B * H * ((size_t)Dk * Dv + (size_t)ns * ((size_t)Dk * Dv + Dk)) * 4;
}

hipError_t la_elem_launch(const LAElemParams &p, int Dk, int Dv, hipStream_t s) {
    switch (Dk) {
        case 16: return launch_dv<16>(p, Dv, s);
        case 32: return launch_dv<32>(p, Dv, s);
        case 64: return launch_dv<64>(p, Dv, s);
        case 128: return launch_dv<128>(p, Dv, s);
        default: return hipErrorNotSupported;
    }
}

}  // namespace drs
