// wkv.hip -- RWKV-4 WKV forward on gfx950: sequential and time-parallel paths.
//
// Definition (RWKV-LM issue #167, the att_seq recurrence; RWKV-LM discussion
// #189, the exponentially weighted (value, log-scale) pairs): per channel the
// state (aa, bb, pp) stands for the sums aa e^pp (values) and bb e^pp
// (weights).  Token t with key k and value v is read out against the state
// with the bonus u, then absorbed after one step of decay w:
//     m = max(pp, u + k):   y = (aa e^{pp-m} + v e^{u+k-m}) / (bb e^{pp-m} + e^{u+k-m})
//     m'= max(pp + w, k):   aa <- aa e^{pp+w-m'} + v e^{k-m'},  bb likewise,  pp <- m'
// In each max one of the two exponentials is e^0 = 1; the read-out is taken in
// a select-free form (below), so a step costs two exp2 and one reciprocal.
//
// Log-scales are kept in log2 units, and pp is held as an anchor plus a step
// count: pp = anchor + n w with one rounding (fma) instead of one rounding
// per step, so a large key that stays the running maximum for many steps
// does not drift.  The value is the same in exact arithmetic.
//
// Sequential path: one lane per (b, c), coalesced [T, C] streaming, the next
// block of PF steps of k and v loaded while the current block is computed.
// Time-parallel paths use the segment combine of two consecutive spans
//     (aa1,bb1,pp1) then (aa2,bb2,pp2) over n2 steps:
//     q = pp1 + n2 w, m = max(q, pp2), aa = aa1 2^{q-m} + aa2 2^{pp2-m}, ...
// (an associative operator, the scan form of RWKV-LM discussion #189).
// Walk mode (at least 512 groups of 64 channels, the WKV workload): one
// workgroup walks all time blocks of its 64 channels, its waves splitting each
// block and exchanging span summaries through LDS.  Chained single pass (fewer
// groups, while one resident round holds every (group, block)): each wave keeps
// 64 steps of k and v of 64 channels in registers, summarises them from the empty
// state, combines the summaries of its workgroup through LDS, gets the state
// entering its workgroup's time block by folding the published aggregates of the
// earlier blocks (look-back), and runs its outputs from the registers -- k and v
// are read once.  Two-pass scan (otherwise): pass 1 summarises every segment,
// pass 2 folds the summaries of the earlier segments and re-runs its segment,
// writing y.
#include "common.h"
#include "lookback.h"
#include "wkv.h"

namespace drs {

struct WKVState {
    float aa, bb, anc, n;   // pp (log2 units) = anc + n * w2
};

__device__ __forceinline__ WKVState wkv_empty() { return WKVState{0.f, 0.f, -1e38f * kLog2e, 0.f}; }

// The step.  The read-out weighs the current token against the absorbed sums by
// F = 2^(u + k - pp): y = (aa + F v) / (bb + F), with F clamped at 2^64.  The
// clamp only binds when the token outweighs the sums by more than 2^64, where y is
// v to within 2^-64 (times bb and |aa / v|); for the empty state F = 2^64 exactly
// and y = v exactly.  This form needs no selects.
__device__ __forceinline__ float wkv_out_step(WKVState &s, float w2, float wu2, float k, float v) {
    const float cand = fmaf(s.n + 1.f, w2, s.anc);   // pp + w, one rounding
    const float x = fmaf(k, -kLog2e, cand);           // pp + w - k (log2 units)
    const float f = exp2_fast(fminf(wu2 - x, 64.f));
    const float y = fmaf(f, v, s.aa) * rcp_fast(s.bb + f);
    const float ex = exp2_fast(-fabsf(x));
    const bool keep = x >= 0.f;                       // the decayed past stays the scale
    const float e1 = keep ? 1.f : ex, e2 = keep ? ex : 1.f;
    s.aa = fmaf(s.aa, e1, v * e2);
    s.bb = fmaf(s.bb, e1, e2);
    s.anc = keep ? s.anc : k * kLog2e;
    s.n = keep ? s.n + 1.f : 0.f;
    return y;
}

// Absorb only (summaries).
__device__ __forceinline__ void wkv_absorb_step(WKVState &s, float w2, float k, float v) {
    const float x = fmaf(k, -kLog2e, fmaf(s.n + 1.f, w2, s.anc));
    const float ex = exp2_fast(-fabsf(x));
    const bool keep = x >= 0.f;
    const float e1 = keep ? 1.f : ex, e2 = keep ? ex : 1.f;
    s.aa = fmaf(s.aa, e1, v * e2);
    s.bb = fmaf(s.bb, e1, e2);
    s.anc = keep ? s.anc : k * kLog2e;
    s.n = keep ? s.n + 1.f : 0.f;
}

// One token: the read-out (when OUT), then the absorb.  wu2 = w2 + u2.
template <bool OUT>
__device__ __forceinline__ float wkv_step(WKVState &s, float w2, float wu2, float k, float v) {
    if (OUT) return wkv_out_step(s, w2, wu2, k, v);
    wkv_absorb_step(s, w2, k, v);
    return 0.f;
}

// Run steps [t0, t1) of one channel; k, v, y point at element (b, 0, c), stride C.
// Whole blocks of PF steps stream without predicates, the next block's loads
// in flight while the current block is computed; the tail runs step by step.
template <bool OUT, int PF>
__device__ __forceinline__ void wkv_run(WKVState &s, float w2, float wu2, const float *__restrict__ k,
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
            const float yy = wkv_step<OUT>(s, w2, wu2, kc[i], vc[i]);
            if (OUT) y[(size_t)(tb + i) * C] = yy;
        }
#pragma unroll
        for (int i = 0; i < PF; ++i) { kc[i] = kn[i]; vc[i] = vn[i]; }
    }
    for (int t = t0 + nfull * PF; t < t1; ++t) {
        const float yy = wkv_step<OUT>(s, w2, wu2, k[(size_t)t * C], v[(size_t)t * C]);
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
    wkv_run<true, kWkvPF>(s, w2, w2 + u2, p.k + base, p.v + base, p.y + base, 0, p.T, p.C);
    if (p.state_out) wkv_store_state(p.state_out, s, w2, p.B, p.C, b, c);
}

// Combine of two consecutive spans, x then y (y spanning n2 steps), on states whose
// log-scale is kept as anchor + n w (in log2 units).  The larger of the two
// decayed scales keeps its anchor and step count exactly (x's count grows by
// n2), so a span boundary adds no rounding to the log-scale; only their
// difference, which weights the smaller side, is rounded (once).  Log-scales
// reach ~90 with keys of +-60, where rounding them to one fp32 value at every
// boundary costs ~1e-5 relative.
__device__ __forceinline__ WKVState wkv_combine(const WKVState &x, const WKVState &y, float n2, float w2) {
    const float xn = x.n + n2;
    const float d = fmaf(xn - y.n, w2, x.anc - y.anc);   // log2 of x's scale over y's
    const bool xbig = d >= 0.f;
    const float ex = exp2_fast(-fabsf(d));
    const float e1 = xbig ? 1.f : ex, e2 = xbig ? ex : 1.f;
    return WKVState{fmaf(x.aa, e1, y.aa * e2), fmaf(x.bb, e1, y.bb * e2), xbig ? x.anc : y.anc, xbig ? xn : y.n};
}

// Look-back mode: one workgroup of kWkvChainWaves waves per (64 channels of one batch
// row, time block); the state entering its block comes from the aggregates that the
// workgroups of the earlier blocks publish.
__global__ __launch_bounds__(64 * kWkvChainWaves, 2) void wkv_chain_fwd(WKVParams p) {
    __shared__ WKVState sums[kWkvChainWaves][64];
    __shared__ unsigned info[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar branches below
    const unsigned units = (unsigned)p.B * (unsigned)p.ncblk, total = units * (unsigned)p.nblk;
    // virtual ids, earlier blocks first: the workgroup id (the hardware starts lower ids
    // first, and a wave computes an aggregate that has not appeared in time itself), or
    // the start order from the ticket where the final state overwrites the initial one:
    // there every earlier block must have read it before the last block writes
    if (tid == 0) {
        info[0] = p.ticket ? atomicAdd(p.ws_ctr + 0, 1u) : blockIdx.x;
        info[1] = __hip_atomic_load(p.ws_ctr + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const unsigned vid = info[0], epoch = info[1];
    auto finish = [&]() {   // the last workgroup to finish re-arms the counters
        __syncthreads();
        if (tid == 0) {
            const unsigned done = atomicAdd(p.ws_ctr + 1, 1u);
            if (done == total - 1) {
                __hip_atomic_store(p.ws_ctr + 0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(p.ws_ctr + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(p.ws_ctr + 2, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    };
    if (vid >= total) {   // only with counters that were not zero before the first use
        if (tid == 0) atomicAdd(p.ws_ctr + 3, 1u);
        finish();
        return;
    }
    const int blk0 = (int)(vid / units), blk1 = blk0 + 1;
    const int unit = (int)(vid - (unsigned)blk0 * units);
    const int b = unit / p.ncblk, c = (unit - b * p.ncblk) * 64 + lane;
    const int T = p.T, C = p.C;
    const int cc = min(c, C - 1);
    const float w2 = p.w[cc] * kLog2e, wu2 = w2 + p.u[cc] * kLog2e;

    // the initial state, read before anything is published (state_out may alias it)
    WKVState cin = wkv_load_state(p.state_in, p.B, C, b, cc);

    const size_t row0 = (size_t)b * T * C;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y + row0, T * C * 4);

    for (int blk = blk0; blk < blk1; ++blk) {
        auto span = [&](int j) { return min(max(T - (blk * kWkvChainBlock + j * kWkvChainSub), 0), kWkvChainSub); };
        const int t0 = blk * kWkvChainBlock + wv * kWkvChainSub, n = span(wv);

        // this wave's steps, out of range (zeros) past the end or past the last channel
        float kc[kWkvChainSub], vc[kWkvChainSub];
#pragma unroll
        for (int i = 0; i < kWkvChainSub; ++i) {
            const unsigned off = (i < n && c < C) ? (unsigned)(((t0 + i) * C + c) * 4) : kOutOfRange;
            kc[i] = buffer_load4<kNonTemporal>(rk, off);
            vc[i] = buffer_load4<kNonTemporal>(rv, off);
        }

        // summary of this wave's steps from the empty state (full spans, the common
        // case, without per-step guards)
        WKVState s = wkv_empty();
        if (n == kWkvChainSub) {
#pragma unroll
            for (int i = 0; i < kWkvChainSub; ++i) wkv_step<false>(s, w2, wu2, kc[i], vc[i]);
        } else {
#pragma unroll
            for (int i = 0; i < kWkvChainSub; ++i)
                if (i < n) wkv_step<false>(s, w2, wu2, kc[i], vc[i]);
        }
        wait_stores_complete();   // every load of this wave has completed (initial state included)
        __syncthreads();          // the previous block's summaries are no longer read
        sums[wv][lane] = s;
        __syncthreads();

        // the block's aggregate: the waves' summaries combined in order
        WKVState agg = sums[0][lane];
#pragma unroll
        for (int j = 1; j < kWkvChainWaves; ++j) agg = wkv_combine(agg, sums[j][lane], (float)span(j), w2);

        {
            // publish the aggregate, then fold the earlier blocks' aggregates into the
            // initial state in order (fixed order: bitwise reproducible)
            const size_t slot = (size_t)unit * p.nblk + blk;
            if (blk < p.nblk - 1 && wv == 0) {
                float *d = p.ws_agg + (slot * 64 + lane) * 4;
                coherent_store2(d, agg.aa, agg.bb);
                coherent_store2(d + 2, agg.anc, agg.n);
                wait_stores_complete();
                if (lane == 0)
                    __hip_atomic_store(p.ws_flags + slot, flag_word(epoch, kAgg), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            bool all_ok = !p.own_aggs;
            for (int j0 = 0; j0 < blk && all_ok; j0 += 64) {
                const int j = j0 + lane;
                bool ok = j >= blk;
                for (unsigned it = 0; it < p.spin_limit; ++it) {
                    if (!ok)
                        ok = flag_state(__hip_atomic_load(p.ws_flags + (size_t)unit * p.nblk + j, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT),
                                        epoch) == kAgg;
                    if (__all(ok)) break;
                    __builtin_amdgcn_s_sleep(2);
                }
                all_ok = __all(ok);
            }
            if (!all_ok && p.ticket && lane == 0) atomicAdd(p.ws_ctr + 3, 1u);   // gave up (never expected)
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            constexpr int kBlkLoads = 8;
            if (!all_ok && !p.ticket) {
                // block by block; an aggregate still missing is computed here from the
                // block's k and v (every earlier block is a full one) and counted
                for (int j = 0; j < blk; ++j) {
                    const bool have = !p.own_aggs &&
                                      flag_state(__hip_atomic_load(p.ws_flags + (size_t)unit * p.nblk + j,
                                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                                 epoch) == kAgg;   // one word for the wave: uniform
                    __atomic_signal_fence(__ATOMIC_SEQ_CST);
                    WKVState x;
                    if (have) {
                        const float *d = p.ws_agg + (((size_t)unit * p.nblk + j) * 64 + lane) * 4;
                        coherent_load2(d, x.aa, x.bb);
                        coherent_load2(d + 2, x.anc, x.n);
                    } else {
                        x = wkv_empty();
                        for (int i = 0; i < kWkvChainBlock; ++i) {
                            const unsigned off = c < C ? (unsigned)(((j * kWkvChainBlock + i) * C + c) * 4)
                                                       : kOutOfRange;
                            wkv_step<false>(x, w2, wu2, buffer_load4(rk, off), buffer_load4(rv, off));
                        }
                        if (lane == 0) atomicAdd(p.ws_ctr + 3, 1u);
                    }
                    cin = wkv_combine(cin, x, (float)kWkvChainBlock, w2);
                }
            }
            for (int jb = 0; jb < (all_ok || p.ticket ? blk : 0); jb += kBlkLoads) {
                WKVState xs[kBlkLoads];
#pragma unroll
                for (int q = 0; q < kBlkLoads; ++q) {
                    if (jb + q < blk) {
                        const float *d = p.ws_agg + (((size_t)unit * p.nblk + jb + q) * 64 + lane) * 4;
                        coherent_load2(d, xs[q].aa, xs[q].bb);
                        coherent_load2(d + 2, xs[q].anc, xs[q].n);
                    }
                }
#pragma unroll
                for (int q = 0; q < kBlkLoads; ++q)
                    if (jb + q < blk) cin = wkv_combine(cin, xs[q], (float)kWkvChainBlock, w2);
            }
            wait_stores_complete();   // nothing but the output stores is outstanding below
        }

        // state entering this wave's steps: the block's entering state, then the
        // summaries of the earlier waves of the block
        WKVState ent = cin;
        for (int j = 0; j < wv; ++j) ent = wkv_combine(ent, sums[j][lane], (float)kWkvChainSub, w2);

        // outputs of this wave's steps from the registers
        s = ent;
        const unsigned off0 = c < C ? (unsigned)((t0 * C + c) * 4) : kOutOfRange;
        const unsigned dstep = c < C ? (unsigned)(C * 4) : 0u;
        auto out_step = [&](int i) {
            buffer_store4(ry, off0 + (unsigned)i * dstep, wkv_step<true>(s, w2, wu2, kc[i], vc[i]));
        };
        if (n == kWkvChainSub) {
#pragma unroll
            for (int i = 0; i < kWkvChainSub; ++i) out_step(i);
        } else {
#pragma unroll
            for (int i = 0; i < kWkvChainSub; ++i)
                if (i < n) out_step(i);
        }
        if (p.state_out && n > 0 && t0 + n == T && c < C) wkv_store_state(p.state_out, s, w2, p.B, C, b, c);
    }
    finish();
}

// Walk mode: a workgroup of W waves walks the time blocks of 64 channels of one
// batch row; wave j owns steps j*SUB ... j*SUB+SUB-1 of each block, held in
// registers.  Per block: waves 0..W-2 summarise their steps from the empty state,
// the summaries go through LDS, and every wave combines the block's entering state
// with the summaries of the waves before it and runs its outputs.  Each register is
// reloaded with the next block's step as soon as its output is written, so the next
// block's loads are in flight through the output and summary passes without a
// second register buffer.  A wave has at most 3 SUB memory operations outstanding.
// k and v are read once: their loads carry the non-temporal hint (measured ~12%
// faster than default caching at 8 x 1024 x 4096; the hint on the stores was slower).
//
template <int W, int SUB>
__global__ __launch_bounds__(64 * W, W / 2) void wkv_walk_fwd(WKVParams p) {
    constexpr int BLK = W * SUB;
    __shared__ WKVState sums[W - 1][64];   // the summaries that later waves need
    __shared__ WKVState carry[64];         // state after the previous block
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int unit = blockIdx.x;
    const int b = unit / p.ncblk, c = (unit - b * p.ncblk) * 64 + lane;
    const int T = p.T, C = p.C;
    const int cc = min(c, C - 1);
    const float w2 = p.w[cc] * kLog2e, u2 = p.u[cc] * kLog2e, wu2 = w2 + u2;
    WKVState cin = wkv_load_state(p.state_in, p.B, C, b, cc);
    const size_t row0 = (size_t)b * T * C;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y + row0, T * C * 4);
    const int nblk = (T + BLK - 1) / BLK;
    // lane part of the offsets (channel; out of range past the last channel), step part
    // in a scalar register, clamped to the last step so that it is always in range (a
    // step past the end reloads that row, unused)
    const unsigned voff = c < C ? (unsigned)(c * 4) : kOutOfRange;
    auto soff = [&](int t) { return (unsigned)(min(t, T - 1) * C * 4); };

    // the first block's steps, in the order of the output loop's memory operations
    // (a store, dropped as out of range, then the two loads), so that the waits
    // the compiler places at the loop head fit both the first and the later blocks
    float kr[SUB], vr[SUB];
#pragma unroll
    for (int i = 0; i < SUB; ++i) {
        buffer_store4s(ry, kOutOfRange, (unsigned)(i * 4), 0.f);
        kr[i] = buffer_load4s<kNonTemporal>(rk, voff, soff(wv * SUB + i));
        vr[i] = buffer_load4s<kNonTemporal>(rv, voff, soff(wv * SUB + i));
        __builtin_amdgcn_sched_barrier(0);   // keep this order
    }
    for (int blk = 0; blk < nblk; ++blk) {
        const int t0 = blk * BLK + wv * SUB, n = min(max(T - t0, 0), SUB);
        WKVState s = wkv_empty();
        if (wv < W - 1) {
            if (n == SUB) {
#pragma unroll
                for (int i = 0; i < SUB; ++i) wkv_absorb_step(s, w2, kr[i], vr[i]);
            } else {
#pragma unroll
                for (int i = 0; i < SUB; ++i)
                    if (i < n) wkv_absorb_step(s, w2, kr[i], vr[i]);
            }
        }
        __syncthreads();   // the previous block's summaries are read and its carry written
        if (blk > 0) cin = carry[lane];
        if (wv < W - 1) sums[wv][lane] = s;
        __syncthreads();
        s = cin;
        for (int j = 0; j < wv; ++j) s = wkv_combine(s, sums[j][lane], (float)SUB, w2);
        if (n == SUB) {
            // next block's steps (out of range after the last block: no traffic)
            const unsigned vn = blk + 1 < nblk ? voff : kOutOfRange;
#pragma unroll
            for (int i = 0; i < SUB; ++i) {
                buffer_store4s(ry, voff, (unsigned)((t0 + i) * C * 4), wkv_out_step(s, w2, wu2, kr[i], vr[i]));
                kr[i] = buffer_load4s<kNonTemporal>(rk, vn, soff(t0 + BLK + i));
                vr[i] = buffer_load4s<kNonTemporal>(rv, vn, soff(t0 + BLK + i));
            }
        } else {   // the last block, ragged
#pragma unroll
            for (int i = 0; i < SUB; ++i)
                if (i < n) buffer_store4s(ry, voff, (unsigned)((t0 + i) * C * 4), wkv_out_step(s, w2, wu2, kr[i], vr[i]));
        }
        if (p.state_out && n > 0 && t0 + n == T && c < C) wkv_store_state(p.state_out, s, w2, p.B, C, b, c);
        if (wv == W - 1) carry[lane] = s;
    }
}

// Row-owning sweep (DRS_FORCE_ROWS): a workgroup owns 256 W neighbouring channels
// of one batch row -- each lane four of them (16-byte loads), so every wave reads
// 1 KB and the workgroup W KB of each row it visits -- over a span of S steps.  A
// lane runs its channels through the span in order: the span's summary from the
// empty state (published), the state entering the span from a look-back over the
// earlier spans of the same channels, the inclusive state (published), then the
// outputs from the registers.  The look-back walks back from the previous span
// and stops at the first span whose inclusive state is out, combining the
// summaries of the spans it passes on the way (decoupled look-back).  Each wave
// is a chain of its own (its channels have their own flags); the kernel has no
// barrier.  Slots are unit-major: [unit][span][wave], data [2][4][2][64] words of
// 8 bytes per slot (summary, inclusive; channel; (aa, bb), (anchor, n); lane).
constexpr unsigned kIncl = 2u;   // flag state: the inclusive state is out as well
#ifndef DRS_WKV_ROWS_BATCH
#define DRS_WKV_ROWS_BATCH 2
#endif
constexpr int kRowsBatch = DRS_WKV_ROWS_BATCH;   // earlier spans' states loaded at once

__device__ __forceinline__ float lane_f(const u32x4 &x, int j) { return __uint_as_float(x[j]); }

template <int W, int S>
__global__ __launch_bounds__(64 * W) void wkv_rows_fwd(WKVParams p) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const unsigned units = (unsigned)p.B * (unsigned)p.ncblk;
    const int span = (int)(blockIdx.x / units), unit = (int)(blockIdx.x - (unsigned)span * units);
    const int b = unit / p.ncblk, grp = unit - b * p.ncblk;
    const int T = p.T, C = p.C;
    const int c = (grp * W + wv) * 256 + 4 * lane;   // channels c .. c + 3 (C % 4 == 0: all or none)
    const bool valid = c < C;
    const int cc = valid ? c : 0;
    // every wave of the launch reads the same epoch (advanced by the kernel before it)
    const unsigned epoch = __hip_atomic_load(p.ws_ctr + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float w2[4], wu2[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        w2[j] = p.w[cc + j] * kLog2e;
        wu2[j] = w2[j] + p.u[cc + j] * kLog2e;
    }
    const int t0 = span * S, n = min(S, T - t0);
    const size_t row0 = (size_t)b * T * C;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + row0, T * C * 4);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(p.y + row0, T * C * 4);
    auto off_of = [&](int t, bool live) { return live && valid ? (unsigned)((t * C + c) * 4) : kOutOfRange; };

    u32x4 kr[S], vr[S];
#pragma unroll
    for (int i = 0; i < S; ++i) {
        kr[i] = buffer_load16<kNonTemporal>(rk, off_of(t0 + i, i < n));
        vr[i] = buffer_load16<kNonTemporal>(rv, off_of(t0 + i, i < n));
    }

    WKVState a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = wkv_empty();
    if (n == S) {
#pragma unroll
        for (int i = 0; i < S; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) wkv_absorb_step(a[j], w2[j], lane_f(kr[i], j), lane_f(vr[i], j));
    } else {
#pragma unroll
        for (int i = 0; i < S; ++i)
            if (i < n)
#pragma unroll
                for (int j = 0; j < 4; ++j) wkv_absorb_step(a[j], w2[j], lane_f(kr[i], j), lane_f(vr[i], j));
    }

    auto data = [&](int sp, int which) {
        return p.ws_agg + ((((size_t)unit * p.nblk + sp) * W + wv) * 2 + which) * (8 * 64 * 2);
    };
    auto flag_of = [&](int sp) { return p.ws_flags + ((size_t)unit * p.nblk + sp) * W + wv; };
    auto put = [&](float *d, const WKVState (&st)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            coherent_store2(d + ((2 * j) * 64 + lane) * 2, st[j].aa, st[j].bb);
            coherent_store2(d + ((2 * j + 1) * 64 + lane) * 2, st[j].anc, st[j].n);
        }
    };
    auto get = [&](const float *d, WKVState (&st)[4]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            coherent_load2(d + ((2 * j) * 64 + lane) * 2, st[j].aa, st[j].bb);
            coherent_load2(d + ((2 * j + 1) * 64 + lane) * 2, st[j].anc, st[j].n);
        }
    };
    auto raise_flag = [&](int sp, unsigned state) {
        wait_stores_complete();   // the data are visible device-wide before the flag
        if (lane == 0) __hip_atomic_store(flag_of(sp), flag_word(epoch, state), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    const bool last = span == p.nblk - 1;
    if (!last) {
        put(data(span, 0), a);
        raise_flag(span, kAgg);
    }

    // state entering the span: a window of up to 64 earlier spans at a time, lane l
    // watching span base - l; the window closes at the nearest span whose inclusive
    // state is out (or at span 0), and its states are combined nearest first
    WKVState ent[4];
    {
        WKVState acc[4];
        bool have = false, closed = false;
        float accn = 0.f;   // steps that acc spans
        int base = span - 1;
        while (base >= 0 && !closed) {
            const int spl = base - lane;
            unsigned st = 0u;
            int cnt = min(64, base + 1);
            if (!p.own_aggs) {
                for (unsigned it = 0; it < p.spin_limit; ++it) {
                    if (spl >= 0 && st != kIncl) {
                        const unsigned f = flag_state(
                            __hip_atomic_load(flag_of(spl), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), epoch);
                        st = f > st ? f : st;
                    }
                    const unsigned long long incl = __ballot(spl >= 0 && st == kIncl);
                    const unsigned long long rdy = __ballot(spl < 0 || st != 0u);
                    const int e = incl ? __builtin_ctzll(incl) + 1 : 64;   // lanes the window needs
                    const unsigned long long m = e >= 64 ? ~0ull : (1ull << e) - 1ull;
                    cnt = min(e, base + 1);
                    if ((rdy & m) == m) break;
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            for (int j0 = 0; j0 < cnt && !closed; j0 += kRowsBatch) {
                WKVState xs[kRowsBatch][4];
                unsigned sts[kRowsBatch];
#pragma unroll
                for (int q = 0; q < kRowsBatch; ++q) {
                    sts[q] = j0 + q < cnt ? __builtin_amdgcn_readlane(st, j0 + q) : 0u;
                    if (sts[q] != 0u) get(data(base - j0 - q, sts[q] == kIncl ? 1 : 0), xs[q]);
                }
#pragma unroll
                for (int q = 0; q < kRowsBatch; ++q) {
                    if (j0 + q < cnt && !closed) {
                        if (sts[q] == 0u) {   // not out within the wait (or forced): from k and v
                            const int sp = base - j0 - q;
#pragma unroll
                            for (int j = 0; j < 4; ++j) xs[q][j] = wkv_empty();
#pragma unroll 1
                            for (int i = 0; i < S; ++i) {
                                const u32x4 kk = buffer_load16(rk, off_of(sp * S + i, true));
                                const u32x4 vv = buffer_load16(rv, off_of(sp * S + i, true));
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    wkv_absorb_step(xs[q][j], w2[j], lane_f(kk, j), lane_f(vv, j));
                            }
                            if (lane == 0) atomicAdd(p.ws_ctr + 3, 1u);
                        }
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            acc[j] = have ? wkv_combine(xs[q][j], acc[j], accn, w2[j]) : xs[q][j];
                        have = true;
                        accn += (float)S;
                        closed = sts[q] == kIncl;
                    }
                }
            }
            base -= cnt;
        }
        if (closed) {
#pragma unroll
            for (int j = 0; j < 4; ++j) ent[j] = acc[j];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const WKVState init = wkv_load_state(p.state_in, p.B, C, b, cc + j);
                ent[j] = have ? wkv_combine(init, acc[j], accn, w2[j]) : init;
            }
        }
    }
    if (!last) {
        WKVState inc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) inc[j] = wkv_combine(ent[j], a[j], (float)S, w2[j]);
        put(data(span, 1), inc);
        raise_flag(span, kIncl);
    }

    // outputs from the registers
    auto out = [&](int i) {
        u32x4 yo;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            yo[j] = __float_as_uint(wkv_out_step(ent[j], w2[j], wu2[j], lane_f(kr[i], j), lane_f(vr[i], j)));
        buffer_store16(ry, off_of(t0 + i, true), yo);
    };
    if (n == S) {
#pragma unroll
        for (int i = 0; i < S; ++i) out(i);
    } else {
#pragma unroll
        for (int i = 0; i < S; ++i)
            if (i < n) out(i);
    }
    if (p.state_out && last && valid)
#pragma unroll
        for (int j = 0; j < 4; ++j) wkv_store_state(p.state_out, ent[j], w2[j], p.B, C, b, c + j);
}

// The epoch of a rows launch, advanced by a one-thread kernel ahead of it on the
// stream (so the sweep itself counts nothing: a finish counter taken by every wave
// serialised at ~40 ns per wave).  Graph replays run it too.
__global__ void wkv_rows_epoch(unsigned *ctr) {
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
    wkv_run<false, kWkvPF>(s, w2, w2 + u2, p.k + base, p.v + base, nullptr, t0, t1, p.C);
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
    wkv_run<true, kWkvPF>(s, w2, w2 + u2, p.k + base, p.v + base, p.y + base, t0, t1, p.C);
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
    const long smax = ((long)T + 63) / 64;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    long L = ((long)T + s - 1) / s;
    L = (L + 15) / 16 * 16;
    if (((long)T + L - 1) / L > 65535) L = ((long)T + 65534) / 65535;   // grid z limit
    *seg_len = (int)L;
    *nseg = (int)(((long)T + L - 1) / L);
}

bool wkv_chain_supported(int B, int T, int C) {
    const long nblk = ((long)T + kWkvChainBlock - 1) / kWkvChainBlock;
    return (long)T * C * 4 < (1L << 31) && nblk <= kWkvChainMaxBlocks &&
           (long)B * (((long)C + 63) / 64) * nblk < (1L << 31);
}

size_t wkv_chain_ws_bytes(int B, int T, int C) {
    const size_t units = (size_t)B * (((size_t)C + 63) / 64), nblk = ((size_t)T + kWkvChainBlock - 1) / kWkvChainBlock;
    const size_t flags = (units * nblk * 8 + 255) / 256 * 256;
    return kWkvCtrBytes + flags + units * nblk * 64 * 4 * sizeof(float);
}

hipError_t wkv_launch_chain(const WKVParams &p, hipStream_t stream) {
    if (p.walk) {
        hipLaunchKernelGGL((wkv_walk_fwd<kWkvWalkWaves, kWkvWalkSub>), dim3((unsigned)(p.B * p.ncblk)),
                           dim3(64 * kWkvWalkWaves), 0, stream, p);
        return hipGetLastError();
    }
    dim3 grid((unsigned)(p.B * p.ncblk * p.nblk));
    hipLaunchKernelGGL(wkv_chain_fwd, grid, dim3(64 * kWkvChainWaves), 0, stream, p);
    return hipGetLastError();
}

#ifndef DRS_WKV_ROWS_WAVES
#define DRS_WKV_ROWS_WAVES 4
#endif
#ifndef DRS_WKV_ROWS_SPAN
#define DRS_WKV_ROWS_SPAN 16
#endif
constexpr int kRowsWaves = DRS_WKV_ROWS_WAVES, kRowsSpan = DRS_WKV_ROWS_SPAN;

void wkv_rows_plan(int B, int T, int C, int *ngroups, int *nspan) {
    *ngroups = (int)(((long)C + 256L * kRowsWaves - 1) / (256L * kRowsWaves));
    *nspan = (int)(((long)T + kRowsSpan - 1) / kRowsSpan);
}

bool wkv_rows_supported(int B, int T, int C) {
    int g, n;
    wkv_rows_plan(B, T, C, &g, &n);
    return C % 4 == 0 && (long)T * C * 4 < (1L << 31) && (long)B * g * n * kRowsWaves < (1L << 31);
}

size_t wkv_rows_ws_bytes(int B, int T, int C) {
    int g, n;
    wkv_rows_plan(B, T, C, &g, &n);
    const size_t slots = (size_t)B * g * n * kRowsWaves;
    return kWkvCtrBytes + (slots * 8 + 255) / 256 * 256 + slots * 2 * 8 * 64 * 2 * sizeof(float);
}

void wkv_rows_layout(char *ws, WKVParams &p) {
    wkv_rows_plan(p.B, p.T, p.C, &p.ncblk, &p.nblk);
    const size_t slots = (size_t)p.B * p.ncblk * p.nblk * kRowsWaves;
    p.ws_ctr = reinterpret_cast<unsigned *>(ws);
    p.ws_flags = reinterpret_cast<unsigned long long *>(ws + kWkvCtrBytes);
    p.ws_agg = reinterpret_cast<float *>(ws + kWkvCtrBytes + (slots * 8 + 255) / 256 * 256);
}

hipError_t wkv_launch_rows(const WKVParams &p, hipStream_t stream) {
    hipLaunchKernelGGL(wkv_rows_epoch, dim3(1), dim3(64), 0, stream, p.ws_ctr);
    hipLaunchKernelGGL((wkv_rows_fwd<kRowsWaves, kRowsSpan>), dim3((unsigned)(p.B * p.ncblk * p.nblk)),
                       dim3(64 * kRowsWaves), 0, stream, p);
    return hipGetLastError();
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
