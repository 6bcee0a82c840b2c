// ema.hip -- gated element-wise EMA forward on gfx950.
//
// Definition (RetNet issue #21: cumulative_ema, its associative operator and
// the variant in which a layer produces factors and values of one shape): per
// channel, out_t = f_t out_{t-1} + x_t, the factor of step t multiplying the
// output carried in from the step before; reverse = the forward recurrence on
// time-reversed inputs, the output reversed back (an index map here).  The
// operator on spans, (x_a, f_a) o (x_b, f_b) = (x_a f_b + x_b, f_a f_b), is what
// the time-parallel parts below combine.
//
// One workgroup = kEmaWaves waves = 64 channels of one batch row; wave j owns
// kEmaSub consecutive steps of a time block of kEmaWaves * kEmaSub steps and
// keeps its x and f in registers.  Per block: waves 0 .. kEmaWaves-2 summarise
// their steps (local scan A from zero, factor product P); the summaries go
// through LDS; wave j's entering state is the block's entering state combined
// with the summaries of waves 0 .. j-1; every wave then runs its outputs from
// its registers.
//   walk mode      (enough channel groups to fill the GPU, or more (group,
//                  block) pairs than one resident round): the workgroup walks
//                  all time blocks, the next block's loads in flight, the state
//                  entering the next block taken from the last wave's run;
//   look-back mode (few groups and blocks): one workgroup per time block; the
//                  block aggregate is published and later blocks fold the
//                  earlier aggregates onto the initial state in a fixed order.
// x, f and y are read and written once (bounds-checked buffer access; rows past
// the end and channels past C are out of range).  In walk mode with bf16 data and
// an even channel count each lane takes two neighbouring channels (one 4-byte
// access per step) and a workgroup has twice the waves, each with half the steps,
// over 128 channels; the fused bidirectional kernel below does the same.
#include "common.h"
#include "ema.h"
#include "lookback.h"

namespace drs {

template <typename TI> struct EmaIO;
template <> struct EmaIO<float> {
    static constexpr int SZ = 4;
    __device__ static float load(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
        return buffer_load4s<kNonTemporal>(r, voff, soff);
    }
    __device__ static void store(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, float v) {
        buffer_store4s(r, voff, soff, v);
    }
};
template <> struct EmaIO<uint16_t> {
    static constexpr int SZ = 2;
    __device__ static float load(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
        const unsigned short b = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kNonTemporal);
        return __uint_as_float((unsigned)b << 16);
    }
    __device__ static void store(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, float v) {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_bits(v), r, voff, soff, 0);
    }
};

// Two neighbouring bf16 channels of one lane: one 4-byte access per step, so that a
// wave moves 256 bytes of a row per instruction (one 2-byte channel per lane moved 128,
// and measured ~12% below fp32 in bytes per second at the same shape).
struct EmaIOPair {
    static constexpr int SZ = 2;
    __device__ static void load(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, float (&v)[2]) {
        const unsigned w = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNonTemporal);
        v[0] = bf16_lo(w);
        v[1] = bf16_hi(w);
    }
    __device__ static void store(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, const float (&v)[2]) {
        __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(v[0], v[1]), r, voff, soff, 0);
    }
};
template <typename TI, int CPL> struct EmaLane;
template <typename TI> struct EmaLane<TI, 1> {
    static constexpr int SZ = EmaIO<TI>::SZ;
    __device__ static void load(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, float (&v)[1]) {
        v[0] = EmaIO<TI>::load(r, voff, soff);
    }
    __device__ static void store(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff, const float (&v)[1]) {
        EmaIO<TI>::store(r, voff, soff, v[0]);
    }
};
template <> struct EmaLane<uint16_t, 2> : EmaIOPair {};

struct EmaSum {
    float a, p;   // local scan from zero, product of the factors
};

// CPL channels per lane (2: bf16 pairs, walk mode only); a time block keeps kEmaBlock
// steps over W waves of SUB steps each, so both layouts hold the same registers.
template <typename TI, bool WALK, int CPL = 1>
__global__ __launch_bounds__(64 * (CPL == 2 ? 2 * kEmaWaves : kEmaWaves), CPL == 2 ? 1 : 2) void ema_fwd(EmaParams p) {
    static_assert(CPL == 1 || (WALK && sizeof(TI) == 2), "channel pairs: bf16, walk mode");
    constexpr int W = CPL == 2 ? 2 * kEmaWaves : kEmaWaves, SUB = kEmaBlock / W;
    typedef EmaLane<TI, CPL> IO;
    __shared__ EmaSum sums[W - 1][64 * CPL];
    __shared__ float carry[64 * CPL];
    __shared__ unsigned info[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const unsigned units = (unsigned)p.B * (unsigned)p.ncblk;
    const unsigned total = WALK ? units : units * (unsigned)p.nblk;
    unsigned vid = blockIdx.x, epoch = 0;
    if constexpr (!WALK) {   // virtual ids in start order, earlier blocks first
        if (tid == 0) {
            info[0] = atomicAdd(p.ws_ctr + 0, 1u);
            info[1] = __hip_atomic_load(p.ws_ctr + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        vid = info[0];
        epoch = info[1];
    }
    auto finish = [&]() {   // look-back: the last workgroup to finish re-arms the counters
        if constexpr (!WALK) {
            __syncthreads();
            if (tid == 0) {
                const unsigned done = atomicAdd(p.ws_ctr + 1, 1u);
                if (done == total - 1) {
                    __hip_atomic_store(p.ws_ctr + 0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(p.ws_ctr + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(p.ws_ctr + 2, epoch + 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
    };
    if (vid >= total) {   // only with counters that were not zero before the first use
        if (tid == 0) atomicAdd(p.ws_ctr + 3, 1u);
        finish();
        return;
    }
    const int blk0 = WALK ? 0 : (int)(vid / units);
    const int blk1 = WALK ? p.nblk : blk0 + 1;
    const int unit = (int)(vid - (unsigned)blk0 * units);
    // the lane's first channel (CPL neighbours; C is a multiple of CPL)
    const int b = unit / p.ncblk, c = ((unit - b * p.ncblk) * 64 + lane) * CPL;
    const int T = p.T, C = p.C;

    // the initial state, read before anything is published (state_out may alias it)
    float cin[CPL];
#pragma unroll
    for (int q = 0; q < CPL; ++q) cin[q] = p.state_in ? p.state_in[(size_t)b * C + min(c + q, C - 1)] : 0.f;

    const size_t row0 = (size_t)b * T * C;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const char *>(p.x) + row0 * IO::SZ, T * C * IO::SZ);
    const __amdgpu_buffer_rsrc_t rf = make_rsrc(static_cast<const char *>(p.f) + row0 * IO::SZ, T * C * IO::SZ);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(static_cast<char *>(p.y) + row0 * IO::SZ, T * C * IO::SZ);
    // channel part of the offsets (out of range past the last channel); the step part
    // is wave-uniform (scalar), clamped to the last step so that it stays in range
    const unsigned voff = c < C ? (unsigned)(c * IO::SZ) : kOutOfRange;
    auto soff = [&](int t) {
        const int tt = min(t, T - 1);
        return (unsigned)((p.reverse ? T - 1 - tt : tt) * C * IO::SZ);
    };
    auto span = [&](int blk, int j) { return min(max(T - (blk * kEmaBlock + j * SUB), 0), SUB); };

    struct Buf {
        float x[SUB][CPL], f[SUB][CPL];
    };
    auto load = [&](Buf &bf, int blk) {
        const int t0 = blk * kEmaBlock + wv * SUB;
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
            const unsigned so = soff(t0 + i);
            IO::load(rx, voff, so, bf.x[i]);
            IO::load(rf, voff, so, bf.f[i]);
        }
    };

    auto block = [&](Buf &cur, Buf &nxt, int blk, bool prefetch) {
        if (prefetch) load(nxt, blk + 1);   // walk: in flight while this block is computed
        const int t0 = blk * kEmaBlock + wv * SUB, n = span(blk, wv);
        // summary of this wave's steps (the last wave's is never needed)
        EmaSum sm[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) sm[q] = EmaSum{0.f, 1.f};
        if (wv < W - 1) {
            if (n == SUB) {
#pragma unroll
                for (int i = 0; i < SUB; ++i)
#pragma unroll
                    for (int q = 0; q < CPL; ++q) {
                        sm[q].a = fmaf(cur.f[i][q], sm[q].a, cur.x[i][q]);
                        sm[q].p *= cur.f[i][q];
                    }
            } else {
#pragma unroll
                for (int i = 0; i < SUB; ++i)
                    if (i < n) {
#pragma unroll
                        for (int q = 0; q < CPL; ++q) {
                            sm[q].a = fmaf(cur.f[i][q], sm[q].a, cur.x[i][q]);
                            sm[q].p *= cur.f[i][q];
                        }
                    }
            }
        }
        if constexpr (!WALK) wait_stores_complete();   // the initial state has been read
        __syncthreads();   // the previous block's summaries are read and its carry written
        if (WALK && blk > 0) {
#pragma unroll
            for (int q = 0; q < CPL; ++q) cin[q] = carry[lane * CPL + q];
        }
        if (wv < W - 1) {
#pragma unroll
            for (int q = 0; q < CPL; ++q) sums[wv][lane * CPL + q] = sm[q];
        }
        __syncthreads();

        if constexpr (!WALK) {
            // publish the block aggregate, then fold the earlier blocks' aggregates
            // into the initial state in order (fixed order: bitwise reproducible).  The
            // last wave, which has no summary of its own, forms the aggregate: the
            // other waves' summaries, then its own (full) span from its registers.
            const size_t slot = (size_t)unit * p.nblk + blk;
            if (blk < p.nblk - 1 && wv == W - 1) {
                EmaSum agg = sums[0][lane];
#pragma unroll
                for (int j = 1; j < W - 1; ++j) {
                    agg.a = fmaf(agg.a, sums[j][lane].p, sums[j][lane].a);
                    agg.p *= sums[j][lane].p;
                }
                // this wave's own span (a full one: the block has a successor)
#pragma unroll
                for (int i = 0; i < SUB; ++i) {
                    agg.a = fmaf(cur.f[i][0], agg.a, cur.x[i][0]);
                    agg.p *= cur.f[i][0];
                }
                float *d = p.ws_agg + (slot * 64 + lane) * 2;
                coherent_store2(d, agg.a, agg.p);
                wait_stores_complete();
                if (lane == 0)
                    __hip_atomic_store(p.ws_flags + slot, flag_word(epoch, kAgg), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            for (int j0 = 0; j0 < blk; j0 += 64) {
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
                if (!__all(ok) && lane == 0) atomicAdd(p.ws_ctr + 3, 1u);   // gave up (never expected)
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            constexpr int kLoads = 8;
            for (int jb = 0; jb < blk; jb += kLoads) {
                EmaSum xs[kLoads];
#pragma unroll
                for (int q = 0; q < kLoads; ++q)
                    if (jb + q < blk)
                        coherent_load2(p.ws_agg + (((size_t)unit * p.nblk + jb + q) * 64 + lane) * 2, xs[q].a, xs[q].p);
#pragma unroll
                for (int q = 0; q < kLoads; ++q)
                    if (jb + q < blk) cin[0] = fmaf(cin[0], xs[q].p, xs[q].a);
            }
            wait_stores_complete();   // nothing but the output stores is outstanding below
        }

        // entering state of this wave: the block's, then the earlier waves' spans
        float h[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            h[q] = cin[q];
            for (int j = 0; j < wv; ++j) h[q] = fmaf(h[q], sums[j][lane * CPL + q].p, sums[j][lane * CPL + q].a);
        }
        auto out_step = [&](int i) {
#pragma unroll
            for (int q = 0; q < CPL; ++q) h[q] = fmaf(cur.f[i][q], h[q], cur.x[i][q]);
            IO::store(ry, voff, soff(t0 + i), h);
        };
        if (n == SUB) {
#pragma unroll
            for (int i = 0; i < SUB; ++i) out_step(i);
        } else {
#pragma unroll
            for (int i = 0; i < SUB; ++i)
                if (i < n) out_step(i);
        }
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            if (p.state_out && n > 0 && t0 + n == T && c + q < C) p.state_out[(size_t)b * C + c + q] = h[q];
            if (WALK && wv == W - 1) carry[lane * CPL + q] = h[q];   // the state entering the next block
        }
    };

    Buf ba, bb;
    load(ba, blk0);
    if constexpr (WALK) {
        int blk = 0;
        for (; blk + 1 < blk1; blk += 2) {   // whole pairs: the same memory-operation order on every path
            block(ba, bb, blk, true);
            block(bb, ba, blk + 1, true);
        }
        if (blk < blk1) block(ba, bb, blk, true);
    } else {
        block(ba, bb, blk0, false);
    }
    finish();
}

// Bidirectional EMA, fused (walk layout: one workgroup per 64 channels of one
// batch row walks all time blocks): y_t = fwd_t + rev_t with fwd the forward scan
// and rev the reverse one (out_t = f_t out_{t+1} + x_t), both from zero.
//   pass 1: per block, every wave summarises its span in both directions (the
//           forward scan from zero, the reverse scan from zero, the factor
//           product); the block aggregates of both directions go to the workspace;
//   carries: wave 0 folds the forward aggregates from the first block, wave 1 the
//           reverse ones from the last, giving every block both entering states;
//   pass 2: per block, each wave's entering states come from the block's and the
//           other waves' span summaries; it runs its forward outputs into registers,
//           then the reverse scan, and stores the sum once.
// x and f are read twice and y written once (composing two calls and an add would
// read x, f twice and move y three times more).
struct EmaSum3 {
    float af, ar, p;   // forward scan from zero, reverse scan from zero, factor product
};

// CPL channels per lane as in ema_fwd (2: bf16 pairs, over twice the waves).
template <typename TI, int CPL = 1>
__global__ __launch_bounds__(64 * (CPL == 2 ? 2 * kEmaWaves : kEmaWaves), CPL == 2 ? 1 : 2) void ema_bidir(EmaParams p) {
    static_assert(CPL == 1 || sizeof(TI) == 2, "channel pairs: bf16");
    constexpr int W = CPL == 2 ? 2 * kEmaWaves : kEmaWaves, SUB = kEmaBlock / W, NL = 64 * CPL;
    typedef EmaLane<TI, CPL> IO;
    __shared__ EmaSum3 sums[W][NL];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int unit = blockIdx.x;
    const int b = unit / p.ncblk, c = ((unit - b * p.ncblk) * 64 + lane) * CPL;
    const int T = p.T, C = p.C, nblk = p.nblk;
    // workspace of this unit: [block][5][NL] = forward aggregate, reverse aggregate,
    // product, then the entering forward and reverse states (channel lane * CPL + q)
    float *wsu = p.ws_agg + (size_t)unit * nblk * 5 * NL;
    auto wsf = [&](int blk, int field, int q) -> float & {
        return wsu[((size_t)blk * 5 + field) * NL + lane * CPL + q];
    };

    const size_t row0 = (size_t)b * T * C;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(static_cast<const char *>(p.x) + row0 * IO::SZ, T * C * IO::SZ);
    const __amdgpu_buffer_rsrc_t rf = make_rsrc(static_cast<const char *>(p.f) + row0 * IO::SZ, T * C * IO::SZ);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(static_cast<char *>(p.y) + row0 * IO::SZ, T * C * IO::SZ);
    const unsigned voff = c < C ? (unsigned)(c * IO::SZ) : kOutOfRange;
    auto soff = [&](int t) { return (unsigned)(min(t, T - 1) * C * IO::SZ); };
    auto span = [&](int blk, int j) { return min(max(T - (blk * kEmaBlock + j * SUB), 0), SUB); };

    struct Buf {
        float x[SUB][CPL], f[SUB][CPL];
        float cf[CPL], cr[CPL];   // pass 2: the block's entering states (prefetched with its data)
    };
    auto load = [&](Buf &bf, int blk) {
        const int t0 = blk * kEmaBlock + wv * SUB;
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
            const unsigned so = soff(t0 + i);
            IO::load(rx, voff, so, bf.x[i]);
            IO::load(rf, voff, so, bf.f[i]);
        }
    };
    // both summaries of this wave's span for channel q (steps past the end: identity)
    auto summarise = [&](const Buf &cur, int n, int q) {
        EmaSum3 sm = {0.f, 0.f, 1.f};
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
            const bool in = i < n;
            sm.af = in ? fmaf(cur.f[i][q], sm.af, cur.x[i][q]) : sm.af;
            sm.p *= in ? cur.f[i][q] : 1.f;
        }
#pragma unroll
        for (int i = SUB - 1; i >= 0; --i) sm.ar = i < n ? fmaf(cur.f[i][q], sm.ar, cur.x[i][q]) : sm.ar;
        return sm;
    };

    // ---- pass 1: block aggregates of both directions -------------------------------
    auto pass1 = [&](Buf &cur, Buf &nxt, int blk) {
        if (blk + 1 < nblk) load(nxt, blk + 1);
#pragma unroll
        for (int q = 0; q < CPL; ++q) sums[wv][lane * CPL + q] = summarise(cur, span(blk, wv), q);
        __syncthreads();
        if (wv == 0) {
#pragma unroll
            for (int q = 0; q < CPL; ++q) {
                const int l = lane * CPL + q;
                EmaSum3 a = sums[0][l];
#pragma unroll
                for (int j = 1; j < W; ++j) {
                    a.af = fmaf(a.af, sums[j][l].p, sums[j][l].af);
                    a.p *= sums[j][l].p;
                }
                wsf(blk, 0, q) = a.af;
                wsf(blk, 2, q) = a.p;
            }
        } else if (wv == 1) {
#pragma unroll
            for (int q = 0; q < CPL; ++q) {
                const int l = lane * CPL + q;
                float r = sums[W - 1][l].ar;
#pragma unroll
                for (int j = W - 2; j >= 0; --j) r = fmaf(sums[j][l].p, r, sums[j][l].ar);
                wsf(blk, 1, q) = r;
            }
        }
        __syncthreads();   // sums is rewritten by the next block
    };
    Buf ba, bb;
    load(ba, 0);
    {
        int blk = 0;
        for (; blk + 1 < nblk; blk += 2) {
            pass1(ba, bb, blk);
            pass1(bb, ba, blk + 1);
        }
        if (blk < nblk) pass1(ba, bb, blk);
    }
    load(ba, 0);   // pass 2 starts at the first block again (in flight during the carries)

    // ---- entering states of every block (aggregates fetched eight blocks at a time) ---
    constexpr int kBatch = 8;
    if (wv == 0) {
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            float cf = 0.f;
            for (int b0 = 0; b0 < nblk; b0 += kBatch) {
                float a[kBatch], pr[kBatch];
#pragma unroll
                for (int k = 0; k < kBatch; ++k)
                    if (b0 + k < nblk) {
                        a[k] = wsf(b0 + k, 0, q);
                        pr[k] = wsf(b0 + k, 2, q);
                    }
#pragma unroll
                for (int k = 0; k < kBatch; ++k)
                    if (b0 + k < nblk) {
                        wsf(b0 + k, 3, q) = cf;
                        cf = fmaf(cf, pr[k], a[k]);
                    }
            }
        }
    } else if (wv == 1) {
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            float cr = 0.f;
            for (int b1 = nblk - 1; b1 >= 0; b1 -= kBatch) {
                float a[kBatch], pr[kBatch];
#pragma unroll
                for (int k = 0; k < kBatch; ++k)
                    if (b1 - k >= 0) {
                        a[k] = wsf(b1 - k, 1, q);
                        pr[k] = wsf(b1 - k, 2, q);
                    }
#pragma unroll
                for (int k = 0; k < kBatch; ++k)
                    if (b1 - k >= 0) {
                        wsf(b1 - k, 4, q) = cr;
                        cr = fmaf(pr[k], cr, a[k]);
                    }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
        ba.cf[q] = wsf(0, 3, q);
        ba.cr[q] = wsf(0, 4, q);
    }

    // ---- pass 2: outputs ---------------------------------------------------------------
    auto pass2 = [&](Buf &cur, Buf &nxt, int blk) {
        if (blk + 1 < nblk) {
            load(nxt, blk + 1);
#pragma unroll
            for (int q = 0; q < CPL; ++q) {
                nxt.cf[q] = wsf(blk + 1, 3, q);
                nxt.cr[q] = wsf(blk + 1, 4, q);
            }
        }
        const int t0 = blk * kEmaBlock + wv * SUB, n = span(blk, wv);
#pragma unroll
        for (int q = 0; q < CPL; ++q) sums[wv][lane * CPL + q] = summarise(cur, n, q);
        __syncthreads();
        float hf[CPL], hr[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
            const int l = lane * CPL + q;
            hf[q] = cur.cf[q];
            hr[q] = cur.cr[q];
            for (int j = 0; j < wv; ++j) hf[q] = fmaf(hf[q], sums[j][l].p, sums[j][l].af);
            for (int j = W - 1; j > wv; --j) hr[q] = fmaf(sums[j][l].p, hr[q], sums[j][l].ar);
        }
        float yf[SUB][CPL];
#pragma unroll
        for (int i = 0; i < SUB; ++i)
#pragma unroll
            for (int q = 0; q < CPL; ++q) {
                hf[q] = fmaf(cur.f[i][q], hf[q], cur.x[i][q]);
                yf[i][q] = hf[q];
            }
#pragma unroll
        for (int i = SUB - 1; i >= 0; --i) {
            if (i < n) {
                float o[CPL];
#pragma unroll
                for (int q = 0; q < CPL; ++q) {
                    hr[q] = fmaf(cur.f[i][q], hr[q], cur.x[i][q]);
                    o[q] = yf[i][q] + hr[q];
                }
                IO::store(ry, voff, soff(t0 + i), o);
            }
        }
        __syncthreads();   // sums is rewritten by the next block
    };
    {
        int blk = 0;
        for (; blk + 1 < nblk; blk += 2) {
            pass2(ba, bb, blk);
            pass2(bb, ba, blk + 1);
        }
        if (blk < nblk) pass2(ba, bb, blk);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

bool ema_supported(int B, int T, int C, int esize) {
    const long nblk = ((long)T + kEmaBlock - 1) / kEmaBlock;
    return (long)T * C * esize < (1L << 31) && (long)B * (((long)C + 63) / 64) * nblk < (1L << 31);
}

// Walk mode unless one resident round (two workgroups per CU) holds every
// (channel group, time block): beyond that, look-back workgroups start cold and
// wait on the previous round, 4-6x slower than a walk even over few channel
// groups (bf16: 299 vs 75 us at B=2, T=4096, C=4096; 115 vs 25 us at 16 x 1024 x 1024).
bool ema_walk(int B, int T, int C) {
    const long nblk = ((long)T + kEmaBlock - 1) / kEmaBlock, units = (long)B * (((long)C + 63) / 64);
    return units >= kEmaWalkUnits || nblk > kEmaMaxLookbackBlocks || units * nblk > kEmaOneRound;
}

size_t ema_ws_bytes(int B, int T, int C) {
    if (ema_walk(B, T, C)) return 0;
    const size_t units = (size_t)B * (((size_t)C + 63) / 64), nblk = ((size_t)T + kEmaBlock - 1) / kEmaBlock;
    const size_t flags = (units * nblk * 8 + 255) / 256 * 256;
    return kEmaCtrBytes + flags + units * nblk * 64 * 2 * sizeof(float);
}

template <typename TI>
hipError_t ema_launch_t(const EmaParams &p, hipStream_t s) {
    const dim3 block(64 * kEmaWaves);
    const unsigned units = (unsigned)p.B * (unsigned)p.ncblk;
    if (p.walk && sizeof(TI) == 2 && p.C % 2 == 0) {
        // bf16 channel pairs: 128 channels per workgroup of twice the waves
        EmaParams q = p;
        q.ncblk = (p.C + 127) / 128;
        hipLaunchKernelGGL((ema_fwd<uint16_t, true, 2>), dim3((unsigned)q.B * (unsigned)q.ncblk),
                           dim3(64 * 2 * kEmaWaves), 0, s, q);
    } else if (p.walk) {
        hipLaunchKernelGGL((ema_fwd<TI, true>), dim3(units), block, 0, s, p);
    } else {
        hipLaunchKernelGGL((ema_fwd<TI, false>), dim3(units * (unsigned)p.nblk), block, 0, s, p);
    }
    return hipGetLastError();
}

hipError_t ema_launch(const EmaParams &p, bool bf16, hipStream_t s) {
    return bf16 ? ema_launch_t<uint16_t>(p, s) : ema_launch_t<float>(p, s);
}

size_t ema_bidir_ws_bytes(int B, int T, int C) {
    // room for either layout: 64 channels per workgroup, or 128 in bf16 pairs
    const size_t nblk = ((size_t)T + kEmaBlock - 1) / kEmaBlock;
    const size_t lanes1 = ((size_t)C + 63) / 64 * 64, lanes2 = ((size_t)C + 127) / 128 * 128;
    return kEmaCtrBytes + (size_t)B * (lanes1 > lanes2 ? lanes1 : lanes2) * nblk * 5 * sizeof(float);
}

hipError_t ema_bidir_launch(const EmaParams &p, bool bf16, hipStream_t s) {
    const dim3 grid((unsigned)p.B * (unsigned)p.ncblk), block(64 * kEmaWaves);
    if (bf16 && p.C % 2 == 0) {
        // bf16 channel pairs: 128 channels per workgroup of twice the waves
        EmaParams q = p;
        q.ncblk = (p.C + 127) / 128;
        hipLaunchKernelGGL((ema_bidir<uint16_t, 2>), dim3((unsigned)q.B * (unsigned)q.ncblk), dim3(64 * 2 * kEmaWaves),
                           0, s, q);
    } else if (bf16)
        hipLaunchKernelGGL(ema_bidir<uint16_t>, grid, block, 0, s, p);
    else
        hipLaunchKernelGGL(ema_bidir<float>, grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace drs
