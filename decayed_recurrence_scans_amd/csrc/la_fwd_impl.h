// la_fwd_impl.h -- causal decayed linear attention, forward, gfx950.
//
// What is computed (definitions: tensortonic "cs336 linear attention duality"
// exercise for the recurrence; RetNet issue #21 for per-step decay factors,
// the decay-mask (Q K^T * D) V parallel form and reverse = flip/forward/flip;
// flash-linear-attention issue #268 for QKV/QK1 normalisation and the cached
// key sum):
//     S_t = g_t S_{t-1} + k_t v_t^T,   z_t = g_t z_{t-1} + k_t,
//     y_t = q_t^T S_t                 (or  q_t^T S_t / q_t^T z_t).
//
// Work decomposition.  One workgroup owns one (b, h, time segment); its
// DV / 16 waves own one 16-column slice of v / y / S each.  A segment is L
// chunks of C steps, walked in order.  Within a chunk, with
// b_t = sum_{r<=t} log2 g_r (chunk-local, inclusive):
//     intra:   O   = (Q K^T (.) M) V,   M[t,s] = 2^(b_t - b_s) for s <= t, else 0
//     inter:   O  += diag(2^b_t) Q S
//     state:   S  <- 2^b_last S + K^T diag(2^(b_last - b_s)) V
// Q and K tiles are staged once per chunk in LDS for the whole workgroup, the
// masked score tile is computed once (its 16x16 tiles dealt round-robin over
// the waves) and shared through LDS; every wave then runs P V, the read-out
// and the state update for its own columns, with its slice of S in registers.
//
// Segments: a workgroup with a successor first sweeps K and V of its segment
// (pass A) to form the segment's aggregate -- the decayed prefix operator
// (x_a, f_a) o (x_b, f_b) = (x_a f_b + x_b, f_a f_b) of RetNet issue #21 over
// the segment -- and publishes it.  Pass B (the outputs) starts at once: its
// first chunk computes the masked intra-chunk product and the chunk's own
// state contribution, and only then does the workgroup wait for its
// predecessors, fold their aggregates and the initial state in a fixed order
// (bitwise reproducible) into its entering state, and finish that chunk's
// read-out.  The exchange latency thus overlaps with the first chunk's work
// and with the loads of the next chunks.  Workgroup ids run segments first,
// so a workgroup waits only on lower ids, which the hardware starts first;
// the launch is sized to be resident at once.  No wait depends on that order,
// though: an aggregate that has not appeared within the wait budget (its
// workgroup not started, e.g. while other kernels hold the compute units) is
// computed by the waiting wave itself from K and V.  (An atomic start ticket
// would guarantee the order but costs a serialised device-wide atomic per
// workgroup before its first load; only the in-place final state, whose last
// segment waits for every segment to have read the initial state, takes it.)
// The exchange uses device-coherent (sc1) stores and loads, ordered by waiting
// for the stores to complete before the flag store; no cache write-back or
// invalidation is needed.
//
// Layout (MFMA 16x16 tiles; lane l = c16 + 16 g):
//   * a wave's state slice lives in the MFMA output layout: tile a, register r
//     holds S[dk = 16 a + 4 g + r][dv = dv0 + c16];
//   * dk contractions (Q K^T, Q S) take lane group g's dk values in that same
//     order (bf16: e < 4 -> 32p + 4g + e, e >= 4 -> 32p + 16 + 4g + e - 4; fp32:
//     16p + 4g + e), so S feeds the read-out MFMA with no re-layout;
//   * s contractions (P V, K^T V) take s = 16 st + 4 g + r, the rows a score-
//     tile register holds; K^T and V fragments come from LDS through the
//     gfx950 transpose read (ds_read_b64_tr_b16);
//   * outputs are computed transposed (O^T = V^T P^T + S^T Q^T): a lane owns
//     one row t and four consecutive columns (one 8-byte bf16 store per tile).
//
// Precision: the mask is applied before exponentiation (every exponent <= 0);
// the query-side decay is applied in fp32 after the MFMA; the fp32 operands of
// the state path (decayed V and S) enter the bf16 MFMA as hi + lo bf16 pairs
// (~16 mantissa bits).  fp32 inputs use the fp32 MFMA throughout.
//
// Fused bidirectional form (RetNet issue #21, the bidirectional encoder: a forward
// and a reverse scan over the same inputs, summed; one factor g per head or none,
// zero states).  Every output row takes both orders' contributions, so within a
// chunk the score mask becomes g^|t-s| with the diagonal counted once per order,
// and each workgroup reads its segment's q, k and v once:
//   * forward, as above: kept outputs, the forward aggregate;
//   * reverse, in the same sweep: chunk i's summary R_i = K^T diag(g^s) V (s local)
//     is added to the kept outputs of the segment's earlier chunks c < i with
//     g^((i - c) C - t), and to the segment's reverse aggregate with g^(i C);
//   * the reverse aggregate is exchanged like the forward one but with the later
//     segments of the unit, which carry the reverse state into the segment's last
//     row + 1; row t of the segment takes it with g^(row after the segment - t).
// A unit's segments take consecutive workgroup ids, so the segments a workgroup
// waits on in either direction start with it (the same bounded waits and
// computed-aggregate fallback apply).
#pragma once

#include <type_traits>

#include "common.h"
#include "lookback.h"

namespace drs {

typedef short v4i16 __attribute__((ext_vector_type(4)));

struct LAParams {
    const void *q, *k, *v;
    void *y;
    const float *decay;
    const float *state_in, *cum_k_in;
    float *state_out, *cum_k_out;
    unsigned *ws_ctr;               // [0] next virtual workgroup id (ticketed launches),
                                    // [1] finished workgroups, [2] epoch, [3] aggregates a
                                    // workgroup computed itself (and waits that gave up)
    unsigned long long *ws_flags;   // [B*H*NW * nseg] flag words (see flag_word)
    float *ws_agg;                  // [B*H*NW * nseg][SLOT_F] segment aggregates (+ segment decay)
    int B, H, T;
    int mode;                       // 0 none, 1 head, 2 step
    int reverse, normalize;
    int nchunks, nbh, nseg, L;
    int onepass;                    // single pass (L <= kOnePassChunks, Dk, Dv <= 64)
    int alias_state;                // state_out == state_in or cum_k_out == cum_k_in
    int y_f32;                      // bf16 inputs, y stored as fp32 (internal: gradient scans)
    int accumulate;                 // y += the result (y read before each store; not with y_f32)
    int ticket;                     // virtual ids from the atomic ticket (else the workgroup id)
    int own_aggs;                   // compute every earlier segment's aggregate instead of waiting
    unsigned spin_limit;
    unsigned tag;                   // flag tag of the counter set at ws_ctr (0 .. 3, see flag_word)
};

// Up to kMaxGroup independent problems of one shape in one launch: problem i takes
// workgroups [i * per_grid, (i + 1) * per_grid) and its own workspace; each problem's
// look-back waits only on lower ids of the same problem, which start first.
constexpr int kMaxGroup = 4;
#ifndef DRS_LA_FLAG_STRIDE
#define DRS_LA_FLAG_STRIDE 16
#endif
// Flag words per look-back slot: 16 puts each segment's flag in a 128-byte line of its
// own (about 1% faster at every linear-attention workload than packed flags, which a
// segment's successors poll while its neighbours store theirs).
constexpr int kFlagStride = DRS_LA_FLAG_STRIDE;
struct LAGroup {
    LAParams p[kMaxGroup];
    unsigned per_grid;   // workgroups per problem
    int count;
};

template <typename TI> struct InTraits;
template <> struct InTraits<float> {
    static constexpr int E = 4;      // contraction elements per lane group
    typedef f32x4 Frag;              // 4 fp32
};
template <> struct InTraits<uint16_t> {
    static constexpr int E = 8;
    typedef u32x4 Frag;              // 8 bf16 as four 32-bit words: word k = elements 2k, 2k+1
};

template <typename TI, int DK, int DV, int C, int NQ = 1>
struct FwdLayout {
    static constexpr bool BF16 = sizeof(TI) == 2;
    static constexpr int SZ = (int)sizeof(TI);
    static constexpr int E = InTraits<TI>::E;
    static constexpr int KB = 4 * E;                // dk per contraction fragment
    static constexpr int DKP = DK < KB ? KB : DK;   // dk zero-padded to a whole fragment
    static constexpr int NW = DV / 16;              // waves = 16-column slices
    static constexpr int NTH = 64 * NW;
    static constexpr int NT = C / 16;               // 16-row tiles per chunk
    static constexpr int NA = DKP / 16;             // dk tiles of a state slice
    static constexpr int NP = DKP / KB;             // dk contraction fragments
    static constexpr int NSF = BF16 ? (NT + 1) / 2 : NT;   // s contraction fragments
    // LDS tiles (row pitch in elements)
    static constexpr int QP = DKP + 4;                     // Q: fragment reads
    static constexpr int KP = DKP + (BF16 ? 16 : 4);       // K: fragment and transpose reads
    static constexpr int PP = C + 4;                       // masked scores [t][s]
    static constexpr int VP = 16 + (BF16 ? 16 : 4);        // V slice of one wave
    static constexpr int QT_B = (C * QP * SZ + 15) / 16 * 16;
    static constexpr int KT_B = (C * KP * SZ + 15) / 16 * 16;
    static constexpr int PT_B = (C * PP * SZ + 15) / 16 * 16;
    static constexpr int VT_B = (C * VP * SZ + 15) / 16 * 16;
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_K = OFF_Q + NQ * QT_B;   // NQ query tiles
    static constexpr int OFF_P = OFF_K + KT_B;
    static constexpr int OFF_V = OFF_P + PT_B;
    static constexpr int OFF_B2 = OFF_V + NW * VT_B;
    // fp32 inputs keep the per-step log2 prefix as a (high, low) pair: a second table
    static constexpr int OFF_B2L = OFF_B2 + NW * C * 4;
    static constexpr int OFF_INFO = OFF_B2L + (BF16 ? 0 : NW * C * 4);
    static constexpr int LDS_B = OFF_INFO + 16;
    // cooperative loads: 16-byte pieces of the Q / K tiles per thread, of a V slice per lane
    static constexpr int QK_PIECES_ROW = DK * SZ / 16;
    static constexpr int QK_PIECES = C * QK_PIECES_ROW;
    static constexpr int QK_PT = (QK_PIECES + NTH - 1) / NTH;
    // V is loaded in whole rows by the workgroup (coalesced) and scattered to the
    // waves' 16-column slices in LDS
    static constexpr int V_PIECES_ROW = DV * SZ / 16;
    static constexpr int V_PIECES = C * V_PIECES_ROW;
    static constexpr int V_PL = (V_PIECES + NTH - 1) / NTH;
    static constexpr int EP = 16 / SZ;                     // elements per 16-byte piece
    // exchange slot of one wave's slice: S tiles in register order [NA][64 lanes][4],
    // z [NA][4 groups][4], segment decay
    static constexpr int S_F = NA * 256;
    static constexpr int Z_F = NA * 16;
    static constexpr int SLOT_F = S_F + Z_F + 4;
    static_assert(C == 16 || C == 32 || C == 64, "chunk");
    static_assert(DK % 16 == 0 && DV % 16 == 0 && DKP % KB == 0, "dims");
};

// ----------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mma_k(const u32x4 &a, const u32x4 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k(const f32x4 &a, const f32x4 &b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}

// log2 of a factor is floored here: log2 0 = -inf would turn prefix differences into
// NaN, and 2^-256 (what a zero factor becomes) is exactly zero in fp32, so a zero
// factor still removes everything before it exactly.
constexpr float kLog2Floor = -256.f;

// Double-float arithmetic for the per-step log2 prefix of fp32 inputs.  A running
// sum of log2 factors grows to hundreds within a chunk when factors are tiny; the
// difference of two such fp32 sums would be rounded at the sums' scale (ulp(100) is
// 7.6e-6, which fails a 1e-5 bar).  As (high, low) pairs the difference is exact to
// ~2^-48 of the operands.
// (hi, lo) += (ohi, olo)
__device__ __forceinline__ void df_add(float &hi, float &lo, float ohi, float olo) {
    const float s = hi + ohi;
    const float bb = s - hi;
    const float e = (hi - (s - bb)) + (ohi - bb);   // the rounding error of hi + ohi
    const float l = lo + olo + e;
    hi = s + l;
    lo = l - (hi - s);
}
// (ah + al) - (bh + bl), rounded once
__device__ __forceinline__ float df_diff(float ah, float al, float bh, float bl) {
    const float s = ah - bh;
    const float bb = s - ah;
    const float e = (ah - (s - bb)) + (-bh - bb);   // the rounding error of ah - bh
    return s + ((al - bl) + e);
}

// A contraction fragment whose every element is 1: with it as one operand the MFMA
// sums the other operand along the contraction, the same sum in every output column.
__device__ __forceinline__ void ones_frag(u32x4 &f) { f = u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u}; }
__device__ __forceinline__ void ones_frag(f32x4 &f) { f = f32x4{1.f, 1.f, 1.f, 1.f}; }

// Transposed fragment of a row-major LDS tile: element r = tile[16 st + 4 g + r][col0 + c16].
// bf16: ds_read_b64_tr_b16 works on 16-lane blocks; output lane 4j+e gathers
// element e of source lanes j, j+4, j+8, j+12, so source lane 4m+j addresses
// row 4g+m, column 4j.
__device__ __forceinline__ u32x2 tr_frag(const uint16_t *tile, int pitch, int st, int col0, int lane) {
    const int src = lane & 15, g = lane >> 4;
    const uint16_t *pa = tile + (16 * st + 4 * g + (src >> 2)) * pitch + col0 + 4 * (src & 3);
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(pa));
    return __builtin_bit_cast(u32x2, r);
}
__device__ __forceinline__ f32x4 tr_frag(const float *tile, int pitch, int st, int col0, int lane) {
    const int c16 = lane & 15, g = lane >> 4;
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = tile[(16 * st + 4 * g + i) * pitch + col0 + c16];
    return r;
}

// dk-contraction fragment of a row-major LDS tile: row `row`; bf16 elements
// 0..3 = dk 32 pb + 4 g + 0..3, elements 4..7 = dk 32 pb + 16 + 4 g + 0..3
__device__ __forceinline__ u32x4 dk_frag(const uint16_t *tile, int pitch, int row, int pb, int g) {
    const uint16_t *pr = tile + row * pitch + 32 * pb + 4 * g;
    const u32x2 lo = *reinterpret_cast<const u32x2 *>(pr);
    const u32x2 hi = *reinterpret_cast<const u32x2 *>(pr + 16);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
}
__device__ __forceinline__ f32x4 dk_frag(const float *tile, int pitch, int row, int pb, int g) {
    return *reinterpret_cast<const f32x4 *>(tile + row * pitch + 16 * pb + 4 * g);
}

// MODE: 0 no decay, 1 one factor per head, 2 one factor per (b, h, t).
// ONEPASS: segments of at most kOnePassChunks chunks, computed in a single pass.
#ifndef DRS_LA_ONEPASS_CHUNKS
#define DRS_LA_ONEPASS_CHUNKS 4
#endif
#ifndef DRS_LA_MIN_BLOCKS_SMALL
#define DRS_LA_MIN_BLOCKS_SMALL 2     // workgroups per CU the compiler budgets registers for (Dv <= 64)
#endif
#ifndef DRS_LA_MIN_BLOCKS_LARGE
#define DRS_LA_MIN_BLOCKS_LARGE 1     // (Dv = 128)
#endif
constexpr int kOnePassChunks = DRS_LA_ONEPASS_CHUNKS;
// BIDIR: both scan orders at once (forward plus reverse, from zero states; one factor
// per head or none, no normaliser), single pass, segments of at most kBidirChunks chunks.
#ifndef DRS_LA_BIDIR_CHUNKS
#define DRS_LA_BIDIR_CHUNKS 4
#endif
constexpr int kBidirChunks = DRS_LA_BIDIR_CHUNKS;
#ifndef DRS_LA_BIDIR_STAGES
#define DRS_LA_BIDIR_STAGES 1
#endif
template <typename TI, int DK, int DV, int C, int MODE, bool NORM, bool ONEPASS, bool BIDIR = false>
__global__ __launch_bounds__(4 * DV, DV <= 64 ? DRS_LA_MIN_BLOCKS_SMALL : DRS_LA_MIN_BLOCKS_LARGE)
void la_fwd_kernel(LAGroup grp) {
    static_assert(!BIDIR || (ONEPASS && !NORM && MODE != 2), "fused bidirectional form");
    const int prob = (int)(blockIdx.x / grp.per_grid);
    const LAParams &p = grp.p[prob];
    const unsigned bid = blockIdx.x - (unsigned)prob * grp.per_grid;   // id within the problem
    constexpr int LMAX = ONEPASS ? (BIDIR ? kBidirChunks : kOnePassChunks) : 1;
    typedef FwdLayout<TI, DK, DV, C, LMAX> L;
    constexpr bool DECAY = MODE != 0;
    typedef typename InTraits<TI>::Frag Frag;
    constexpr bool BF16 = L::BF16;
    constexpr int NT = L::NT, NA = L::NA, E = L::E, NP = L::NP, NSF = L::NSF, NW = L::NW, NTH = L::NTH;

    __shared__ __attribute__((aligned(16))) char smem[L::LDS_B];
    TI *const qbase = reinterpret_cast<TI *>(smem + L::OFF_Q);
    TI *qtile = qbase;   // the query tile in use (one per kept chunk in a single pass)
    TI *ktile = reinterpret_cast<TI *>(smem + L::OFF_K);
    TI *ptile = reinterpret_cast<TI *>(smem + L::OFF_P);
    unsigned *info = reinterpret_cast<unsigned *>(smem + L::OFF_INFO);

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, c16 = lane & 15, g = lane >> 4;
    TI *vtile = reinterpret_cast<TI *>(smem + L::OFF_V + w * L::VT_B);
    float *b2tab = reinterpret_cast<float *>(smem + L::OFF_B2) + w * C;

    // ---- virtual workgroup id: the workgroup id, or the start order from the ticket
    // where the in-place final state needs every wait to be on a running workgroup
    if (tid == 0) {
        info[0] = p.ticket ? atomicAdd(p.ws_ctr + 0, 1u) : bid;
        info[1] = __hip_atomic_load(p.ws_ctr + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const unsigned vid = info[0], epoch = info[1];
    const unsigned total = (unsigned)p.nbh * (unsigned)p.nseg;

    auto finish = [&]() {   // the last workgroup to finish re-arms the workspace
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
    if (vid >= total) {   // only with a workspace whose counters were not zero before first use
        if (tid == 0) atomicAdd(p.ws_ctr + 3, 1u);
        finish();
        return;
    }

    // Segments first, so that a forward wait is on lower ids (and, with B*H a multiple
    // of 8, every segment of a unit on one XCD: workgroups are dealt to the eight XCDs
    // round-robin by id).  The bidirectional kernel, whose reverse waits are on later
    // segments, starts each unit's segments together instead: workgroup id = 8 k + x
    // takes segment k % nseg of the (k / nseg)-th unit of XCD x, so a unit's segments
    // are nseg consecutive ids of one XCD (B*H not a multiple of 8: unit-major ids).
    int seg, bh;
    if constexpr (BIDIR) {
        const unsigned ns = (unsigned)p.nseg;
        if ((p.nbh & 7) == 0) {
            const unsigned k = vid >> 3;
            seg = (int)(k % ns);
            bh = (int)((k / ns) * 8u + (vid & 7u));
        } else {
            seg = (int)(vid % ns);
            bh = (int)(vid / ns);
        }
    } else {
        seg = (int)(vid / (unsigned)p.nbh);
        bh = (int)(vid - (unsigned)seg * p.nbh);
    }
    const int h = bh % p.H;
    const int dv0 = 16 * w;
    const int T = p.T;
    const int ch0 = seg * p.L, ch1 = min(ch0 + p.L, p.nchunks);
    const bool has_pred = seg > 0, has_succ = seg < p.nseg - 1;
    const size_t unit = (size_t)bh * NW + w;
    const size_t slot = unit * p.nseg + seg;

    const TI *__restrict__ qg = static_cast<const TI *>(p.q) + (size_t)bh * T * DK;
    const TI *__restrict__ kg = static_cast<const TI *>(p.k) + (size_t)bh * T * DK;
    const TI *__restrict__ vg = static_cast<const TI *>(p.v) + (size_t)bh * T * DV + dv0;
    auto mem_row = [&](int r) { return p.reverse ? (T - 1 - r) : r; };
    // Buffer resources over this unit's rows: loads and stores at an offset past the
    // end (rows >= T, chunks past the segment) return zero / are dropped by the
    // hardware, so every path through the chunk loop issues the same memory
    // instructions and the compiler's wait counts stay exact.
    const char *unit_q = static_cast<const char *>(p.q) + (size_t)bh * T * DK * L::SZ;
    const char *unit_k = static_cast<const char *>(p.k) + (size_t)bh * T * DK * L::SZ;
    const char *unit_v = static_cast<const char *>(p.v) + (size_t)bh * T * DV * L::SZ;
    const int ysz = (BF16 && p.y_f32) ? 4 : L::SZ;   // bytes per stored output
    char *unit_y = static_cast<char *>(p.y) + (size_t)bh * T * DV * ysz;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(unit_q, T * DK * L::SZ);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(unit_k, T * DK * L::SZ);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(unit_v, T * DV * L::SZ);
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(unit_y, T * DV * ysz);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(MODE == 2 ? p.decay + (size_t)bh * T : p.q, MODE == 2 ? T * 4 : 0);

    // ---- per-head decay: the factors of a full chunk are the same for every chunk -----
    //   hfs[x][r] = g^(C-1-s)       (state update, s = 16 x + 4 g + r)
    //   het[t]    = g^(t+1)         (read-out, t = 16 tt + c16)
    //   hmf[d][r] = g^(t-s), t-s = 16 d + c16 - 4 g - r >= 0, else 0 (score mask, d = tt - st)
    //   hgc       = g^C
    // (kept in registers by the single-pass kernel without normaliser, where they fit;
    // the other variants recompute them from the per-chunk log2 table)
    constexpr bool HPRE = ONEPASS && MODE == 1 && !NORM && !BIDIR;
    // Every wave computes its own score tiles (no shared P tile in LDS, no barrier between
    // the scores and P V): in the fused bidirectional form, which needs all NT^2 tiles,
    // 43.0 against 45.9-46.4 us at bidir_retention_bf16; the causal single-direction
    // kernels, with NT (NT + 1) / 2 tiles to share, measured slower that way (29.7-30.4
    // against 26.8-27.7 us per headline scan).
    constexpr bool PRIVP = BIDIR;
    // Per-step factors of fp32 inputs: the chunk-local prefix as (high, low) pairs.
    constexpr bool PREC = MODE == 2 && !BF16;
    float *b2lo = reinterpret_cast<float *>(smem + L::OFF_B2L) + w * C;
    float hlg = 0.f, hgc = 1.f;
    f32x4 hfs[NT], hmf[NT];
    float het[NT];
    if constexpr (MODE == 1) hlg = fmaxf(log2f(p.decay[h]), kLog2Floor);
    if constexpr (HPRE) {
#pragma unroll
        for (int x = 0; x < NT; ++x) {
            het[x] = exp2_fast((float)(16 * x + c16 + 1) * hlg);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                hfs[x][r] = exp2_fast((float)(C - 1 - (16 * x + 4 * g + r)) * hlg);
                const int dd = 16 * x + c16 - 4 * g - r;
                hmf[x][r] = dd >= 0 ? exp2_fast((float)dd * hlg) : 0.f;
            }
        }
        hgc = exp2_fast((float)C * hlg);
    }

    // ---- register staging: PD chunks in flight (two where the registers allow it
    // without spilling: not with the normaliser's extra state, not at Dk = 128) ----------
    constexpr int STAGE_REGS = 4 * (2 * L::QK_PT + L::V_PL);
#ifdef DRS_LA_PD_LARGE
    constexpr int PD = (STAGE_REGS <= 32 && !NORM && DK <= 64) ? 2 : DRS_LA_PD_LARGE;
#else
    constexpr int PD = (STAGE_REGS <= 32 && !NORM && DK <= 64) ? 2 : 1;
#endif
    // Whether the first output chunk of a segment is computed before the entering
    // state is known (its read-out deferred); not where the extra live registers
    // would spill (Dk = 128).
    constexpr bool DEFER = DK <= 64;
    constexpr int KB_REGS = 64;
    struct Staged {
        u32x4 Q[L::QK_PT], K[L::QK_PT], V[L::V_PL];
        float g;
    };
    // live = false issues the same loads at an out-of-range offset (zeros, no traffic).
    auto issue_loads = [&](Staged &sg, int ch, bool with_q, bool live) {
#pragma unroll
        for (int i = 0; i < L::QK_PT; ++i) {
            const int piece = tid + NTH * i;
            const int row = piece / L::QK_PIECES_ROW, col = piece - row * L::QK_PIECES_ROW;
            const int r = ch * C + row;
            const unsigned off = (live && piece < L::QK_PIECES && r < T)
                                     ? (unsigned)(mem_row(r) * DK * L::SZ + 16 * col) : kOutOfRange;
            if (with_q) sg.Q[i] = buffer_load16(rq, off);
            sg.K[i] = buffer_load16(rk, off);
        }
#pragma unroll
        for (int i = 0; i < L::V_PL; ++i) {
            const int piece = tid + NTH * i;
            const int row = piece / L::V_PIECES_ROW, col = piece - row * L::V_PIECES_ROW;
            const int r = ch * C + row;
            const unsigned off = (live && piece < L::V_PIECES && r < T)
                                     ? (unsigned)(mem_row(r) * DV * L::SZ + 16 * col) : kOutOfRange;
            sg.V[i] = buffer_load16(rv, off);
        }
        if constexpr (MODE == 2) {
            const int r = ch * C + lane;
            sg.g = buffer_load4(rg, (live && lane < C && r < T) ? (unsigned)(mem_row(r) * 4) : kOutOfRange);
        }
    };

    // registers -> LDS tiles, chunk-local log2 decay prefix (per wave).  The caller
    // brackets this with workgroup barriers.
    auto stage = [&](const Staged &sg, int ch, bool with_q) {
#pragma unroll
        for (int i = 0; i < L::QK_PT; ++i) {
            const int piece = tid + NTH * i;
            if (piece < L::QK_PIECES) {
                const int row = piece / L::QK_PIECES_ROW, col = piece - row * L::QK_PIECES_ROW;
                const int e0 = col * (16 / L::SZ);   // first element of the piece
                if (with_q) {
                    char *dq = reinterpret_cast<char *>(qtile + row * L::QP + e0);
                    *reinterpret_cast<u32x2 *>(dq) = u32x2{sg.Q[i].x, sg.Q[i].y};
                    *reinterpret_cast<u32x2 *>(dq + 8) = u32x2{sg.Q[i].z, sg.Q[i].w};
                }
                char *dk = reinterpret_cast<char *>(ktile + row * L::KP + e0);
                *reinterpret_cast<u32x2 *>(dk) = u32x2{sg.K[i].x, sg.K[i].y};
                *reinterpret_cast<u32x2 *>(dk + 8) = u32x2{sg.K[i].z, sg.K[i].w};
            }
        }
        if constexpr (L::DKP > DK) {   // zero the dk padding of the tiles (bf16, Dk = 16)
            for (int idx = tid; idx < C * (L::DKP - DK); idx += NTH) {
                const int row = idx / (L::DKP - DK), col = DK + idx % (L::DKP - DK);
                ktile[row * L::KP + col] = TI(0);
                qtile[row * L::QP + col] = TI(0);
            }
        }
#pragma unroll
        for (int i = 0; i < L::V_PL; ++i) {
            const int piece = tid + NTH * i;
            if (piece < L::V_PIECES) {
                const int row = piece / L::V_PIECES_ROW, col = piece - row * L::V_PIECES_ROW;
                const int e = col * L::EP;   // first column of the piece: wave e / 16, offset e % 16
                TI *dst = reinterpret_cast<TI *>(smem + L::OFF_V + (e / 16) * L::VT_B) + row * L::VP + e % 16;
                *reinterpret_cast<u32x4 *>(dst) = sg.V[i];
            }
        }
        const int nvalid = min(C, T - ch * C);
        if constexpr (MODE == 1) {
            // the count of factors through row t (the log2 prefix is count * hlg, so
            // every difference is an exact integer times hlg); full chunks use the
            // factors precomputed per workgroup
            if (!(HPRE && nvalid == C) && lane < C) b2tab[lane] = (float)(min(lane, nvalid - 1) + 1);
        } else if constexpr (MODE == 2) {
            const float gr = (lane < C && ch * C + lane < T) ? sg.g : 1.f;
            float b2 = fmaxf(log2f(gr), kLog2Floor), b2l = 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(b2, off, 64);
                if constexpr (PREC) {
                    const float ol = __shfl_up(b2l, off, 64);
                    if (lane >= off) df_add(b2, b2l, o, ol);
                } else {
                    if (lane >= off) b2 += o;
                }
            }
            if (lane < C) {
                b2tab[lane] = b2;
                if constexpr (PREC) b2lo[lane] = b2l;
            }
        }
    };

    // V^T fragments of this wave's slice (element e <-> s = 16 st(e) + 4 g + r(e), dv = c16)
    auto load_vfrags = [&](Frag (&Vt)[NSF]) {
#pragma unroll
        for (int x = 0; x < NSF; ++x) {
            if constexpr (BF16) {
                const u32x2 lo = tr_frag(reinterpret_cast<const uint16_t *>(vtile), L::VP, 2 * x, 0, lane);
                u32x2 hi = {0u, 0u};
                if (2 * x + 1 < NT) hi = tr_frag(reinterpret_cast<const uint16_t *>(vtile), L::VP, 2 * x + 1, 0, lane);
                Vt[x] = u32x4{lo.x, lo.y, hi.x, hi.y};
            } else {
                Vt[x] = tr_frag(reinterpret_cast<const float *>(vtile), L::VP, x, 0, lane);
            }
        }
    };

    // From the staged prefix values of rows t >= s (b, and for fp32 per-step factors
    // the low part l): log2 of the product of the factors after s through t, and of
    // the factors through t.
    auto ldiff = [&](float bt, float lt, float bs, float ls) -> float {
        if constexpr (MODE == 1) return (bt - bs) * hlg;   // an exact count times hlg
        else if constexpr (PREC) return df_diff(bt, lt, bs, ls);
        else return bt - bs;
    };
    auto lpre = [&](float bt, float lt) -> float {
        if constexpr (MODE == 1) return bt * hlg;
        else if constexpr (PREC) return bt + lt;
        else return bt;
    };

    // S <- 2^b_last S + K^T diag(f) V, z <- 2^b_last z + K^T f, f_s = 2^(b_last - b_s);
    // returns 2^b_last.
    auto state_update = [&](const Frag (&Vt)[NSF], f32x4 (&S)[NA], f32x4 (&z)[NA], bool fast) {
        f32x4 fs[NT];
        float gc = 1.f;
        if (HPRE && fast) {
#pragma unroll
            for (int x = 0; x < NT; ++x) fs[x] = hfs[x];
            gc = hgc;
        } else if constexpr (DECAY) {
            const float b2last = b2tab[C - 1], l2last = PREC ? b2lo[C - 1] : 0.f;
#pragma unroll
            for (int x = 0; x < NT; ++x) {
                const f32x4 bs = *reinterpret_cast<const f32x4 *>(b2tab + 16 * x + 4 * g);
                f32x4 ls = {0.f, 0.f, 0.f, 0.f};
                if constexpr (PREC) ls = *reinterpret_cast<const f32x4 *>(b2lo + 16 * x + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) fs[x][r] = exp2_fast(ldiff(b2last, l2last, bs[r], ls[r]));
            }
            gc = exp2_fast(lpre(b2last, l2last));
        } else {
#pragma unroll
            for (int x = 0; x < NT; ++x) fs[x] = f32x4{1.f, 1.f, 1.f, 1.f};
        }
        // decayed V as hi + lo (exact V when there is no decay); with the normaliser also
        // the factors alone, f_s in every column, so that K^T f (the key sum's update)
        // comes out of the MFMA in the state's own layout, the same in every column
        Frag vh[NSF], vl[NSF], fh[NSF], fl[NSF];
#pragma unroll
        for (int x = 0; x < NSF; ++x) {
            if constexpr (BF16) {
                if constexpr (DECAY) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int st = 2 * x + (k >> 1), r0 = 2 * (k & 1);
                        const float f0 = st < NT ? fs[st < NT ? st : 0][r0] : 0.f;
                        const float f1 = st < NT ? fs[st < NT ? st : 0][r0 + 1] : 0.f;
                        const float a = bf16_lo(Vt[x][k]) * f0, b = bf16_hi(Vt[x][k]) * f1;
                        const unsigned hw = pack_bf16x2(a, b);
                        vh[x][k] = hw;
                        vl[x][k] = pack_bf16x2(a - bf16_lo(hw), b - bf16_hi(hw));
                        if constexpr (NORM) {
                            const unsigned fw = pack_bf16x2(f0, f1);
                            fh[x][k] = fw;
                            fl[x][k] = pack_bf16x2(f0 - bf16_lo(fw), f1 - bf16_hi(fw));
                        }
                    }
                } else {
                    vh[x] = Vt[x];
                    if constexpr (NORM) ones_frag(fh[x]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) vh[x][e] = Vt[x][e] * fs[x][e];
                if constexpr (NORM) fh[x] = fs[x];
            }
        }
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            f32x4 acc, zacc;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                acc[r] = gc * S[a][r];
                if constexpr (NORM) zacc[r] = gc * z[a][r];
            }
#pragma unroll
            for (int x = 0; x < NSF; ++x) {
                Frag ka;
                if constexpr (BF16) {
                    const u32x2 lo = tr_frag(reinterpret_cast<const uint16_t *>(ktile), L::KP, 2 * x, 16 * a, lane);
                    u32x2 hi = {0u, 0u};
                    if (2 * x + 1 < NT)
                        hi = tr_frag(reinterpret_cast<const uint16_t *>(ktile), L::KP, 2 * x + 1, 16 * a, lane);
                    ka = u32x4{lo.x, lo.y, hi.x, hi.y};
                } else {
                    ka = tr_frag(reinterpret_cast<const float *>(ktile), L::KP, x, 16 * a, lane);
                }
                acc = mma_k(ka, vh[x], acc);
                if constexpr (BF16 && DECAY) acc = mma_k(ka, vl[x], acc);
                if constexpr (NORM) {
                    zacc = mma_k(ka, fh[x], zacc);
                    if constexpr (BF16 && DECAY) zacc = mma_k(ka, fl[x], zacc);
                }
            }
            S[a] = acc;
            if constexpr (NORM) z[a] = zacc;
        }
        return gc;
    };

    // Reverse summary of the staged chunk (the fused bidirectional form):
    // Rt = K^T diag(g^s) V, s chunk-local -- what the chunk's steps add to the state a
    // reverse scan carries into the chunk's first step.
    auto rev_summary = [&](const Frag (&Vt)[NSF], f32x4 (&Rt)[NA]) {
        f32x4 fs[NT];
#pragma unroll
        for (int x = 0; x < NT; ++x)
#pragma unroll
            for (int r = 0; r < 4; ++r) fs[x][r] = DECAY ? exp2_fast((float)(16 * x + 4 * g + r) * hlg) : 1.f;
        Frag vh[NSF], vl[NSF];
#pragma unroll
        for (int x = 0; x < NSF; ++x) {
            if constexpr (BF16) {
                if constexpr (DECAY) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const int st = 2 * x + (k >> 1), r0 = 2 * (k & 1);
                        const float f0 = st < NT ? fs[st < NT ? st : 0][r0] : 0.f;
                        const float f1 = st < NT ? fs[st < NT ? st : 0][r0 + 1] : 0.f;
                        const float a = bf16_lo(Vt[x][k]) * f0, b = bf16_hi(Vt[x][k]) * f1;
                        const unsigned hw = pack_bf16x2(a, b);
                        vh[x][k] = hw;
                        vl[x][k] = pack_bf16x2(a - bf16_lo(hw), b - bf16_hi(hw));
                    }
                } else {
                    vh[x] = Vt[x];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) vh[x][e] = Vt[x][e] * fs[x][e];
            }
        }
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int x = 0; x < NSF; ++x) {
                Frag ka;
                if constexpr (BF16) {
                    const u32x2 lo = tr_frag(reinterpret_cast<const uint16_t *>(ktile), L::KP, 2 * x, 16 * a, lane);
                    u32x2 hi = {0u, 0u};
                    if (2 * x + 1 < NT)
                        hi = tr_frag(reinterpret_cast<const uint16_t *>(ktile), L::KP, 2 * x + 1, 16 * a, lane);
                    ka = u32x4{lo.x, lo.y, hi.x, hi.y};
                } else {
                    ka = tr_frag(reinterpret_cast<const float *>(ktile), L::KP, x, 16 * a, lane);
                }
                acc = mma_k(ka, vh[x], acc);
                if constexpr (BF16 && DECAY) acc = mma_k(ka, vl[x], acc);
            }
            Rt[a] = acc;
        }
    };

    f32x4 S[NA], z[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) { S[a] = f32x4{0.f, 0.f, 0.f, 0.f}; z[a] = f32x4{0.f, 0.f, 0.f, 0.f}; }

    // publish this wave's slice of the segment aggregate (S, z, decay gseg)
    auto publish = [&](float gseg) {
        float *dst = p.ws_agg + slot * L::SLOT_F;
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            float *d = dst + (a * 64 + lane) * 4;
            coherent_store2(d, S[a][0], S[a][1]);
            coherent_store2(d + 2, S[a][2], S[a][3]);
        }
        if (NORM && c16 == 0) {
#pragma unroll
            for (int a = 0; a < NA; ++a) {
                float *d = dst + L::S_F + (a * 4 + g) * 4;
                coherent_store2(d, z[a][0], z[a][1]);
                coherent_store2(d + 2, z[a][2], z[a][3]);
            }
        }
        if (lane == 0) coherent_store2(dst + L::S_F + L::Z_F, gseg, 0.f);
        wait_stores_complete();   // callers issue no load before this: only the stores are waited for
        if (lane == 0)
            __hip_atomic_store(p.ws_flags + slot * kFlagStride, flag_word(epoch, kAgg, p.tag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    // The initial state decayed by gp, added to (Sx, zx): this wave's slice.
    auto add_initial = [&](f32x4 (&Sx)[NA], f32x4 (&zx)[NA], float gp) {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int dk = 16 * a + 4 * g + r;
                if (p.state_in && dk < DK)
                    Sx[a][r] = fmaf(gp, p.state_in[((size_t)bh * DK + dk) * DV + dv0 + c16], Sx[a][r]);
                if (NORM && p.cum_k_in && dk < DK) zx[a][r] = fmaf(gp, p.cum_k_in[(size_t)bh * DK + dk], zx[a][r]);
            }
    };

    // Aggregate of segment j for this wave's slice, computed from K and V (and the
    // decay factors) directly: fp32, token by token from the segment's last row
    // back, f = the product of the factors after the token.  Returns the segment's
    // decay.  Used only when segment j's own aggregate has not appeared.
    // With rev, the reverse aggregate instead: f = the product of the factors from the
    // segment's first row through the token's predecessor (one factor per head or none).
    auto own_aggregate = [&](int j, float (&xs)[NA][4], float (&xz)[NA][4], bool rev) -> float {
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) { xs[a][r] = 0.f; xz[a][r] = 0.f; }
        const int r0 = j * p.L * C, r1 = min((j + 1) * p.L * C, T);
        double lg = 0.0;   // log2 of the product of the factors after row r (per-step factors)
        for (int r = r1 - 1; r >= r0; --r) {
            const int mr = mem_row(r);
            const float f = MODE == 1 ? exp2_fast((float)(rev ? r - r0 : r1 - 1 - r) * hlg) : exp2_fast((float)lg);
            float vv;
            if constexpr (BF16) vv = __uint_as_float((unsigned)vg[(size_t)mr * DV + c16] << 16);
            else vv = vg[(size_t)mr * DV + c16];
            const float fv = f * vv;
#pragma unroll
            for (int a = 0; a < NA; ++a) {
                if (16 * a >= DK) continue;
                float kk[4];
                const TI *src = kg + (size_t)mr * DK + 16 * a + 4 * g;
                if constexpr (BF16) {
                    const u32x2 w2 = *reinterpret_cast<const u32x2 *>(src);
                    kk[0] = bf16_lo(w2.x); kk[1] = bf16_hi(w2.x); kk[2] = bf16_lo(w2.y); kk[3] = bf16_hi(w2.y);
                } else {
                    const f32x4 w4 = *reinterpret_cast<const f32x4 *>(src);
                    kk[0] = w4[0]; kk[1] = w4[1]; kk[2] = w4[2]; kk[3] = w4[3];
                }
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    xs[a][r4] = fmaf(kk[r4], fv, xs[a][r4]);
                    if constexpr (NORM) xz[a][r4] = fmaf(kk[r4], f, xz[a][r4]);
                }
            }
            if constexpr (MODE == 2) lg += (double)fmaxf(log2f(p.decay[(size_t)bh * T + mr]), kLog2Floor);
        }
        return MODE == 1 ? exp2_fast((float)(r1 - r0) * hlg) : exp2_fast((float)lg);
    };

    // Entering state of the segment: wait for every predecessor at once (lane j
    // watches segment j), then fold their aggregates in a fixed order -- segments
    // seg-1 .. 0, then the initial state -- so the result is bitwise reproducible.
    // Segment 0 gets the initial state alone.  A wave whose wait runs out folds
    // segment by segment instead, computing each aggregate that is still missing.
    auto fold_entering = [&](f32x4 (&Sx)[NA], f32x4 (&zx)[NA]) {
#pragma unroll
        for (int a = 0; a < NA; ++a) { Sx[a] = f32x4{0.f, 0.f, 0.f, 0.f}; zx[a] = f32x4{0.f, 0.f, 0.f, 0.f}; }
        bool all_ok = !p.own_aggs;
        for (int j0 = 0; j0 < seg && all_ok; j0 += 64) {
            const int j = j0 + lane;
            bool ok = j >= seg;
            for (unsigned n = 0; n < p.spin_limit; ++n) {
                if (!ok)
                    ok = flag_state(__hip_atomic_load(p.ws_flags + (unit * p.nseg + j) * kFlagStride, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT),
                                    epoch, p.tag) >= kAgg;
                if (__all(ok)) break;
                __builtin_amdgcn_s_sleep(2);
            }
            all_ok = __all(ok);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (!all_ok) {
            float gp = 1.f;
            for (int j = seg - 1; j >= 0; --j) {
                float xs[NA][4], xz[NA][4], gj;
                // the same flag word for every lane: the branch is uniform
                const bool have = !p.own_aggs &&
                                  flag_state(__hip_atomic_load(p.ws_flags + (unit * p.nseg + j) * kFlagStride, __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT),
                                             epoch, p.tag) >= kAgg;
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                if (have) {
                    const float *src = p.ws_agg + (unit * p.nseg + j) * L::SLOT_F;
#pragma unroll
                    for (int a = 0; a < NA; ++a) {
                        const float *d = src + (a * 64 + lane) * 4;
                        coherent_load2(d, xs[a][0], xs[a][1]);
                        coherent_load2(d + 2, xs[a][2], xs[a][3]);
                        if constexpr (NORM) {
                            const float *dz = src + L::S_F + (a * 4 + g) * 4;
                            coherent_load2(dz, xz[a][0], xz[a][1]);
                            coherent_load2(dz + 2, xz[a][2], xz[a][3]);
                        }
                    }
                    float unused;
                    coherent_load2(src + L::S_F + L::Z_F, gj, unused);
                } else {
                    gj = own_aggregate(j, xs, xz, false);
                    if (lane == 0) atomicAdd(p.ws_ctr + 3, 1u);
                }
#pragma unroll
                for (int a = 0; a < NA; ++a)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        Sx[a][r] = fmaf(gp, xs[a][r], Sx[a][r]);
                        if constexpr (NORM) zx[a][r] = fmaf(gp, xz[a][r], zx[a][r]);
                    }
                gp *= gj;
            }
            add_initial(Sx, zx, gp);
            return;
        }
        // slots fetched per round trip, within ~KB_REGS registers of staging
        constexpr int kRegs = NA * 4 * (NORM ? 2 : 1);
        constexpr int kBlk = kRegs >= KB_REGS ? 1 : (KB_REGS / kRegs > 8 ? 8 : KB_REGS / kRegs);
        float gp = 1.f;
        for (int jb = seg - 1; jb >= 0; jb -= kBlk) {
            float xs[kBlk][NA][4], xz[kBlk][NA][4], gj[kBlk];
#pragma unroll
            for (int i = 0; i < kBlk; ++i) {
                const int j = jb - i;
                gj[i] = 1.f;
                if (j < 0) continue;
                const float *src = p.ws_agg + (unit * p.nseg + j) * L::SLOT_F;
#pragma unroll
                for (int a = 0; a < NA; ++a) {
                    const float *d = src + (a * 64 + lane) * 4;
                    coherent_load2(d, xs[i][a][0], xs[i][a][1]);
                    coherent_load2(d + 2, xs[i][a][2], xs[i][a][3]);
                    if constexpr (NORM) {
                        const float *dz = src + L::S_F + (a * 4 + g) * 4;
                        coherent_load2(dz, xz[i][a][0], xz[i][a][1]);
                        coherent_load2(dz + 2, xz[i][a][2], xz[i][a][3]);
                    }
                }
                float unused;
                coherent_load2(src + L::S_F + L::Z_F, gj[i], unused);
            }
#pragma unroll
            for (int i = 0; i < kBlk; ++i) {
                if (jb - i < 0) continue;
#pragma unroll
                for (int a = 0; a < NA; ++a)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        Sx[a][r] = fmaf(gp, xs[i][a][r], Sx[a][r]);
                        if constexpr (NORM) zx[a][r] = fmaf(gp, xz[i][a][r], zx[a][r]);
                    }
                gp *= gj[i];
            }
        }
        add_initial(Sx, zx, gp);
    };

    // ---- the fused bidirectional form's reverse exchange: a second set of flags and
    // slots after the forward ones; segment j's reverse aggregate is the state a
    // reverse scan carries into its first row from its own rows alone, with the
    // segment's decay.  Published by every segment with a predecessor.
    const size_t nslots = (size_t)p.nbh * NW * p.nseg;
    unsigned long long *const flags_r = p.ws_flags + nslots * kFlagStride;
    float *const agg_r = p.ws_agg + nslots * L::SLOT_F;
    auto publish_rev = [&](const f32x4 (&X)[NA], float gseg) {
        float *dst = agg_r + slot * L::SLOT_F;
#pragma unroll
        for (int a = 0; a < NA; ++a) {
            float *d = dst + (a * 64 + lane) * 4;
            coherent_store2(d, X[a][0], X[a][1]);
            coherent_store2(d + 2, X[a][2], X[a][3]);
        }
        if (lane == 0) coherent_store2(dst + L::S_F + L::Z_F, gseg, 0.f);
        wait_stores_complete();
        if (lane == 0)
            __hip_atomic_store(flags_r + slot * kFlagStride, flag_word(epoch, kAgg, p.tag), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    };
    // State a reverse scan carries into the row after this segment: every later
    // segment's reverse aggregate, folded in a fixed order (seg + 1 first), each
    // decayed by the segments between.  Waits as fold_entering does, on later ids.
    auto fold_reverse = [&](f32x4 (&Sx)[NA]) {
#pragma unroll
        for (int a = 0; a < NA; ++a) Sx[a] = f32x4{0.f, 0.f, 0.f, 0.f};
        bool all_ok = !p.own_aggs;
        for (int j0 = seg + 1; j0 < p.nseg && all_ok; j0 += 64) {
            const int j = j0 + lane;
            bool ok = j >= p.nseg;
            for (unsigned n = 0; n < p.spin_limit; ++n) {
                if (!ok)
                    ok = flag_state(__hip_atomic_load(flags_r + (unit * p.nseg + j) * kFlagStride, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT),
                                    epoch, p.tag) >= kAgg;
                if (__all(ok)) break;
                __builtin_amdgcn_s_sleep(2);
            }
            all_ok = __all(ok);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        float gp = 1.f;
        if (!all_ok) {
            for (int j = seg + 1; j < p.nseg; ++j) {
                float xs[NA][4], xz[NA][4], gj;
                const bool have = !p.own_aggs &&
                                  flag_state(__hip_atomic_load(flags_r + (unit * p.nseg + j) * kFlagStride,
                                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                             epoch, p.tag) >= kAgg;
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                if (have) {
                    const float *src = agg_r + (unit * p.nseg + j) * L::SLOT_F;
#pragma unroll
                    for (int a = 0; a < NA; ++a) {
                        const float *d = src + (a * 64 + lane) * 4;
                        coherent_load2(d, xs[a][0], xs[a][1]);
                        coherent_load2(d + 2, xs[a][2], xs[a][3]);
                    }
                    float unused;
                    coherent_load2(src + L::S_F + L::Z_F, gj, unused);
                } else {
                    gj = own_aggregate(j, xs, xz, true);
                    if (lane == 0) atomicAdd(p.ws_ctr + 3, 1u);
                }
#pragma unroll
                for (int a = 0; a < NA; ++a)
#pragma unroll
                    for (int r = 0; r < 4; ++r) Sx[a][r] = fmaf(gp, xs[a][r], Sx[a][r]);
                gp *= gj;
            }
            return;
        }
        constexpr int kBlk = NA * 4 >= KB_REGS ? 1 : (KB_REGS / (NA * 4) > 8 ? 8 : KB_REGS / (NA * 4));
        for (int jb = seg + 1; jb < p.nseg; jb += kBlk) {
            float xs[kBlk][NA][4], gj[kBlk];
#pragma unroll
            for (int i = 0; i < kBlk; ++i) {
                const int j = jb + i;
                gj[i] = 1.f;
                if (j >= p.nseg) continue;
                const float *src = agg_r + (unit * p.nseg + j) * L::SLOT_F;
#pragma unroll
                for (int a = 0; a < NA; ++a) {
                    const float *d = src + (a * 64 + lane) * 4;
                    coherent_load2(d, xs[i][a][0], xs[i][a][1]);
                    coherent_load2(d + 2, xs[i][a][2], xs[i][a][3]);
                }
                float unused;
                coherent_load2(src + L::S_F + L::Z_F, gj[i], unused);
            }
#pragma unroll
            for (int i = 0; i < kBlk; ++i) {
                if (jb + i >= p.nseg) continue;
#pragma unroll
                for (int a = 0; a < NA; ++a)
#pragma unroll
                    for (int r = 0; r < 4; ++r) Sx[a][r] = fmaf(gp, xs[i][a][r], Sx[a][r]);
                gp *= gj[i];
            }
        }
    };

    // In-place final state: a segment with a successor reports that it has read the
    // initial state; the last segment waits for all of them before overwriting it.
    auto mark_folded = [&]() {
        if (p.alias_state && has_succ) {
            wait_stores_complete();   // the initial-state loads have completed
            if (lane == 0)
                __hip_atomic_store(p.ws_flags + slot * kFlagStride, flag_word(epoch, kFolded, p.tag), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    // Every wave of every earlier segment has read the initial state and key sum (each
    // wave reads the whole key sum; wave 0 writes it).  Returns false if the wait ran
    // out (never expected: the ids come from the start ticket), which is counted; the
    // caller then leaves the initial state as it is rather than overwrite it early.
    auto wait_all_folded = [&]() -> bool {
        bool all_ok = true;
        for (int i0 = 0; i0 < seg * NW; i0 += 64) {
            const int i = i0 + lane, j = i / NW, wj = i - j * NW;
            bool ok = i >= seg * NW;
            for (unsigned n = 0; n < p.spin_limit; ++n) {
                if (!ok)
                    ok = flag_state(__hip_atomic_load(p.ws_flags + (((size_t)bh * NW + wj) * p.nseg + j) * kFlagStride,
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                                    epoch, p.tag) == kFolded;
                if (__all(ok)) break;
                __builtin_amdgcn_s_sleep(2);
            }
            if (!__all(ok)) all_ok = false;
        }
        if (!all_ok && lane == 0) atomicAdd(p.ws_ctr + 3, 1u);
        return all_ok;
    };

    // ---- intra-chunk part of a staged chunk: masked, decayed score tiles (dealt
    // round-robin over the waves, shared through LDS), O^T = V^T P^T, the row sums of
    // P (normaliser, complete in every lane) and the query-side factors et = 2^b_t -----
    auto intra = [&](bool fast, Frag (&Vt)[NSF], f32x4 (&OT)[NT], float (&den)[NT], float (&et)[NT]) {
        float b2t[NT], l2t[NT];
        f32x4 b2s[NT], l2s[NT];
        if (DECAY && !fast) {
#pragma unroll
            for (int x = 0; x < NT; ++x) {
                b2t[x] = b2tab[16 * x + c16];
                b2s[x] = *reinterpret_cast<const f32x4 *>(b2tab + 16 * x + 4 * g);
                l2t[x] = 0.f;
                l2s[x] = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (PREC) {
                    l2t[x] = b2lo[16 * x + c16];
                    l2s[x] = *reinterpret_cast<const f32x4 *>(b2lo + 16 * x + 4 * g);
                }
            }
        }
        if constexpr (PRIVP) {
            // Every wave computes the score tiles it needs itself: the score MFMA leaves
            // lane (c16, g) holding P[16 tt + c16][16 st + 4 g + r], which is that lane's
            // share of the P V operand, so P goes from registers to the next MFMA with no
            // LDS tile and no barrier (the same values, masks and rounding as the shared
            // tile below).
            load_vfrags(Vt);
            Frag ones;
            ones_frag(ones);
            constexpr int SPF = BF16 ? 2 : 1;   // score tiles per P V fragment
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                OT[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
                f32x4 rs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int x = 0; x < NSF; ++x) {
                    const int st0 = SPF * x;
                    if (!BIDIR && st0 > tt) break;
                    f32x4 sc[SPF];
#pragma unroll
                    for (int h = 0; h < SPF; ++h) {
                        const int st = st0 + h;
                        sc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if (st < NT && (BIDIR || st <= tt)) {
#pragma unroll
                            for (int pb = 0; pb < NP; ++pb)
                                sc[h] = mma_k(dk_frag(ktile, L::KP, 16 * st + c16, pb, g),
                                              dk_frag(qtile, L::QP, 16 * tt + c16, pb, g), sc[h]);
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                if constexpr (BIDIR) {
                                    const int d = 16 * (tt - st) + c16 - 4 * g - r;
                                    sc[h][r] *= exp2_fast((float)(d < 0 ? -d : d) * hlg) + (d == 0 ? 1.f : 0.f);
                                } else if (st == tt && 4 * g + r > c16) {
                                    sc[h][r] = 0.f;
                                } else if constexpr (DECAY) {
                                    sc[h][r] *= (HPRE && fast) ? hmf[tt - st][r]
                                                               : exp2_fast(ldiff(b2t[tt], l2t[tt], b2s[st][r], l2s[st][r]));
                                }
                            }
                        }
                    }
                    Frag pf;
                    if constexpr (BF16) {
                        pf = u32x4{pack_bf16x2(sc[0][0], sc[0][1]), pack_bf16x2(sc[0][2], sc[0][3]),
                                   pack_bf16x2(sc[SPF - 1][0], sc[SPF - 1][1]), pack_bf16x2(sc[SPF - 1][2], sc[SPF - 1][3])};
                    } else {
                        pf = sc[0];
                    }
                    if constexpr (NORM) rs = mma_k(ones, pf, rs);
                    OT[tt] = mma_k(Vt[x], pf, OT[tt]);
                }
                den[tt] = rs[0];
            }
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                if (HPRE && fast) et[tt] = het[tt];
                else if constexpr (DECAY) et[tt] = exp2_fast(lpre(b2t[tt], l2t[tt]));
                else et[tt] = 1.f;
            }
            return;
        }
        auto score_tiles = [&](auto mfac) {
            int i = 0;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int st = 0; st < (BIDIR ? NT : tt + 1); ++st, ++i) {
                    if (i % NW != w) continue;
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int pb = 0; pb < NP; ++pb)
                        acc = mma_k(dk_frag(ktile, L::KP, 16 * st + c16, pb, g),
                                    dk_frag(qtile, L::QP, 16 * tt + c16, pb, g), acc);
                    // lane holds t = 16 tt + c16, s = 16 st + 4 g + r
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if constexpr (BIDIR) {
                            // both orders: g^|t - s|, and the diagonal once for each
                            const int d = 16 * (tt - st) + c16 - 4 * g - r;
                            acc[r] *= exp2_fast((float)(d < 0 ? -d : d) * hlg) + (d == 0 ? 1.f : 0.f);
                        } else if (st == tt && 4 * g + r > c16) {
                            acc[r] = 0.f;
                        } else if constexpr (DECAY) {
                            acc[r] *= mfac(tt, st, r);
                        }
                    }
                    TI *dst = ptile + (16 * tt + c16) * L::PP + 16 * st + 4 * g;
                    if constexpr (BF16) {
                        *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
                    } else {
                        *reinterpret_cast<f32x4 *>(dst) = acc;
                    }
                }
        };
        if (HPRE && fast)
            score_tiles([&](int tt, int st, int r) { return hmf[tt - st][r]; });
        else
            score_tiles([&](int tt, int st, int r) {
                return exp2_fast(ldiff(b2t[tt], l2t[tt], b2s[st][r], l2s[st][r]));
            });
        load_vfrags(Vt);
        __syncthreads();   // score tile complete

        Frag ones;
        ones_frag(ones);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            OT[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 rs = {0.f, 0.f, 0.f, 0.f};   // row sums of P (normaliser), in every register
#pragma unroll
            for (int x = 0; x < NSF; ++x) {
                const int st0 = BF16 ? 2 * x : x;
                if (!BIDIR && st0 > tt) break;
                const TI *prow = ptile + (16 * tt + c16) * L::PP + 4 * g;
                Frag pf;
                if constexpr (BF16) {
                    const u32x2 lo = *reinterpret_cast<const u32x2 *>(prow + 16 * st0);
                    u32x2 hi = {0u, 0u};
                    if (st0 + 1 <= (BIDIR ? NT - 1 : tt)) hi = *reinterpret_cast<const u32x2 *>(prow + 16 * (st0 + 1));
                    pf = u32x4{lo.x, lo.y, hi.x, hi.y};
                } else {
                    pf = *reinterpret_cast<const f32x4 *>(prow + 16 * st0);
                }
                if constexpr (NORM) rs = mma_k(ones, pf, rs);
                OT[tt] = mma_k(Vt[x], pf, OT[tt]);
            }
            den[tt] = rs[0];
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
            if (HPRE && fast) et[tt] = het[tt];
            else if constexpr (DECAY) et[tt] = exp2_fast(lpre(b2t[tt], l2t[tt]));
            else et[tt] = 1.f;
        }
    };

    // ---- read-out of the staged chunk's queries from a state (Sx, zx): for each
    // 16-row tile tt, use(tt, ox = S^T Q^T tile, dx = q . z) --------------------------
    // S (and z, the same in every column) enter the bf16 MFMA as hi + lo pairs.
    auto split_frag = [&](const f32x4 (&X)[NA], int pb, Frag &hi, Frag &lo) {
        if constexpr (BF16) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int a = 2 * pb + (k >> 1), r0 = 2 * (k & 1);
                const float s0 = X[a][r0], s1 = X[a][r0 + 1];
                const unsigned hw = pack_bf16x2(s0, s1);
                hi[k] = hw;
                lo[k] = pack_bf16x2(s0 - bf16_lo(hw), s1 - bf16_hi(hw));
            }
        } else {
            hi = X[pb];
        }
    };
    auto readout = [&](const f32x4 (&Sx)[NA], const f32x4 (&zx)[NA], auto use) {
        if constexpr (!NORM) {
            Frag shi[NP], slo[NP];
#pragma unroll
            for (int pb = 0; pb < NP; ++pb) split_frag(Sx, pb, shi[pb], slo[pb]);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                f32x4 ox = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int pb = 0; pb < NP; ++pb) {
                    const Frag qf = dk_frag(qtile, L::QP, 16 * tt + c16, pb, g);
                    ox = mma_k(shi[pb], qf, ox);
                    if constexpr (BF16) ox = mma_k(slo[pb], qf, ox);
                }
                use(tt, ox, 0.f);
            }
        } else {
            // fragment by fragment, every tile's sums kept (fewer live registers than
            // the four split operands of every fragment)
            f32x4 ox[NT], dx[NT];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) { ox[tt] = f32x4{0.f, 0.f, 0.f, 0.f}; dx[tt] = ox[tt]; }
#pragma unroll
            for (int pb = 0; pb < NP; ++pb) {
                Frag shi, slo, zhi, zlo;
                split_frag(Sx, pb, shi, slo);
                split_frag(zx, pb, zhi, zlo);
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) {
                    const Frag qf = dk_frag(qtile, L::QP, 16 * tt + c16, pb, g);
                    ox[tt] = mma_k(shi, qf, ox[tt]);
                    dx[tt] = mma_k(zhi, qf, dx[tt]);
                    if constexpr (BF16) {
                        ox[tt] = mma_k(slo, qf, ox[tt]);
                        dx[tt] = mma_k(zlo, qf, dx[tt]);
                    }
                }
            }
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) use(tt, ox[tt], dx[tt][0]);
        }
    };

    // cast and store four consecutive outputs of row 16 tt + c16 of chunk ch (added in
    // fp32 to the values y holds, rounded once, when accumulating)
    auto store_out = [&](int ch, int tt, const f32x4 &o) {
        const int row = ch * C + 16 * tt + c16;
        const unsigned off = row < T ? (unsigned)((mem_row(row) * DV + dv0 + 4 * g) * ysz) : kOutOfRange;
        if constexpr (BF16) {
            if (p.y_f32) {
                buffer_store16(ry, off, __builtin_bit_cast(u32x4, o));
            } else {
                f32x4 sum = o;
                if (p.accumulate) {
                    const u32x2 was = buffer_load8(ry, off);
                    sum[0] += bf16_lo(was.x); sum[1] += bf16_hi(was.x);
                    sum[2] += bf16_lo(was.y); sum[3] += bf16_hi(was.y);
                }
                buffer_store8(ry, off, u32x2{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])});
            }
        } else {
            f32x4 sum = o;
            if (p.accumulate) sum += __builtin_bit_cast(f32x4, buffer_load16(ry, off));
            buffer_store16(ry, off, __builtin_bit_cast(u32x4, sum));
        }
    };

    if constexpr (ONEPASS) {
        // ======================= single pass (segments of at most LMAX chunks) ===========
        // Every segment runs its chunks from a zero state, keeping each chunk's outputs
        // (fp32, before the entering state's contribution) in registers and its Q tile
        // in LDS; then it publishes its aggregate, folds its entering state and adds
        // 2^B_t q_t^T S_in (B_t: log2 decay from the segment start through t) to the
        // kept outputs before storing them.
        // Two chunks of loads are in flight; every step issues its loads (out of range
        // past the segment), so the memory-operation order is the same on all paths.
        f32x4 ho[LMAX][NT];
        float hf[LMAX][NT], hd[LMAX][NT];
        f32x4 Rs[NA];   // fused bidirectional form: the segment's reverse aggregate
#pragma unroll
        for (int a = 0; a < NA; ++a) Rs[a] = f32x4{0.f, 0.f, 0.f, 0.f};
        // (the fused bidirectional form keeps one chunk in flight: its extra live
        // registers leave no room for a second staging buffer without spilling)
        constexpr int NB = BIDIR ? DRS_LA_BIDIR_STAGES : 2;
        Staged sbuf[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) issue_loads(sbuf[b], ch0 + b, true, b == 0 || ch0 + b < ch1);
        float gprev = 1.f;
#pragma unroll
        for (int i = 0; i < LMAX; ++i) {
            const int ch = ch0 + i;
            Staged &sg = sbuf[i % NB];
            if (ch < ch1) {
                qtile = qbase + i * (L::QT_B / L::SZ);
                __syncthreads();   // the previous chunk's tile reads are complete
                stage(sg, ch, true);
                __syncthreads();
            }
            issue_loads(sg, ch + NB, true, ch + NB < ch1);
            if (ch < ch1) {
                const bool fast = HPRE && ch * C + C <= T;
                Frag Vt[NSF];
                f32x4 OT[NT];
                float den[NT], et[NT];
                intra(fast, Vt, OT, den, et);
                if (i == 0) {
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt) {
                        ho[i][tt] = OT[tt];
                        hd[i][tt] = NORM ? den[tt] : 1.f;
                        if constexpr (!BIDIR) hf[i][tt] = et[tt];
                    }
                } else {
                    readout(S, z, [&](int tt, const f32x4 &ox, float dx) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) ho[i][tt][r] = fmaf(et[tt], ox[r], OT[tt][r]);
                        hd[i][tt] = NORM ? fmaf(et[tt], dx, den[tt]) : 1.f;
                        if constexpr (!BIDIR) hf[i][tt] = gprev * et[tt];
                    });
                }
                if constexpr (BIDIR) {
                    // the reverse order: this chunk's summary joins the segment's reverse
                    // aggregate and reaches the kept outputs of the segment's earlier chunks
                    // (row t of chunk c takes g^((i - c) C - t))
                    f32x4 Rt[NA];
                    rev_summary(Vt, Rt);
                    const float gi = exp2_fast((float)(i * C) * hlg);
#pragma unroll
                    for (int a = 0; a < NA; ++a)
#pragma unroll
                        for (int r = 0; r < 4; ++r) Rs[a][r] = fmaf(gi, Rt[a][r], Rs[a][r]);
#pragma unroll
                    for (int c = 0; c < LMAX; ++c) {
                        if (c < i) {
                            qtile = qbase + c * (L::QT_B / L::SZ);
                            readout(Rt, Rt, [&](int tt, const f32x4 &ox, float) {
                                const float wr = exp2_fast((float)((i - c) * C - 16 * tt - c16) * hlg);
#pragma unroll
                                for (int r = 0; r < 4; ++r) ho[c][tt][r] = fmaf(wr, ox[r], ho[c][tt][r]);
                            });
                        }
                    }
                    qtile = qbase + i * (L::QT_B / L::SZ);
                }
                gprev *= state_update(Vt, S, z, fast);
            }
        }
        if (has_succ) publish(gprev);
        if constexpr (BIDIR) {
            if (has_pred) publish_rev(Rs, gprev);
        }
        f32x4 Sin[NA], zin[NA], Srv[NA];
        fold_entering(Sin, zin);
        if constexpr (BIDIR) fold_reverse(Srv);
        mark_folded();
#pragma unroll
        for (int i = 0; i < LMAX; ++i) {
            const int ch = ch0 + i;
            if (ch < ch1) {
                qtile = qbase + i * (L::QT_B / L::SZ);
                if constexpr (BIDIR) {
                    // the reverse state entering from the later segments (at row ch1 C)
                    readout(Srv, Srv, [&](int tt, const f32x4 &ox, float) {
                        const float wr = exp2_fast((float)((ch1 - ch) * C - 16 * tt - c16) * hlg);
#pragma unroll
                        for (int r = 0; r < 4; ++r) ho[i][tt][r] = fmaf(wr, ox[r], ho[i][tt][r]);
                    });
                }
                readout(Sin, zin, [&](int tt, const f32x4 &ox, float dx) {
                    // the entering state's factor at row t: the factors from the segment
                    // start through t (the fused bidirectional form recomputes it: every
                    // chunk before t's in the segment is full)
                    const float ef = BIDIR ? exp2_fast((float)(i * C + 16 * tt + c16 + 1) * hlg) : hf[i][tt];
                    const float inv = NORM ? 1.f / fmaf(ef, dx, hd[i][tt]) : 1.f;
                    f32x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = fmaf(ef, ox[r], ho[i][tt][r]) * inv;
                    store_out(ch, tt, o);
                });
            }
        }
        // state after the segment
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                S[a][r] = fmaf(gprev, Sin[a][r], S[a][r]);
                if constexpr (NORM) z[a][r] = fmaf(gprev, zin[a][r], z[a][r]);
            }
    } else {
        // ======================= pass A: segment aggregate ===============================
        float gseg = 1.f;
        Staged sa, sb;
        if (has_succ) {
            auto stepA = [&](Staged &sg, int ch) {
                __syncthreads();   // the previous chunk's tile reads are complete
                stage(sg, ch, false);
                __syncthreads();
                issue_loads(sg, ch + PD, false, ch + PD < ch1);
                Frag Vt[NSF];
                load_vfrags(Vt);
                gseg *= state_update(Vt, S, z, HPRE && ch * C + C <= T);
            };
            issue_loads(sa, ch0, false, true);
            if (PD == 2) issue_loads(sb, ch0 + 1, false, ch0 + 1 < ch1);
            int ch = ch0;
            if constexpr (PD == 2) {
                for (; ch + 1 < ch1; ch += 2) {
                    stepA(sa, ch);
                    stepA(sb, ch + 1);
                }
            }
            for (; ch < ch1; ++ch) stepA(sa, ch);
            publish(gseg);
        }
        // the first chunks of pass B are in flight during the exchange
        issue_loads(sa, ch0, true, true);
        if (PD == 2) issue_loads(sb, ch0 + 1, true, ch0 + 1 < ch1);

        // ======================= pass B: outputs =========================================
        // Segment 0 starts from the initial state; later segments start from zero and
        // learn their entering state inside their first chunk.
#pragma unroll
        for (int a = 0; a < NA; ++a) { S[a] = f32x4{0.f, 0.f, 0.f, 0.f}; z[a] = f32x4{0.f, 0.f, 0.f, 0.f}; }
        if (!has_pred) {
            add_initial(S, z, 1.f);
            mark_folded();
        }

        // deferred: the first chunk of a segment with predecessors (see below)
        auto stepB = [&](Staged &sg, int ch, auto deferred) {
            __syncthreads();   // the previous chunk's tile reads are complete
            stage(sg, ch, true);
            __syncthreads();
            issue_loads(sg, ch + PD, true, ch + PD < ch1);
            const bool fast = HPRE && ch * C + C <= T;
            Frag Vt[NSF];
            f32x4 OT[NT];
            float den[NT], et[NT];
            intra(fast, Vt, OT, den, et);
            auto out = [&](const f32x4 (&Sx)[NA], const f32x4 (&zx)[NA]) {
                readout(Sx, zx, [&](int tt, const f32x4 &ox, float dx) {
                    const float inv = NORM ? 1.f / fmaf(et[tt], dx, den[tt]) : 1.f;
                    f32x4 o;
#pragma unroll
                    for (int r = 0; r < 4; ++r) o[r] = fmaf(et[tt], ox[r], OT[tt][r]) * inv;
                    store_out(ch, tt, o);
                });
            };
            if constexpr (decltype(deferred)::value) {
                // first chunk of a segment with predecessors: S, z are still zero, so the
                // update leaves this chunk's own contribution; the entering state is folded
                // in only now, while the next chunks' loads are in flight
                const float gc = state_update(Vt, S, z, fast);
                f32x4 Sin[NA], zin[NA];
                fold_entering(Sin, zin);
                mark_folded();
                out(Sin, zin);
#pragma unroll
                for (int a = 0; a < NA; ++a)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        S[a][r] = fmaf(gc, Sin[a][r], S[a][r]);
                        if constexpr (NORM) z[a][r] = fmaf(gc, zin[a][r], z[a][r]);
                    }
            } else {
                out(S, z);
                state_update(Vt, S, z, fast);
            }
        };
        typedef std::integral_constant<bool, true> Deferred;
        typedef std::integral_constant<bool, false> Direct;
        // The staging buffers alternate chunk by chunk; each loop body covers one full
        // alternation, so the compiler sees the same memory-operation order on every
        // path into the loop.
        if (has_pred) {
            if constexpr (DEFER) {
                stepB(sa, ch0, Deferred());
            } else {
                f32x4 Sin[NA], zin[NA];
                fold_entering(Sin, zin);
                mark_folded();
#pragma unroll
                for (int a = 0; a < NA; ++a) { S[a] = Sin[a]; z[a] = zin[a]; }
                stepB(sa, ch0, Direct());
            }
            if constexpr (PD == 2) {
                int ch = ch0 + 1;
                for (; ch + 1 < ch1; ch += 2) {
                    stepB(sb, ch, Direct());
                    stepB(sa, ch + 1, Direct());
                }
                if (ch < ch1) stepB(sb, ch, Direct());
            } else {
                for (int ch = ch0 + 1; ch < ch1; ++ch) stepB(sa, ch, Direct());
            }
        } else {
            if constexpr (PD == 2) {
                int ch = ch0;
                for (; ch + 1 < ch1; ch += 2) {
                    stepB(sa, ch, Direct());
                    stepB(sb, ch + 1, Direct());
                }
                if (ch < ch1) stepB(sa, ch, Direct());
            } else {
                for (int ch = ch0; ch < ch1; ++ch) stepB(sa, ch, Direct());
            }
        }
    }

    // ---- final state (last segment) ---------------------------------------------------
    if (!has_succ) {
        bool write = true;
        if (p.alias_state) {
            write = wait_all_folded();
            __syncthreads();   // and every wave of this workgroup has used the initial key sum
            if (tid == 0) info[2] = 1u;
            __syncthreads();
            if (!write) info[2] = 0u;   // any wave that gave up stops every wave's overwrite
            __syncthreads();
            write = info[2] != 0u;
        }
        if (p.state_out && write) {
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int dk = 16 * a + 4 * g + r;
                    if (dk < DK) p.state_out[((size_t)bh * DK + dk) * DV + dv0 + c16] = S[a][r];
                }
        }
        if (NORM && p.cum_k_out && write && w == 0 && c16 == 0) {
#pragma unroll
            for (int a = 0; a < NA; ++a)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int dk = 16 * a + 4 * g + r;
                    if (dk < DK) p.cum_k_out[(size_t)bh * DK + dk] = z[a][r];
                }
        }
    }
    finish();
}

}  // namespace drs
