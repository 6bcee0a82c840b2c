/*
 * drs.h -- C ABI of libdrs: decayed recurrence scans on AMD Instinct MI355X (gfx950).
 *
 * Three forward operations (inference / training forward pass), the
 * bidirectional sums of two of them, and the backwards of linear attention and
 * WKV:
 *
 *   la_forward   causal decayed linear attention
 *                  S_t = g_t * S_{t-1} + k_t v_t^T,   y_t = q_t^T S_t
 *                with an optional normaliser  y_t = q_t^T S_t / q_t^T z_t,
 *                z_t = g_t * z_{t-1} + k_t, and an optional reversed time order.
 *   wkv_forward  the RWKV-4 WKV channel-wise recurrence, evaluated in the
 *                max-shifted (log-scale) form.
 *   ema_forward  the gated element-wise EMA  y_t = f_t * y_{t-1} + x_t.
 *   la_bidirectional, ema_bidirectional
 *                the forward and the reverse call summed (a bidirectional
 *                encoder built from the two directions).
 *   la_backward  gradients of la_forward (every mode, normalised or not).
 *   wkv_backward gradients of wkv_forward.
 *
 * Sources of the definitions (titles of the pages they are taken from):
 *   - tensortonic exercise "cs336 linear attention duality": the plain
 *     recurrence, zero initial state, current token included, shapes
 *     (B, S, Dk|Dv) and final state (B, Dk, Dv), output dtype = q's dtype.
 *   - RetNet issue #21 "removing the O(T^2) training cost": per-step decay
 *     factors of the same shape as the values, the cumulative EMA whose factor
 *     at step i multiplies the output of step i-1, the reverse flag defined as
 *     flip / forward / flip, the retention example with one scalar decay, and
 *     the factors-and-values variant used by ema_forward.
 *   - flash-linear-attention issue #268 "fused_recurrent ... normalization":
 *     the QKV / QK1 normalised form, the carried KV state, and the cached key
 *     sum ("cum_k", shape [B,H,1,D]) added to the running sum of new keys.
 *   - RWKV-LM issue #167 "formula 14 and code implementation": the att_seq
 *     WKV loop with state (aa, bb, pp), t_first (u) and t_decay (w).
 *   - RWKV-LM discussion #189 "Numerically stable parallel cumsum-based WKV":
 *     the exponentially weighted (value, log-scale) pairs and the associative
 *     scan over time used by the time-parallel WKV path.
 *
 * Ownership and execution (all entry points):
 *   - Every array pointer is a caller-owned DEVICE pointer to contiguous,
 *     row-major memory on the current HIP device.  The library keeps no
 *     pointer after return and allocates nothing; it is stateless and
 *     reentrant.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and the call returns without synchronising.  Device-side faults surface
 *     at the caller's next synchronisation.
 *   - Arguments are validated before anything is enqueued: a non-zero return
 *     means nothing was launched and no output was written.
 *   - No C++ exception crosses this boundary.
 */
#ifndef DRS_H_
#define DRS_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DRS_API __attribute__((visibility("default")))

/* Return codes. */
typedef enum drs_status {
    DRS_OK = 0,
    DRS_ERR_INVALID = 1,      /* bad pointer / size / flag combination        */
    DRS_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement  */
    DRS_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required    */
    DRS_ERR_DEVICE = 4,       /* a HIP launch or device query failed           */
    DRS_ERR_SCRATCH = 5       /* la_forward_noalloc: the call needs more scratch than
                                 the library's static buffer holds              */
} drs_status;

/* The entry points take `dt` and `mode` as plain ints holding these values, so
 * that a caller's out-of-range value is an argument error (DRS_ERR_INVALID)
 * rather than an invalid enum value. */

/* Storage type of q, k, v and y for la_forward. */
typedef enum drs_dtype {
    DRS_F32 = 0,   /* IEEE binary32                                              */
    DRS_BF16 = 1   /* bfloat16; arithmetic accumulates in fp32, y rounds to nearest even */
} drs_dtype;

/* How the decay factor g_t of la_forward is given. */
typedef enum drs_decay {
    DRS_DECAY_NONE = 0,  /* g_t = 1 (plain cumulative sum); decay must be NULL          */
    DRS_DECAY_HEAD = 1,  /* one factor per head: decay is fp32 [H]                       */
    DRS_DECAY_STEP = 2,  /* one factor per (b, h, t): decay is fp32 [B,H,T]              */
    DRS_DECAY_ELEM = 3   /* one factor per (b, h, t, key channel): fp32 [B,H,T,Dk]; row i
                            of the state (and entry i of z) decays by decay[b,h,t,i]      */
} drs_decay;

/* Flag bits. */
#define DRS_REVERSE    0x1u    /* la: visit t = T-1 .. 0 (flip, forward, flip)              */
#define DRS_NORMALIZE  0x2u    /* la: divide by q_t^T z_t (carried key sum)                */
#define DRS_FORCE_SEQ  0x100u  /* wkv: force the one-lane-per-channel sequential kernel    */
#define DRS_FORCE_SCAN 0x200u  /* wkv: force the two-pass time-parallel segment scan       */
#define DRS_FORCE_CHAIN 0x400u /* wkv: force the chained single-pass time-parallel kernel  */
#define DRS_FORCE_RECURRENT 0x800u /* la: force the step-by-step kernel (state in registers) */
#define DRS_FORCE_CHUNKED 0x1000u  /* la: force the chunked kernels                         */
#define DRS_LA_OWN_AGGREGATES 0x2000u /* la chunked: compute earlier segments' aggregates, no waits */
#define DRS_WKV_OWN_AGGREGATES 0x4000u /* wkv chained: compute earlier blocks' aggregates, no waits */
#define DRS_FORCE_ROWS 0x8000u /* wkv: force the row-owning sweep (spans of rows, look-back)  */
#define DRS_LA_COMPOSE 0x10000u /* la_bidirectional: two scans and a sum, not the fused kernel */

/*
 * la_workspace_bytes -- device scratch that la_forward needs for these sizes
 * (segment states exchanged between workgroups, flags and counters).  Pure
 * host function; 0 when the call needs none (the step-by-step path: T <= 16
 * or DRS_FORCE_RECURRENT) and for invalid or unsupported sizes.  The decay
 * mode does not enter: a per-key-channel call (which needs none) may be given
 * the figure for its sizes all the same.
 */
DRS_API size_t la_workspace_bytes(int B, int H, int T, int Dk, int Dv, int dt, int chunk,
                                  unsigned flags);

/*
 * la_forward -- causal decayed linear attention, forward.
 *
 * Shapes (row-major, contiguous):
 *   q, k       [B, H, T, Dk]   storage `dt`
 *   v, y       [B, H, T, Dv]   storage `dt`
 *   decay      NULL (mode NONE) | fp32 [H] (HEAD) | fp32 [B, H, T] (STEP) |
 *              fp32 [B, H, T, Dk] (ELEM); factors are expected in [0, 1].  In the reversed order the
 *              factor stored at index t still belongs to token t: it
 *              multiplies the state arriving from t+1.
 *   state_in   fp32 [B, H, Dk, Dv] or NULL (zero state).  The decay factor of
 *              the first visited step multiplies it.
 *   cum_k_in   fp32 [B, H, Dk] or NULL (zero); only with DRS_NORMALIZE.
 *   state_out  fp32 [B, H, Dk, Dv] or NULL (not written).  May be exactly
 *              state_in (in-place update); any other overlap is undefined.
 *   cum_k_out  fp32 [B, H, Dk] or NULL; only with DRS_NORMALIZE.  May be
 *              exactly cum_k_in (in-place); any other overlap is undefined.
 *              In place, the chunked kernel's last segment overwrites them only
 *              after every wave of every earlier segment has read them (the
 *              workgroups then take their ids from an atomic start ticket, so
 *              that wait is always on a running workgroup).  Should it ever run
 *              out (~50 ms), state and key sum are left as they were, and word 3
 *              of the workspace counts it (as it counts any earlier aggregate a
 *              wave had to compute itself): a caller that updates in place reads
 *              that word, zero after an ordinary call, to know the update took.
 *   y must not overlap any input.  q, k, v and y must be 16-byte aligned.
 *   workspace  device scratch of at least la_workspace_bytes(...) bytes,
 *              16-byte aligned.  Its first 256 bytes (counters) must be zero
 *              before its first use; every call leaves them re-armed for the
 *              next call, whatever its sizes.  Calls that share a workspace
 *              must be ordered on one stream.
 *
 * Sizes: B, H, T >= 1; Dk, Dv in {16, 32, 64, 128}.
 * chunk: time-chunk length of the kernel, 0 = default; 16, 32 or 64.  The
 *        result does not depend on the chunk length beyond rounding.
 * flags: DRS_REVERSE | DRS_NORMALIZE, and at most one of DRS_FORCE_RECURRENT /
 *        DRS_FORCE_CHUNKED; DRS_LA_OWN_AGGREGATES (below).
 *
 * Segments: the chunked kernel (scalar factors) splits long sequences into
 * time segments run by separate workgroups.  Each publishes its segment's
 * aggregate (the decayed sum of k v^T and the segment's decay, the prefix
 * operator of RetNet issue #21); a later segment folds those of all earlier
 * segments into its entering state.  A wave that does not see an earlier
 * aggregate within its wait budget (~50 ms; its workgroup not started, e.g.
 * while other kernels occupy the GPU) computes it from k, v and the factors
 * itself, in fp32, so the call completes whatever the scheduling.
 * DRS_LA_OWN_AGGREGATES makes every wave do so without waiting (slow: each
 * segment re-reads all earlier keys and values); it exists to test that path
 * and has no effect on the other kernels.
 *
 * Paths: T <= 16 (a decode step is T = 1, with the carried state and key sum
 * of flash-linear-attention issue #268) runs the step-by-step kernel: one
 * workgroup per (b, h) holding the state in registers, bound by the state's own
 * traffic.  Longer sequences run the chunked kernels; for ELEM that is a kernel
 * of its own (bf16 inputs, no DRS_NORMALIZE, decay 16-byte aligned; other ELEM
 * calls take the step-by-step kernel at every length).  It floors each step's
 * factor at 2^-15 (so a zero factor restarts the state up to that share).  The
 * paths agree up to rounding; the FORCE flags pin one (ELEM with
 * DRS_FORCE_CHUNKED outside those conditions is unsupported).
 *
 * The states stay fp32 whatever `dt` is.  With DRS_NORMALIZE there is no
 * epsilon: the division is IEEE, so q_t^T z_t == 0 gives inf/NaN.  A decay
 * factor of 0 restarts the state exactly (scalar factors: log2 0 is floored at
 * -256, and 2^-256 is zero in fp32).
 *
 * Errors: DRS_ERR_INVALID for a NULL q/k/v/y, a size < 1, a decay pointer whose
 * NULL-ness disagrees with `mode`, a cum_k pointer without DRS_NORMALIZE,
 * y == q/k/v, a misaligned pointer, both FORCE flags, an unknown flag bit,
 * mode or dtype; DRS_ERR_UNSUPPORTED for Dk/Dv or chunk outside the lists
 * above, ELEM with DRS_FORCE_CHUNKED outside its conditions, or a step-by-step call with
 * T * Dv * sizeof(dt) >= 2^31; DRS_ERR_WORKSPACE for a missing or short
 * workspace; DRS_ERR_DEVICE if the launch fails.
 */
DRS_API int la_forward(const void *q, const void *k, const void *v, int dt,
                       const float *decay, int mode,
                       const float *state_in, const float *cum_k_in,
                       void *y, float *state_out, float *cum_k_out,
                       int B, int H, int T, int Dk, int Dv,
                       int chunk, unsigned flags,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * la_forward_group -- up to DRS_MAX_GROUP independent la_forward problems of one
 * shape (B, H, T, Dk, Dv, dt, chunk) in one call: for instance the forward and the
 * reverse scan of the same sequences.  When every problem takes the chunked kernel
 * for scalar factors with the same decay mode and normaliser (reverse may differ),
 * they share one launch: problem i owns workgroups [i n, (i + 1) n), and each
 * problem's look-back waits only on its own earlier segments, which have lower ids.
 * The second problem's workgroups then start on compute units that the first one
 * frees, instead of after its last workgroup.  Otherwise the problems run one
 * after another.  The results are those of la_forward for each problem.
 *
 *   probs      count problems: pointers, decay mode and flags as la_forward takes
 *              them (DRS_REVERSE, DRS_NORMALIZE and the force flags).
 *   count      1 .. DRS_MAX_GROUP.
 *   workspace  at least la_forward_group_workspace_bytes(count, ..., flags) bytes,
 *              flags being the union of the problems' flags: the 256 bytes of
 *              counters that every call keeps (problem i uses the four words from
 *              word 0, 32, 16 or 48;
 *              zero before first use, re-armed by every call), then a region of
 *              flags and aggregates per problem.  The same contract as
 *              la_forward's workspace, which it may be.
 *
 * No output of one problem may be an argument of another (they run at the same
 * time).  Errors: DRS_ERR_INVALID for count outside 1 .. DRS_MAX_GROUP, a NULL
 * probs or such an overlap, otherwise la_forward's for the first problem that
 * fails (nothing is launched when any problem is invalid).
 */
#define DRS_MAX_GROUP 4
typedef struct {
    const void *q, *k, *v;      /* [B,H,T,Dk], [B,H,T,Dk], [B,H,T,Dv] in dt */
    const float *decay;         /* as la_forward's, by mode */
    int mode;                   /* drs_decay */
    const float *state_in, *cum_k_in;
    void *y;                    /* [B,H,T,Dv] in dt */
    float *state_out, *cum_k_out;
    unsigned flags;
} drs_la_problem;

DRS_API size_t la_forward_group_workspace_bytes(int count, int B, int H, int T, int Dk, int Dv, int dt,
                                                int chunk, unsigned flags);
DRS_API int la_forward_group(const drs_la_problem *probs, int count, int dt, int B, int H, int T,
                             int Dk, int Dv, int chunk, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * la_forward_noalloc -- la_forward for callers that cannot allocate (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The same operation, arguments, paths and results as la_forward (the same
 * kernels; bitwise equal outputs), minus the workspace: the scratch those
 * kernels need (segment aggregates, flags, counters) is a static device array
 * of DRS_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  Nothing is allocated: no hipMalloc / hipFree, no allocating
 * library call.  On its first call on a device the library looks up that
 * device's copy of the array (hipGetSymbolAddress, with that device current);
 * each call then clears the array's counters and flags with a small fill
 * kernel on `stream` before the attention kernel.
 *
 * Every call on one GPU shares that GPU's array: calls whose execution
 * overlaps on one GPU (different streams, or host threads) race and give
 * undefined results.  Order them on one stream.
 *
 * Errors: those of la_forward (DRS_ERR_WORKSPACE aside), checked first, then
 * DRS_ERR_SCRATCH if the sizes need more than DRS_NOALLOC_SCRATCH_BYTES
 * (la_workspace_bytes bounds the figure; 64 MiB covers, at any T and
 * Dk = Dv = 128, up to 960 (b, h) units with scalar factors and 512 with
 * per-key-channel factors; the step-by-step path, T <= 16, needs none), and
 * DRS_ERR_DEVICE if the array's address cannot be obtained or a launch fails.
 * Nothing is enqueued on an error.
 */
#define DRS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
DRS_API int la_forward_noalloc(const void *q, const void *k, const void *v, int dt,
                               const float *decay, int mode,
                               const float *state_in, const float *cum_k_in,
                               void *y, float *state_out, float *cum_k_out,
                               int B, int H, int T, int Dk, int Dv,
                               int chunk, unsigned flags, void *stream);

/*
 * wkv_workspace_bytes -- device scratch that wkv_forward needs for these
 * sizes and flags (0 when the chosen path needs none).  Pure host function.
 * Returns 0 as well for invalid sizes (wkv_forward then reports the error).
 */
DRS_API size_t wkv_workspace_bytes(int B, int T, int C, unsigned flags);

/*
 * wkv_forward -- RWKV-4 WKV, forward, fp32.
 *
 *   w          fp32 [C]        per-step additive log-decay (t_decay), normally < 0
 *   u          fp32 [C]        bonus of the current token (t_first)
 *   k, v       fp32 [B, T, C]
 *   state_in   fp32 [3, B, C] planes (aa, bb, pp), or NULL for aa = bb = 0 and
 *              pp = -1e38 (the empty state).  (aa, bb, pp) stands for the sums
 *              aa*e^pp (values) and bb*e^pp (weights).
 *   y          fp32 [B, T, C]
 *   state_out  fp32 [3, B, C] or NULL; may be exactly state_in.
 *   workspace  device scratch of at least wkv_workspace_bytes(B, T, C, flags)
 *              bytes (may be NULL when that is 0), 16-byte aligned.  Its first
 *              256 bytes (counters) must be zero before its first use; every
 *              call leaves them re-armed for the next call, whatever its sizes.
 *              Two calls that share one workspace must be ordered on one stream.
 *
 * flags: at most one of DRS_FORCE_SEQ, DRS_FORCE_SCAN, DRS_FORCE_CHAIN,
 * DRS_FORCE_ROWS pins the path.  DRS_FORCE_ROWS (never chosen by itself) runs
 * the row-owning sweep: workgroups own 1 KB pieces of rows (256 channels per
 * wave) over short time spans and pass the state between spans by a look-back;
 * it needs C % 4 == 0, 16-byte aligned k, v and y and a state_out other than
 * state_in, else DRS_ERR_UNSUPPORTED.  Otherwise the library picks the chained single-pass kernel (the
 * state passed between time blocks) when T > 64, its size limits hold and
 * either there are at least 512 groups of 64 channels (B * ceil(C / 64): one
 * workgroup then walks all time blocks of its channels and nothing is
 * exchanged between workgroups) or the groups times the 256-step time blocks
 * number at most 512 (one resident round); else the two-pass segment scan when
 * B*C < 32768 and T >= 256, else the sequential kernel.  All give the same
 * result up to fp32 rounding.  In the chained kernel's look-back a wave that
 * does not see an earlier block's aggregate within its wait budget (~50 ms)
 * computes it from that block's k and v itself (not when state_out is
 * state_in: then the earlier blocks are started first and waited for);
 * DRS_WKV_OWN_AGGREGATES makes it do so for every earlier block without
 * waiting (slow; for testing that path; the row-owning sweep likewise; no
 * effect on the other kernels).
 *
 * Errors: DRS_ERR_INVALID for a NULL required pointer, B, T or C < 1, more than
 * one FORCE flag, an unknown flag bit or a misaligned pointer;
 * DRS_ERR_UNSUPPORTED for sizes a forced path does not cover (B > 65535);
 * DRS_ERR_WORKSPACE for a short workspace; DRS_ERR_DEVICE if a launch fails.
 */
DRS_API int wkv_forward(const float *w, const float *u, const float *k, const float *v,
                        const float *state_in, float *y, float *state_out,
                        int B, int T, int C, unsigned flags,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * ema_workspace_bytes -- device scratch that ema_forward needs for these sizes
 * (0 when the chosen kernel needs none, and for invalid or unsupported sizes).
 * Pure host function.
 */
DRS_API size_t ema_workspace_bytes(int B, int T, int C, int dt, unsigned flags);

/*
 * ema_forward -- gated element-wise exponential moving average, forward:
 *
 *     y_t = f_t * y_{t-1} + x_t        per (b, c), y_{-1} = state_in
 *
 * RetNet issue #21 ("removing the O(T^2) training cost"): the cumulative_ema
 * routine with its associative operator (x_a, f_a) o (x_b, f_b) =
 * (x_a f_b + x_b, f_a f_b) and a `reverse` option, and the variant in which a
 * layer produces factors (sigmoid-activated, so in (0, 1)) and values of one
 * shape and feeds them to it directly.  The factors are taken as given: any
 * activation belongs to the caller.  With DRS_REVERSE the recurrence runs from
 * t = T-1 down to 0 (the forward call on time-reversed inputs, the output
 * reversed back); state_in then enters at t = T-1.
 *
 *   x, f       [B, T, C] values and factors, fp32 or bf16 (both `dt`), contiguous,
 *              aligned to their element size
 *   state_in   fp32 [B, C] or NULL (zero)
 *   y          [B, T, C] in `dt` (RNE rounding for bf16); must not overlap x or f
 *   state_out  fp32 [B, C] or NULL; the output after the last visited step.  May
 *              be exactly state_in.
 *   workspace  device scratch of at least ema_workspace_bytes(...) bytes (may be
 *              NULL when that is 0), 16-byte aligned; its first 256 bytes must be
 *              zero before its first use, every call leaves them re-armed, and
 *              calls that share one must be ordered on one stream.
 *   flags      DRS_REVERSE or 0.
 *
 * All pointers are caller-owned device pointers; work is enqueued on `stream`
 * (hipStream_t, NULL = default) without synchronising; nothing is allocated.
 * Accumulation is fp32.
 *
 * Errors: DRS_ERR_INVALID for a NULL x/f/y, a size < 1, an unknown dtype or flag
 * bit, y overlapping x or f, a misaligned pointer; DRS_ERR_UNSUPPORTED when
 * T*C elements of one batch row exceed 2^31 bytes; DRS_ERR_WORKSPACE for a
 * missing or short workspace; DRS_ERR_DEVICE if the launch fails.
 */
DRS_API int ema_forward(const void *x, const void *f, int dt, const float *state_in, void *y,
                        float *state_out, int B, int T, int C, unsigned flags,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * la_bidirectional_workspace_bytes / la_bidirectional -- bidirectional linear
 * attention: the forward and the reverse la_forward call on the same inputs,
 * from zero state, their outputs summed (RetNet issue #21: a bidirectional
 * encoder combines a call with reverse=False and one with reverse=True; each
 * includes the current token, so its term enters twice).  With DRS_NORMALIZE
 * each direction is normalised on its own before the sum.
 *
 * Arguments as la_forward without states; flags: DRS_NORMALIZE, the FORCE
 * flags, DRS_LA_OWN_AGGREGATES and DRS_LA_COMPOSE (DRS_REVERSE is invalid here).
 * The counters rule of la_forward applies to the workspace.
 *
 * Two paths.  With no factor or one per head, no normaliser, Dk, Dv <= 64, the
 * default chunk size and T above the step-by-step limit, one fused kernel reads
 * q, k and v once and computes both orders (the score mask g^|t-s| with the
 * diagonal counted twice within a chunk; a forward and a reverse segment
 * exchange between workgroups); y is rounded once.  Otherwise, and with
 * DRS_LA_COMPOSE, the forward call writes y and the reverse call adds into it
 * (the chunked kernel for scalar factors: bf16 y is rounded after each call) or
 * into the workspace's second output, which a third kernel adds into y (bf16:
 * one rounding per direction and one after the sum).  The workspace size covers
 * either path: the scan's scratch followed by a second output of y's size, or
 * the fused kernel's two exchange areas, whichever is larger.
 */
DRS_API size_t la_bidirectional_workspace_bytes(int B, int H, int T, int Dk, int Dv, int dt,
                                                int chunk, unsigned flags);
DRS_API int la_bidirectional(const void *q, const void *k, const void *v, int dt,
                             const float *decay, int mode, void *y,
                             int B, int H, int T, int Dk, int Dv, int chunk, unsigned flags,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * ema_bidirectional_workspace_bytes / ema_bidirectional -- the forward and the
 * reverse gated EMA from zero, summed: the O(TC) bidirectional encoder of
 * RetNet issue #21.  Arguments as ema_forward without states; flags must be 0.
 * When B * ceil(C/64) fills the GPU (>= 512) one fused kernel runs: block
 * summaries of both directions, then the outputs, x and f read twice and y
 * written once; the workspace holds the block summaries.  Otherwise the two
 * directions run as two calls and an add, and the workspace holds the scan's
 * scratch followed by a second output of y's size.  Counters rule of
 * ema_forward; errors as ema_forward.
 */
DRS_API size_t ema_bidirectional_workspace_bytes(int B, int T, int C, int dt, unsigned flags);
DRS_API int ema_bidirectional(const void *x, const void *f, int dt, void *y, int B, int T, int C,
                              unsigned flags, void *workspace, size_t workspace_bytes, void *stream);

/*
 * la_backward_workspace_bytes / la_backward -- gradients of la_forward: of
 * L = sum_t dy_t . y_t + <dstate_out, S_final> (+ <dcum_k_out, z_final> with
 * DRS_NORMALIZE) with respect to q, k, v, the factors, the initial state and
 * (normalised) the initial key sum.  RWKV-LM discussion #189 notes that such
 * gradients are again cumulative sums.
 *
 * Without normalisation and with scalar factors (NONE, HEAD, STEP) they are
 * three decayed scans run on the chunked forward kernels,
 *     dq_t = S_t dy_t            (the forward-order scan of v_s k_s^T),
 *     dk_t = G_t v_t, dv_t = G_t^T k_t   (opposite-order scans of q_s dy_s^T,
 *                                 G_t the gradient of the state leaving step t),
 * plus the factor gradient from dL/d(log g_t) = (sum over the steps visited at
 * or after t of q.dq - k.dk) + <dstate_out, S_final>, divided by g_t.
 *
 * With DRS_NORMALIZE (y = QKV / QK1 of flash-linear-attention issue #268), with
 * one factor per key channel (ELEM), or with DRS_FORCE_RECURRENT, a step-by-step
 * kernel pair runs instead, one workgroup per (b, h) with the state and its
 * gradient in registers: a forward sweep recomputes S_t and z_t and passes
 * a_t = dy_t / d_t to the numerator n_t = q_t^T S_t and c_t = -(dy_t . y_t) / d_t
 * to the denominator d_t = q_t^T z_t (dq_t = S_t a_t + z_t c_t); a reverse sweep
 * carries G and the key sum's gradient Gz (dk_t = G v_t + Gz, dv_t = G^T k_t)
 * and the same factor-gradient sum per key channel, including
 * <dcum_k_out, z_final>.  It is bound by one barrier per step.
 *
 *   q, k, v, dt, decay, mode, state_in, cum_k_in, B..Dv, chunk: those of the
 *              forward call (every mode; cum_k_in only with DRS_NORMALIZE).
 *   state_out  fp32 [B, H, Dk, Dv]: the forward call's final state; required
 *              on the chunked path when both ddecay and dstate_out are given,
 *              else may be NULL (the step-by-step path recomputes it).
 *   dy         [B, H, T, Dv] in `dt`; dstate_out fp32 [B,H,Dk,Dv] or NULL (zero);
 *   dcum_k_out fp32 [B, H, Dk] or NULL (zero), only with DRS_NORMALIZE.
 *   dq, dk     [B, H, T, Dk] in `dt`; dv [B, H, T, Dv] in `dt`.
 *   ddecay     NULL, or fp32 with decay's shape: [H] (HEAD: summed over batch
 *              and time), [B, H, T] (STEP) or [B, H, T, Dk] (ELEM); must be NULL
 *              for NONE.  A factor of 0 gives a non-finite gradient (the
 *              division by g_t).
 *   dstate_in  fp32 [B, H, Dk, Dv] or NULL; dcum_k_in fp32 [B, H, Dk] or NULL
 *              (only with DRS_NORMALIZE).
 *   flags      DRS_REVERSE and DRS_NORMALIZE as in the forward call, and at most
 *              one FORCE flag.
 *   workspace  at least la_backward_workspace_bytes(...) bytes, 16-byte aligned;
 *              counters rule of la_forward.  (The decay mode is not an argument
 *              of the query: the figure covers either path.)
 * No output may alias an input or another output; q, k, v, dy, dq, dk, dv
 * 16-byte aligned.
 *
 * Errors: DRS_ERR_INVALID as la_forward, and for a missing output, ddecay with
 * mode NONE, a key-sum pointer without DRS_NORMALIZE, or (chunked path) ddecay
 * with dstate_out but no state_out; DRS_ERR_UNSUPPORTED for sizes la_forward
 * does not cover; DRS_ERR_WORKSPACE for a missing or short workspace;
 * DRS_ERR_DEVICE if a launch fails.
 */
DRS_API size_t la_backward_workspace_bytes(int B, int H, int T, int Dk, int Dv, int dt, int chunk,
                                           unsigned flags);
DRS_API int la_backward(const void *q, const void *k, const void *v, int dt,
                        const float *decay, int mode, const float *state_in,
                        const float *cum_k_in, const float *state_out, const void *dy,
                        const float *dstate_out, const float *dcum_k_out,
                        void *dq, void *dk, void *dv, float *ddecay, float *dstate_in,
                        float *dcum_k_in, int B, int H, int T, int Dk, int Dv, int chunk,
                        unsigned flags, void *workspace, size_t workspace_bytes, void *stream);

/*
 * wkv_backward_workspace_bytes / wkv_backward -- gradients of wkv_forward: of
 * L = sum_t dy_t y_t with respect to w, u (summed over the batch), k and v.
 * RWKV-LM discussion #189 notes that these gradients are again cumulative sums:
 * in the linear form y_t = (A_t + e^{u+k_t} v_t) / D_t the gradients reaching
 * the sums A_t, B_t obey reverse recurrences with the same decay e^w, and all
 * of these first-order recurrences have span summaries that combine exactly.
 * A forward sweep stores the state (and its w-derivative) entering every block
 * of 64 steps; a reverse walk over the blocks, time-parallel inside each block,
 * rebuilds the outputs and denominators (du, dw) and runs the reverse sums
 * (dk, dv), all on max-shifted log2 scales.  With fewer than 256 groups of 64
 * channels the blocks run in parallel instead, joined by per-channel scans of
 * their summaries (the workspace then also holds block summaries and carries).
 * The carried state enters only through the sums A_0 = aa e^pp, B_0 = bb e^pp,
 * so its gradient is d aa = Abar_0 e^pp, d bb = Bbar_0 e^pp, d pp = aa d aa +
 * bb d bb, from the reverse sums left at the first step.  No gradient flows in
 * from the final state (its log-scale is a running maximum, not a smooth
 * function of the inputs).  The outputs y_t are recomputed (not taken from the
 * forward call).  The log2-scales, the running sums and the stored
 * log2 denominators are fp64 (each exponential is the fp32 exp2 of a
 * difference formed in fp64): with keys of +-60 the scales reach ~90, where
 * fp32 rounding alone would cost ~1e-5 relative.
 *
 *   w, u, k, v, state_in  those of the forward call (fp32).
 *   dy         fp32 [B, T, C].
 *   dw, du     fp32 [C] or NULL (not computed).
 *   dk, dv     fp32 [B, T, C].
 *   dstate_in  fp32 [3, B, C] planes (d aa, d bb, d pp) or NULL (not computed);
 *              with state_in NULL (the empty state) it receives zeros.
 *   workspace  at least wkv_backward_workspace_bytes(B, T, C, 0) bytes
 *              (a state checkpoint per 64-step block, per-row partial sums), 16-byte
 *              aligned; contents on entry are ignored and the first 256 bytes
 *              are never touched, so it may be the workspace of the other calls.
 *   flags      0.
 * No output may alias an input or another output.
 *
 * Errors: DRS_ERR_INVALID for a NULL required pointer, a size < 1, a flag bit,
 * aliasing or misalignment; DRS_ERR_UNSUPPORTED for B > 65535 or T * C * 4 >= 2^31;
 * DRS_ERR_WORKSPACE for a missing or short workspace; DRS_ERR_DEVICE if a
 * launch fails.
 */
DRS_API size_t wkv_backward_workspace_bytes(int B, int T, int C, unsigned flags);
DRS_API int wkv_backward(const float *w, const float *u, const float *k, const float *v,
                         const float *state_in, const float *dy,
                         float *dw, float *du, float *dk, float *dv, float *dstate_in,
                         int B, int T, int C, unsigned flags,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Static, NUL-terminated description of a drs_status value. */
DRS_API const char *drs_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
DRS_API int drs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DRS_H_ */
