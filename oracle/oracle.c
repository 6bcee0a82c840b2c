/*
 * oracle.c -- plain, slow, fp64 reference of the decayed recurrences.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or constant with the
 * HIP kernels.
 *
 * Every routine is the sequential definition, one independent unit at a time,
 * in double precision.  The only parallelism is an OpenMP loop over units
 * that never interact (a (b,h) pair for linear attention, a (b,c) pair for
 * WKV), so the result does not depend on the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_DECAY_NONE 0
#define ORACLE_DECAY_HEAD 1
#define ORACLE_DECAY_STEP 2
#define ORACLE_DECAY_ELEM 3

/*
 * Causal decayed linear attention, one (b,h) sequence at a time.
 *
 * Recurrence (tensortonic "cs336 linear attention duality" exercise, problem
 * statement): S_t = S_{t-1} + k_t v_t^T, y_t = q_t^T S_t, the current token
 * included.  Decay (RetNet issue #21, cumulative_ema docstring and retention
 * example): the factor of step t multiplies the state carried in from the
 * step before, S_t = g_t S_{t-1} + k_t v_t^T, so the factor of the first
 * visited step multiplies the initial state.  Reverse (same docstring): the
 * reversed call equals the forward call on inputs flipped along time, with
 * the output flipped back; the visiting order below is exactly that.
 * Normalisation (flash-linear-attention issue #268, the QKV/QK1 form and the
 * cached key sum): y_t = q_t^T S_t / q_t^T z_t where z carries the running
 * key sum (plus the cached sum of earlier keys); with decay, z obeys the same
 * recurrence as S with v replaced by 1.
 *
 * Per-element decay (RetNet issue #21: cumulative_ema takes factors of the
 * values' own shape): in ELEM mode the factor of step t is a vector over the
 * key dimension, g_t[i] multiplying row i of the state (and entry i of z), the
 * same factor for every value column -- the outer-product form with factors
 * broadcast along the value axis.
 *
 * Layouts (row-major): q,k [B,H,T,Dk]; v,y [B,H,T,Dv]; gamma [H] (HEAD),
 * [B,H,T] (STEP) or [B,H,T,Dk] (ELEM); state [B,H,Dk,Dv]; cum_k [B,H,Dk].
 * state_in / cum_k_in may be NULL (zero).  state_out is always written;
 * cum_k_out when normalize.
 */
void oracle_la(const double *q, const double *k, const double *v,
               const double *gamma, int decay_mode,
               const double *state_in, const double *cum_k_in,
               double *y, double *state_out, double *cum_k_out,
               long B, long H, long T, long Dk, long Dv,
               int reverse, int normalize, int nthreads)
{
    long units = B * H;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long unit = 0; unit < units; ++unit) {
        long b = unit / H, h = unit % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)(Dk * Dv));
        double *z = (double *)malloc(sizeof(double) * (size_t)Dk);
        for (long i = 0; i < Dk * Dv; ++i)
            S[i] = state_in ? state_in[unit * Dk * Dv + i] : 0.0;
        for (long i = 0; i < Dk; ++i)
            z[i] = (normalize && cum_k_in) ? cum_k_in[unit * Dk + i] : 0.0;

        for (long n = 0; n < T; ++n) {
            long t = reverse ? (T - 1 - n) : n;
            const double *qt = q + (unit * T + t) * Dk;
            const double *kt = k + (unit * T + t) * Dk;
            const double *vt = v + (unit * T + t) * Dv;
            double g = 1.0;
            if (decay_mode == ORACLE_DECAY_HEAD) g = gamma[h];
            if (decay_mode == ORACLE_DECAY_STEP) g = gamma[(b * H + h) * T + t];

            const double *ge = NULL;
            if (decay_mode == ORACLE_DECAY_ELEM) ge = gamma + ((b * H + h) * T + t) * Dk;

            /* S <- g S + k_t v_t^T ;  z <- g z + k_t  (row i decays by ge[i] in ELEM mode) */
            for (long i = 0; i < Dk; ++i) {
                const double gi = ge ? ge[i] : g;
                for (long j = 0; j < Dv; ++j)
                    S[i * Dv + j] = gi * S[i * Dv + j] + kt[i] * vt[j];
                z[i] = gi * z[i] + kt[i];
            }
            /* y_t = q_t^T S  (divided by q_t^T z when normalising) */
            double den = 0.0;
            if (normalize)
                for (long i = 0; i < Dk; ++i) den += qt[i] * z[i];
            double *yt = y + (unit * T + t) * Dv;
            for (long j = 0; j < Dv; ++j) {
                double acc = 0.0;
                for (long i = 0; i < Dk; ++i) acc += qt[i] * S[i * Dv + j];
                yt[j] = normalize ? acc / den : acc;
            }
        }
        if (state_out)
            memcpy(state_out + unit * Dk * Dv, S, sizeof(double) * (size_t)(Dk * Dv));
        if (normalize && cum_k_out)
            memcpy(cum_k_out + unit * Dk, z, sizeof(double) * (size_t)Dk);
        free(S);
        free(z);
    }
}

/*
 * RWKV-4 WKV, one (b,c) channel at a time (RWKV-LM issue #167 defines the
 * output; RWKV-LM discussion #189 reads it as exponentially weighted
 * (value, log-scale) pairs that combine associatively).
 *
 * By definition y_t is a weighted mean of values: every token s < t already
 * seen has weight e^{k_s + (t-1-s) w} (its key, decayed once per later step),
 * the current token has weight e^{u + k_t} (the bonus u), and the carried state
 * contributes its own weighted sums decayed by e^{t w}.  w is the per-step
 * additive log-decay (t_decay, normally negative), u the bonus (t_first).
 *
 * A weighted sum is kept as a triple (a, b, p): value-sum a e^p and weight-sum
 * b e^p.  wsum_join below adds two such sums, expressing both on the larger of
 * their log-scales so that no exponential has a positive argument (the pair
 * operator of discussion #189).  The carried state (aa, bb, pp) is the sum over
 * the absorbed tokens; per token:
 *   y_t   = value-sum / weight-sum of  (aa, bb, pp) joined with (v_t, 1, u + k_t);
 *   state = (aa, bb, pp + w) joined with (v_t, 1, k_t)  -- one step of decay,
 *           then the token at its own weight;
 * so pp is the largest decayed log-weight seen so far, the canonical scale.
 *
 * Layouts: w,u [C]; k,v,y [B,T,C]; state [3,B,C] as planes (aa, bb, pp).
 * NULL state_in means aa = bb = 0 and pp = -1e38.
 */
struct wsum { double a, b, p; };

static struct wsum wsum_join(struct wsum x, struct wsum y)
{
    const double p = x.p > y.p ? x.p : y.p;
    const double ex = exp(x.p - p), ey = exp(y.p - p);
    struct wsum r = { x.a * ex + y.a * ey, x.b * ex + y.b * ey, p };
    return r;
}

void oracle_wkv(const double *w, const double *u, const double *k, const double *v,
                const double *state_in, double *y, double *state_out,
                long B, long T, long C, int nthreads)
{
    long units = B * C;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (long unit = 0; unit < units; ++unit) {
        long b = unit / C, c = unit % C;
        struct wsum st = { 0.0, 0.0, -1e38 };
        if (state_in) {
            st.a = state_in[0 * B * C + unit];
            st.b = state_in[1 * B * C + unit];
            st.p = state_in[2 * B * C + unit];
        }
        for (long t = 0; t < T; ++t) {
            const long i = (b * T + t) * C + c;
            const struct wsum now = { v[i], 1.0, u[c] + k[i] };     /* current token, with the bonus */
            const struct wsum mean = wsum_join(st, now);
            y[i] = mean.a / mean.b;
            const struct wsum past = { st.a, st.b, st.p + w[c] };   /* one step of decay */
            const struct wsum tok = { v[i], 1.0, k[i] };
            st = wsum_join(past, tok);
        }
        if (state_out) {
            state_out[0 * B * C + unit] = st.a;
            state_out[1 * B * C + unit] = st.b;
            state_out[2 * B * C + unit] = st.p;
        }
    }
}

/*
 * Gated element-wise EMA, one (b,c) channel at a time (RetNet issue #21: the
 * cumulative_ema routine, its associative operator (x_a, f_a) o (x_b, f_b) =
 * (x_a f_b + x_b, f_a f_b), and the O(TC) variant in which a layer produces
 * factors and values of one shape and feeds them to it directly).
 *
 * out_t = f_t out_{t-1} + x_t: the factor of step t multiplies the output
 * carried from the step before (the reading of the garbled docstring line that
 * the operator fixes), so the first visited step's factor multiplies the
 * initial state.  Reverse: the forward call on inputs flipped along time, the
 * output flipped back; the visiting order below is exactly that.
 *
 * Layouts: x, f, y [B,T,C]; state [B,C].  NULL state_in means zero;
 * state_out (if not NULL) receives the output after the last visited step.
 */
void oracle_ema(const double *x, const double *f, const double *state_in,
                double *y, double *state_out, long B, long T, long C,
                int reverse, int nthreads)
{
    long units = B * C;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (long unit = 0; unit < units; ++unit) {
        long b = unit / C, c = unit % C;
        double h = state_in ? state_in[unit] : 0.0;
        for (long n = 0; n < T; ++n) {
            long t = reverse ? (T - 1 - n) : n;
            long i = (b * T + t) * C + c;
            h = f[i] * h + x[i];
            y[i] = h;
        }
        if (state_out) state_out[unit] = h;
    }
}

/*
 * Backward of the causal decayed linear attention above (oracle_la): the
 * gradients of L = sum_t dy_t . y_t + <dstate_out, S_final> (+ <dcum_k_out,
 * z_final> with normalisation) with respect to q, k, v, the factors, the
 * initial state and (normalised) the initial key sum.  The pages only say that
 * the gradient is again a set of cumulative sums (RWKV-LM discussion #189);
 * this routine is the chain rule applied to the recurrence, visited in the
 * opposite order:
 *
 *   forward, keeping every state: S_before[n], z_before[n] enter step n
 *   backward, n = last .. first, with G = dL/dS and Gz = dL/dz (the gradients of
 *   the state and key sum leaving step n; dstate_out / dcum_k_out, or zero,
 *   before the first iteration):
 *     without normalisation y_t = q_t^T S_t, so the read-out passes dy_t on:
 *       a_t = dy_t, c_t = 0;
 *     with it (flash-linear-attention issue #268, QKV / QK1) y_t = n_t / d_t,
 *     n_t = q_t^T S_t, d_t = q_t^T z_t, so
 *       a_t = dL/dn_t = dy_t / d_t,  c_t = dL/dd_t = -(dy_t . y_t) / d_t;
 *     G     += q_t a_t^T,  Gz += q_t c_t      (the read-outs of S_t and z_t)
 *     dq_t   = S_t a_t + z_t c_t               (S_t, z_t leave step n)
 *     dk_t   = G v_t + Gz,  dv_t = G^T k_t     (the terms k_t v_t^T, k_t added)
 *     dg_t   = <G, S_before[n]> + <Gz, z_before[n]>   (per key row i in ELEM mode)
 *     G      = g_t G,  Gz = g_t Gz            (the factor scaled the entering state)
 *   dstate_in = G, dcum_k_in = Gz.
 *
 * dgamma_step receives dg per step: [B,H,T] for scalar modes (the caller sums
 * it for a per-head factor), [B,H,T,Dk] for ELEM.  May be NULL.  dstate_out,
 * dstate_in, cum_k_in, dcum_k_out and dcum_k_in may be NULL; the last three are
 * used only with normalize.
 */
void oracle_la_backward(const double *q, const double *k, const double *v,
                        const double *gamma, int decay_mode, const double *state_in,
                        const double *cum_k_in, const double *dy, const double *dstate_out,
                        const double *dcum_k_out, double *dq, double *dk, double *dv,
                        double *dgamma_step, double *dstate_in, double *dcum_k_in,
                        long B, long H, long T, long Dk, long Dv, int normalize,
                        int reverse, int nthreads)
{
    long units = B * H;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long unit = 0; unit < units; ++unit) {
        long h = unit % H;
        const long SZ = Dk * Dv;
        double *Sb = (double *)malloc(sizeof(double) * (size_t)((T + 1) * SZ));
        double *zb = (double *)malloc(sizeof(double) * (size_t)((T + 1) * Dk));
        double *G = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *Gz = (double *)malloc(sizeof(double) * (size_t)Dk);
        double *gv = (double *)malloc(sizeof(double) * (size_t)Dk);
        double *an = (double *)malloc(sizeof(double) * (size_t)Dv);

        /* forward: Sb[n], zb[n] enter step n, Sb[T], zb[T] are the final ones */
        for (long i = 0; i < SZ; ++i) Sb[i] = state_in ? state_in[unit * SZ + i] : 0.0;
        for (long i = 0; i < Dk; ++i) zb[i] = (normalize && cum_k_in) ? cum_k_in[unit * Dk + i] : 0.0;
        for (long n = 0; n < T; ++n) {
            long t = reverse ? (T - 1 - n) : n;
            const double *kt = k + (unit * T + t) * Dk;
            const double *vt = v + (unit * T + t) * Dv;
            for (long i = 0; i < Dk; ++i) {
                double g = 1.0;
                if (decay_mode == ORACLE_DECAY_HEAD) g = gamma[h];
                if (decay_mode == ORACLE_DECAY_STEP) g = gamma[unit * T + t];
                if (decay_mode == ORACLE_DECAY_ELEM) g = gamma[(unit * T + t) * Dk + i];
                for (long j = 0; j < Dv; ++j)
                    Sb[(n + 1) * SZ + i * Dv + j] = g * Sb[n * SZ + i * Dv + j] + kt[i] * vt[j];
                zb[(n + 1) * Dk + i] = normalize ? g * zb[n * Dk + i] + kt[i] : 0.0;
            }
        }

        /* backward */
        for (long i = 0; i < SZ; ++i) G[i] = dstate_out ? dstate_out[unit * SZ + i] : 0.0;
        for (long i = 0; i < Dk; ++i) Gz[i] = (normalize && dcum_k_out) ? dcum_k_out[unit * Dk + i] : 0.0;
        for (long n = T - 1; n >= 0; --n) {
            long t = reverse ? (T - 1 - n) : n;
            const double *qt = q + (unit * T + t) * Dk;
            const double *kt = k + (unit * T + t) * Dk;
            const double *vt = v + (unit * T + t) * Dv;
            const double *dyt = dy + (unit * T + t) * Dv;
            const double *Sa = Sb + (n + 1) * SZ;   /* the state leaving step n */
            const double *Se = Sb + n * SZ;         /* the state entering step n */
            const double *za = zb + (n + 1) * Dk, *ze = zb + n * Dk;
            /* gradients reaching the numerator (a) and the denominator (c) */
            double den = 1.0, cden = 0.0;
            if (normalize) {
                den = 0.0;
                for (long i = 0; i < Dk; ++i) den += qt[i] * za[i];
                double dyy = 0.0;   /* dy_t . y_t */
                for (long j = 0; j < Dv; ++j) {
                    double num = 0.0;
                    for (long i = 0; i < Dk; ++i) num += qt[i] * Sa[i * Dv + j];
                    dyy += dyt[j] * (num / den);
                }
                cden = -dyy / den;
            }
            for (long j = 0; j < Dv; ++j) an[j] = dyt[j] / den;
            for (long i = 0; i < Dk; ++i)
                for (long j = 0; j < Dv; ++j) G[i * Dv + j] += qt[i] * an[j];
            for (long i = 0; i < Dk; ++i) Gz[i] += qt[i] * cden;
            for (long i = 0; i < Dk; ++i) {
                double a = 0.0, c = 0.0;
                for (long j = 0; j < Dv; ++j) {
                    a += Sa[i * Dv + j] * an[j];
                    c += G[i * Dv + j] * vt[j];
                }
                dq[(unit * T + t) * Dk + i] = a + za[i] * cden;
                dk[(unit * T + t) * Dk + i] = c + Gz[i];
            }
            for (long j = 0; j < Dv; ++j) {
                double a = 0.0;
                for (long i = 0; i < Dk; ++i) a += G[i * Dv + j] * kt[i];
                dv[(unit * T + t) * Dv + j] = a;
            }
            for (long i = 0; i < Dk; ++i) {
                double g = 1.0;
                if (decay_mode == ORACLE_DECAY_HEAD) g = gamma[h];
                if (decay_mode == ORACLE_DECAY_STEP) g = gamma[unit * T + t];
                if (decay_mode == ORACLE_DECAY_ELEM) g = gamma[(unit * T + t) * Dk + i];
                gv[i] = g;
            }
            if (dgamma_step) {
                if (decay_mode == ORACLE_DECAY_ELEM) {
                    for (long i = 0; i < Dk; ++i) {
                        double a = Gz[i] * ze[i];
                        for (long j = 0; j < Dv; ++j) a += G[i * Dv + j] * Se[i * Dv + j];
                        dgamma_step[(unit * T + t) * Dk + i] = a;
                    }
                } else {
                    double a = 0.0;
                    for (long i = 0; i < SZ; ++i) a += G[i] * Se[i];
                    for (long i = 0; i < Dk; ++i) a += Gz[i] * ze[i];
                    dgamma_step[unit * T + t] = a;
                }
            }
            for (long i = 0; i < Dk; ++i) {
                for (long j = 0; j < Dv; ++j) G[i * Dv + j] *= gv[i];
                Gz[i] *= gv[i];
            }
        }
        if (dstate_in) memcpy(dstate_in + unit * SZ, G, sizeof(double) * (size_t)SZ);
        if (normalize && dcum_k_in) memcpy(dcum_k_in + unit * Dk, Gz, sizeof(double) * (size_t)Dk);
        free(Sb);
        free(zb);
        free(G);
        free(Gz);
        free(gv);
        free(an);
    }
}

/*
 * Backward of the WKV recurrence above: the gradients of L = sum_t dy_t y_t
 * with respect to w, u (per batch row and channel; the caller sums over the
 * batch), k, v and the carried state given (its three planes).  No gradient
 * flows in from the final state.
 *
 * The chain rule is applied to the recurrence in its linear form (the one the
 * log-scale state stands for, RWKV-LM discussion #189): with the decayed sums
 * A_t, B_t of the tokens before t (A_0 = aa e^pp, B_0 = bb e^pp of state_in),
 *   A_{t+1} = e^w A_t + e^{k_t} v_t,   B_{t+1} = e^w B_t + e^{k_t},
 *   y_t = (A_t + e^{u+k_t} v_t) / (B_t + e^{u+k_t}).
 * With r_t = dy_t / D_t and s_t = -dy_t y_t / D_t (D_t the denominator) the
 * gradients reaching A_t and B_t obey, for t = T-1 .. 0,
 *   Abar_t = r_t + e^w Abar_{t+1},    Bbar_t = s_t + e^w Bbar_{t+1},
 * and
 *   du     = sum_t e^{u+k_t} (v_t r_t + s_t)
 *   dk_t   = e^{u+k_t} (v_t r_t + s_t) + e^{k_t} (v_t Abar_{t+1} + Bbar_{t+1})
 *   dv_t   = e^{u+k_t} r_t + e^{k_t} Abar_{t+1}
 *   dw     = sum_t e^w (A_t Abar_{t+1} + B_t Bbar_{t+1}).
 * The carried state enters only through A_0 = aa e^pp and B_0 = bb e^pp, so
 *   d aa = Abar_0 e^pp,   d bb = Bbar_0 e^pp,   d pp = aa d aa + bb d bb
 * (all zero for the empty state, pp = -1e38).
 * Everything is formed in fp64 without the max shift, so the routine is
 * exact only while the exponents stay far from fp64's range (|k|, |u|, |pp|
 * well below 700; underflow of long decays to 0 is harmless).
 *
 * Layouts: as oracle_wkv; dw_bc, du_bc [B,C]; dk, dv [B,T,C]; dstate_in NULL
 * or [3,B,C] planes (d aa, d bb, d pp).
 */
void oracle_wkv_backward(const double *w, const double *u, const double *k, const double *v,
                         const double *state_in, const double *dy, double *dw_bc, double *du_bc,
                         double *dk, double *dv, double *dstate_in, long B, long T, long C, int nthreads)
{
    long units = B * C;
    if (nthreads < 1) nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (long unit = 0; unit < units; ++unit) {
        long b = unit / C, c = unit % C;
        double *A = (double *)malloc(sizeof(double) * (size_t)(T + 1));
        double *Bs = (double *)malloc(sizeof(double) * (size_t)(T + 1));
        const double ew = exp(w[c]), uc = u[c];
        A[0] = 0.0;
        Bs[0] = 0.0;
        if (state_in) {
            const double pp0 = state_in[2 * B * C + unit];
            A[0] = state_in[0 * B * C + unit] * exp(pp0);
            Bs[0] = state_in[1 * B * C + unit] * exp(pp0);
        }
        for (long t = 0; t < T; ++t) {
            const long i = (b * T + t) * C + c;
            A[t + 1] = ew * A[t] + exp(k[i]) * v[i];
            Bs[t + 1] = ew * Bs[t] + exp(k[i]);
        }
        double Abar = 0.0, Bbar = 0.0, du = 0.0, dw = 0.0;
        for (long t = T - 1; t >= 0; --t) {
            const long i = (b * T + t) * C + c;
            const double cur = exp(uc + k[i]);
            const double D = Bs[t] + cur;
            const double yt = (A[t] + cur * v[i]) / D;
            const double r = dy[i] / D, s = -dy[i] * yt / D;
            du += cur * (v[i] * r + s);
            dk[i] = cur * (v[i] * r + s) + exp(k[i]) * (v[i] * Abar + Bbar);
            dv[i] = cur * r + exp(k[i]) * Abar;
            dw += ew * (A[t] * Abar + Bs[t] * Bbar);
            Abar = r + ew * Abar;
            Bbar = s + ew * Bbar;
        }
        dw_bc[unit] = dw;
        du_bc[unit] = du;
        if (dstate_in) {
            double daa = 0.0, dbb = 0.0, dpp = 0.0;
            if (state_in) {
                const double aa0 = state_in[0 * B * C + unit], bb0 = state_in[1 * B * C + unit];
                const double e0 = exp(state_in[2 * B * C + unit]);
                daa = Abar * e0;
                dbb = Bbar * e0;
                dpp = aa0 * daa + bb0 * dbb;
            }
            dstate_in[0 * B * C + unit] = daa;
            dstate_in[1 * B * C + unit] = dbb;
            dstate_in[2 * B * C + unit] = dpp;
        }
        free(A);
        free(Bs);
    }
}
