// sanitizer_driver.cpp -- host-side AddressSanitizer / UndefinedBehaviorSanitizer
// run of the fp64 oracle and of the C ABI's host logic (argument checks and
// workspace queries).  tests/test_sanitizers.py builds it together with a
// host-only build of every library source (no device code) and the oracle, all
// instrumented, and runs it on the CPU.  No ABI call here reaches a launch: each
// one fails validation, or is a pure host query.
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "drs.h"

extern "C" {
void oracle_la(const double *q, const double *k, const double *v, const double *gamma, int decay_mode,
               const double *state_in, const double *cum_k_in, double *y, double *state_out, double *cum_k_out,
               long B, long H, long T, long Dk, long Dv, int reverse, int normalize, int nthreads);
void oracle_wkv(const double *w, const double *u, const double *k, const double *v, const double *state_in,
                double *y, double *state_out, long B, long T, long C, int nthreads);
void oracle_ema(const double *x, const double *f, const double *state_in, double *y, double *state_out, long B,
                long T, long C, int reverse, int nthreads);
void oracle_la_backward(const double *q, const double *k, const double *v, const double *gamma, int decay_mode,
                        const double *state_in, const double *cum_k_in, const double *dy, const double *dstate_out,
                        const double *dcum_k_out, double *dq, double *dk, double *dv, double *dgamma_step,
                        double *dstate_in, double *dcum_k_in, long B, long H, long T, long Dk, long Dv,
                        int normalize, int reverse, int nthreads);
void oracle_wkv_backward(const double *w, const double *u, const double *k, const double *v, const double *state_in,
                         const double *dy, double *dw_bc, double *du_bc, double *dk, double *dv, double *dstate_in,
                         long B, long T, long C, int nthreads);
}

static int failures = 0;
#define EXPECT(cond)                                                               \
    do {                                                                           \
        if (!(cond)) {                                                             \
            std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);   \
            ++failures;                                                            \
        }                                                                          \
    } while (0)

static std::mt19937_64 gen(12345);
static std::vector<double> draw(size_t n, double lo, double hi) {
    std::uniform_real_distribution<double> u(lo, hi);
    std::vector<double> x(n);
    for (double &e : x) e = u(gen);
    return x;
}
static bool finite(const std::vector<double> &x) {
    for (double e : x)
        if (!std::isfinite(e)) return false;
    return true;
}

static void oracle_runs() {
    const long B = 2, H = 3, T = 9, Dk = 3, Dv = 4;
    for (int mode = 0; mode < 4; ++mode)
        for (int norm = 0; norm < 2; ++norm)
            for (int rev = 0; rev < 2; ++rev) {
                auto q = draw(B * H * T * Dk, 0.2, 1.5), k = draw(B * H * T * Dk, 0.2, 1.5);
                auto v = draw(B * H * T * Dv, -1, 1), dy = draw(B * H * T * Dv, -1, 1);
                const size_t ng = mode == 1 ? H : mode == 2 ? B * H * T : mode == 3 ? B * H * T * Dk : 1;
                auto g = draw(ng, 0.3, 1.0);
                auto s0 = draw(B * H * Dk * Dv, -1, 1), z0 = draw(B * H * Dk, 0.5, 2);
                auto dsf = draw(B * H * Dk * Dv, -1, 1), dzf = draw(B * H * Dk, -1, 1);
                std::vector<double> y(B * H * T * Dv), sf(B * H * Dk * Dv), zf(B * H * Dk);
                oracle_la(q.data(), k.data(), v.data(), mode ? g.data() : nullptr, mode, s0.data(),
                          norm ? z0.data() : nullptr, y.data(), sf.data(), norm ? zf.data() : nullptr, B, H, T, Dk,
                          Dv, rev, norm, 2);
                EXPECT(finite(y) && finite(sf));
                std::vector<double> dq(B * H * T * Dk), dk(B * H * T * Dk), dv(B * H * T * Dv);
                std::vector<double> dg(mode == 3 ? B * H * T * Dk : B * H * T), ds0(B * H * Dk * Dv), dz0(B * H * Dk);
                oracle_la_backward(q.data(), k.data(), v.data(), mode ? g.data() : nullptr, mode, s0.data(),
                                   norm ? z0.data() : nullptr, dy.data(), dsf.data(), norm ? dzf.data() : nullptr,
                                   dq.data(), dk.data(), dv.data(), mode ? dg.data() : nullptr, ds0.data(),
                                   norm ? dz0.data() : nullptr, B, H, T, Dk, Dv, norm, rev, 2);
                EXPECT(finite(dq) && finite(dk) && finite(dv) && finite(ds0));
            }
    // WKV, with +-60 keys, from the empty state and from a carried one
    const long C = 5;
    auto w = draw(C, -3, -0.1), u = draw(C, -1, 1), kk = draw(B * T * C, -5, 5), vv = draw(B * T * C, -1, 1);
    kk[3] = 60.0;
    kk[11] = -60.0;
    auto st = draw(3 * B * C, 0.5, 2), dyw = draw(B * T * C, -1, 1);
    for (int with_state = 0; with_state < 2; ++with_state) {
        std::vector<double> y(B * T * C), so(3 * B * C);
        oracle_wkv(w.data(), u.data(), kk.data(), vv.data(), with_state ? st.data() : nullptr, y.data(), so.data(), B,
                   T, C, 2);
        EXPECT(finite(y) && finite(so));
        std::vector<double> dw(B * C), du(B * C), dk(B * T * C), dv(B * T * C), ds(3 * B * C);
        oracle_wkv_backward(w.data(), u.data(), kk.data(), vv.data(), with_state ? st.data() : nullptr, dyw.data(),
                            dw.data(), du.data(), dk.data(), dv.data(), ds.data(), B, T, C, 2);
        EXPECT(finite(dk) && finite(dv) && finite(dw) && finite(du) && finite(ds));
    }
    // gated EMA, both orders
    auto x = draw(B * T * C, -1, 1), f = draw(B * T * C, 0, 1), h0 = draw(B * C, -1, 1);
    for (int rev = 0; rev < 2; ++rev) {
        std::vector<double> y(B * T * C), so(B * C);
        oracle_ema(x.data(), f.data(), rev ? h0.data() : nullptr, y.data(), so.data(), B, T, C, rev, 2);
        EXPECT(finite(y) && finite(so));
    }
}

static void abi_checks() {
    // fake, 16-byte aligned addresses that no call here dereferences
    void *P1 = reinterpret_cast<void *>(0x1000), *P2 = reinterpret_cast<void *>(0x2000);
    void *P3 = reinterpret_cast<void *>(0x3000), *P4 = reinterpret_cast<void *>(0x4000);
    void *P5 = reinterpret_cast<void *>(0x5000), *P6 = reinterpret_cast<void *>(0x6000);
    void *P7 = reinterpret_cast<void *>(0x7000), *MIS = reinterpret_cast<void *>(0x1008);
    float *F = reinterpret_cast<float *>(0x8000);
    // workspace queries over small, ragged, huge and invalid sizes (size arithmetic)
    const int Bs[] = {-1, 0, 1, 3, 64, 1 << 16, INT_MAX};
    const int Ts[] = {0, 1, 16, 17, 2049, 1 << 20, INT_MAX};
    const int Ds[] = {16, 48, 128};
    for (int B : Bs)
        for (int T : Ts)
            for (int D : Ds)
                for (int dt = 0; dt < 3; ++dt) {
                    const unsigned flags[] = {0u, DRS_FORCE_RECURRENT, DRS_FORCE_CHUNKED, DRS_NORMALIZE};
                    for (unsigned fl : flags) {
                        (void)la_workspace_bytes(B, 7, T, D, D, (drs_dtype)dt, 0, fl);
                        (void)la_bidirectional_workspace_bytes(B, 7, T, D, 64, (drs_dtype)dt, 0, fl);
                        (void)la_backward_workspace_bytes(B, 7, T, 64, D, (drs_dtype)dt, 0, fl);
                    }
                    (void)wkv_workspace_bytes(B, T, D * 33, 0);
                    (void)wkv_workspace_bytes(B, T, D, DRS_FORCE_CHAIN);
                    (void)wkv_backward_workspace_bytes(B, T, D * 33, 0);
                    (void)ema_workspace_bytes(B, T, D * 5, (drs_dtype)dt, 0);
                    (void)ema_bidirectional_workspace_bytes(B, T, D * 5, (drs_dtype)dt, 0);
                }
    EXPECT(la_workspace_bytes(0, 1, 1, 64, 64, DRS_BF16, 0, 0) == 0);
    EXPECT(la_workspace_bytes(8, 8, 2048, 64, 64, DRS_BF16, 0, 0) > 0);

    // la_forward: each call fails its checks (T = 300 takes the chunked path, and no
    // workspace is given, so even a call whose other checks pass stops there)
    auto la = [&](const void *q, const void *y, int B, int T, int Dk, unsigned flags, drs_decay mode,
                  const float *decay) {
        return la_forward(q, P2, P3, DRS_BF16, decay, mode, nullptr, nullptr, const_cast<void *>(y), nullptr,
                          nullptr, B, 2, T, Dk, 64, 0, flags, nullptr, 0, nullptr);
    };
    EXPECT(la(nullptr, P4, 2, 300, 64, 0, DRS_DECAY_NONE, nullptr) == DRS_ERR_INVALID);
    EXPECT(la(P1, P4, 0, 300, 64, 0, DRS_DECAY_NONE, nullptr) == DRS_ERR_INVALID);
    EXPECT(la(P1, P1, 2, 300, 64, 0, DRS_DECAY_NONE, nullptr) == DRS_ERR_INVALID);
    EXPECT(la(MIS, P4, 2, 300, 64, 0, DRS_DECAY_NONE, nullptr) == DRS_ERR_INVALID);
    EXPECT(la(P1, P4, 2, 300, 64, 0, DRS_DECAY_HEAD, nullptr) == DRS_ERR_INVALID);
    EXPECT(la(P1, P4, 2, 300, 48, 0, DRS_DECAY_NONE, nullptr) == DRS_ERR_UNSUPPORTED);
    EXPECT(la(P1, P4, 2, 300, 64, 0x8u, DRS_DECAY_NONE, nullptr) == DRS_ERR_INVALID);
    EXPECT(la(P1, P4, 2, 300, 64, 0, DRS_DECAY_NONE, nullptr) == DRS_ERR_WORKSPACE);
    EXPECT(la(P1, P4, 2, 300, 64, 0, DRS_DECAY_STEP, F) == DRS_ERR_WORKSPACE);
    EXPECT(la(P1, P4, INT_MAX, INT_MAX, 128, 0, DRS_DECAY_NONE, nullptr) != DRS_OK);
    EXPECT(la(P1, P4, 1 << 20, 1 << 20, 128, DRS_FORCE_CHUNKED, DRS_DECAY_NONE, nullptr) != DRS_OK);
    // the entry point without allocation: the checks of la_forward, then the scratch limit
    EXPECT(la_forward_noalloc(nullptr, P2, P3, DRS_BF16, nullptr, DRS_DECAY_NONE, nullptr, nullptr, P4, nullptr,
                              nullptr, 2, 2, 300, 64, 64, 0, 0, nullptr) == DRS_ERR_INVALID);
    EXPECT(la_forward_noalloc(P1, P2, P3, DRS_BF16, nullptr, DRS_DECAY_NONE, nullptr, nullptr, P4, nullptr, nullptr, 64,
                              64, 4096, 128, 128, 0, 0, nullptr) == DRS_ERR_SCRATCH);
    // la_backward, la_bidirectional
    EXPECT(la_backward(P1, P2, P3, DRS_BF16, nullptr, DRS_DECAY_NONE, nullptr, nullptr, nullptr, P4, nullptr, nullptr,
                       P5, P6, P7, nullptr, nullptr, nullptr, 2, 2, 300, 64, 64, 0, 0, nullptr, 0,
                       nullptr) == DRS_ERR_WORKSPACE);
    EXPECT(la_backward(P1, P2, P3, DRS_BF16, nullptr, DRS_DECAY_NONE, nullptr, F, nullptr, P4, nullptr, nullptr, P5,
                       P6, P7, nullptr, nullptr, nullptr, 2, 2, 300, 64, 64, 0, 0, nullptr, 0,
                       nullptr) == DRS_ERR_INVALID);
    EXPECT(la_backward(P1, P2, P3, DRS_BF16, nullptr, DRS_DECAY_NONE, nullptr, F, nullptr, P4, nullptr, nullptr, P5,
                       P6, P7, nullptr, nullptr, nullptr, 2, 2, 300, 64, 64, 0, DRS_NORMALIZE, nullptr, 0,
                       nullptr) == DRS_ERR_WORKSPACE);
    EXPECT(la_bidirectional(P1, P2, P3, DRS_BF16, nullptr, DRS_DECAY_NONE, P4, 2, 2, 300, 64, 64, 0, DRS_REVERSE,
                            nullptr, 0, nullptr) == DRS_ERR_INVALID);
    EXPECT(la_bidirectional(P1, P2, P3, DRS_BF16, nullptr, DRS_DECAY_NONE, P4, 2, 2, 300, 64, 64, 0, 0, nullptr, 0,
                            nullptr) == DRS_ERR_WORKSPACE);
    // WKV and EMA
    EXPECT(wkv_forward(nullptr, F, F, F, nullptr, F, nullptr, 2, 8, 64, 0, nullptr, 0, nullptr) == DRS_ERR_INVALID);
    EXPECT(wkv_forward(F, F, F, F, nullptr, F, nullptr, 2, 8, 64, DRS_FORCE_SEQ | DRS_FORCE_SCAN, nullptr, 0,
                       nullptr) == DRS_ERR_INVALID);
    EXPECT(wkv_forward(F, F, F, F, nullptr, F, nullptr, 2, 1 << 16, 4096, 0, nullptr, 0, nullptr) != DRS_OK);
    EXPECT(wkv_backward(F, F, F, F, nullptr, F, nullptr, nullptr, F, F, nullptr, 2, 8, 64, 0, nullptr, 0,
                        nullptr) == DRS_ERR_INVALID);
    EXPECT(wkv_backward(F, F, reinterpret_cast<float *>(P1), F, nullptr, reinterpret_cast<float *>(P2), nullptr,
                        nullptr, reinterpret_cast<float *>(P3), reinterpret_cast<float *>(P4), nullptr, 2, 8, 64, 0,
                        nullptr, 0, nullptr) == DRS_ERR_WORKSPACE);
    EXPECT(wkv_backward(F, F, reinterpret_cast<float *>(P1), F, nullptr, reinterpret_cast<float *>(P2), nullptr,
                        nullptr, reinterpret_cast<float *>(P3), reinterpret_cast<float *>(P4),
                        reinterpret_cast<float *>(P3), 2, 8, 64, 0, nullptr, 0, nullptr) == DRS_ERR_INVALID);
    EXPECT(ema_forward(P1, P2, DRS_BF16, nullptr, P1, nullptr, 2, 8, 64, 0, nullptr, 0, nullptr) == DRS_ERR_INVALID);
    EXPECT(ema_forward(P1, P2, DRS_BF16, nullptr, P3, nullptr, 2, 8, 64, 0x2u, nullptr, 0, nullptr) ==
           DRS_ERR_INVALID);
    EXPECT(ema_bidirectional(P1, P2, DRS_BF16, P3, 2, 8, 64, 1u, nullptr, 0, nullptr) == DRS_ERR_INVALID);
    for (int s = -2; s < 8; ++s) EXPECT(drs_status_string(s) != nullptr);
    EXPECT(drs_version() > 0);
}

int main() {
    oracle_runs();
    abi_checks();
    if (failures) {
        std::printf("FAILED: %d checks\n", failures);
        return 1;
    }
    std::printf("sanitizer driver ok\n");
    return 0;
}
