// Host-side driver for the sanitizer tier: the fp64 oracle (oracle/linattn_ref.c)
// and the launch planner (sequence_mixing_amd/csrc/linattn_plan.cpp), built with
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py and
// run over small random and edge-case arguments.  Besides memory and UB errors,
// which the sanitizers report, it checks a few identities the two must keep;
// it exits non-zero on the first failure.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "linattn.h"
#include "linattn_plan.h"

extern "C" {
int linattn_ref_set_feature_map(int kind);
double linattn_ref_phi(double x);
double linattn_ref_dphi(double x);
int linattn_ref_fwd(const double *q, const double *k, const double *v, double *out, int B, int H, int Hkv, int N,
                    int d, int causal, int normalise, double *state_out, double *z_out, int nthreads);
int linattn_ref_fwd_from(const double *q, const double *k, const double *v, double *out, int B, int H, int Hkv, int N,
                         int d, int causal, int normalise, const double *state_in, const double *z_in,
                         double *state_out, double *z_out, int nthreads);
int linattn_ref_fwd_decay(const double *q, const double *k, const double *v, const double *g, double *out, int B,
                          int H, int Hkv, int N, int d, int normalise, const double *state_in, const double *z_in,
                          double *state_out, double *z_out, int nthreads);
int linattn_ref_decode_step(double *state, double *z, const double *q, const double *k, const double *v, double *out,
                            int B, int H, int Hkv, int d, int normalise);
int linattn_ref_decode_step_decay(double *state, double *z, const double *q, const double *k, const double *v,
                                  const double *g, double *out, int B, int H, int Hkv, int d, int normalise);
int linattn_ref_bwd(const double *q, const double *k, const double *v, const double *out, const double *dout,
                    double *dq, double *dk, double *dv, int B, int H, int Hkv, int N, int d, int causal,
                    int normalise, int nthreads);
}

namespace {

unsigned long long g_state = 12345;
double urand()  // uniform in [-2, 2): a plain 64-bit LCG, high bits
{
    g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
    return ((g_state >> 11) * (1.0 / 9007199254740992.0)) * 4.0 - 2.0;
}
// n random values; one spare element, so that an empty array still has a
// valid (non-null) address, as a caller's empty buffer would
std::vector<double> rnd(size_t n)
{
    std::vector<double> x(n + 1);
    for (auto &e : x) e = urand();
    return x;
}

int fails = 0;
void check(bool ok, const char *what)
{
    if (!ok) {
        fprintf(stderr, "FAIL: %s\n", what);
        ++fails;
    }
}

void oracle_cases()
{
    struct Shape {
        int B, H, Hkv, N, d;
    };
    const Shape shapes[] = {{1, 1, 1, 1, 1}, {1, 2, 1, 7, 3}, {2, 4, 2, 33, 16}, {1, 3, 3, 0, 8}, {0, 2, 2, 5, 4},
                            {2, 6, 3, 40, 32}, {1, 1, 1, 70, 64}};
    for (int fm = 0; fm < 3; ++fm) {
        check(linattn_ref_set_feature_map(fm) == 0, "feature map");
        for (const Shape &s : shapes) {
            const size_t nq = (size_t)s.B * s.H * s.N * s.d, nk = (size_t)s.B * s.Hkv * s.N * s.d;
            const size_t ns = (size_t)s.B * s.Hkv * s.d * s.d, nz = (size_t)s.B * s.Hkv * s.d;
            auto q = rnd(nq), k = rnd(nk), v = rnd(nk), dout = rnd(nq), g = rnd((size_t)s.B * s.Hkv * s.N);
            for (auto &e : g) e = -fabs(e);
            auto S0 = rnd(ns), z0 = rnd(nz);
            for (auto &e : z0) e = fabs(e) + 1.0;
            for (int causal = 0; causal < 2; ++causal) {
                for (int normalise = 0; normalise < 2; ++normalise) {
                    for (int nt : {1, 3}) {
                        std::vector<double> out(nq + 1), S(ns + 1), z(nz + 1), out2(nq + 1), dq(nq + 1),
                            dk(nk + 1), dv(nk + 1);
                        check(linattn_ref_fwd(q.data(), k.data(), v.data(), out.data(), s.B, s.H, s.Hkv, s.N, s.d,
                                              causal, normalise, S.data(), z.data(), nt) == 0, "fwd");
                        check(linattn_ref_fwd_from(q.data(), k.data(), v.data(), out2.data(), s.B, s.H, s.Hkv, s.N,
                                                   s.d, causal, normalise, S0.data(), z0.data(), nullptr, nullptr,
                                                   nt) == 0, "fwd_from");
                        check(linattn_ref_bwd(q.data(), k.data(), v.data(), out.data(), dout.data(), dq.data(),
                                              dk.data(), dv.data(), s.B, s.H, s.Hkv, s.N, s.d, causal, normalise,
                                              nt) == 0, "bwd");
                        if (causal)
                            check(linattn_ref_fwd_decay(q.data(), k.data(), v.data(), g.data(), out2.data(), s.B,
                                                        s.H, s.Hkv, s.N, s.d, normalise, nullptr, nullptr, S.data(),
                                                        z.data(), nt) == 0, "fwd_decay");
                    }
                }
            }
            // decode after prefill(N) equals row N of prefill(N + 1) (plain and decayed)
            if (s.B > 0 && s.N > 0) {
                const int N1 = s.N - 1;
                std::vector<double> q1((size_t)s.B * s.H * N1 * s.d + 1), k1((size_t)s.B * s.Hkv * N1 * s.d + 1),
                    v1(k1.size());
                for (int b = 0; b < s.B; ++b) {
                    for (int h = 0; h < s.H; ++h)
                        for (int t = 0; t < N1 * s.d; ++t)
                            q1[((size_t)b * s.H + h) * N1 * s.d + t] = q[((size_t)b * s.H + h) * s.N * s.d + t];
                    for (int h = 0; h < s.Hkv; ++h)
                        for (int t = 0; t < N1 * s.d; ++t) {
                            k1[((size_t)b * s.Hkv + h) * N1 * s.d + t] = k[((size_t)b * s.Hkv + h) * s.N * s.d + t];
                            v1[((size_t)b * s.Hkv + h) * N1 * s.d + t] = v[((size_t)b * s.Hkv + h) * s.N * s.d + t];
                        }
                }
                std::vector<double> full(nq + 1), pre(q1.size() + 1), S(ns + 1), z(nz + 1);
                linattn_ref_fwd(q.data(), k.data(), v.data(), full.data(), s.B, s.H, s.Hkv, s.N, s.d, 1, 1, nullptr,
                                nullptr, 2);
                linattn_ref_fwd(q1.data(), k1.data(), v1.data(), pre.data(), s.B, s.H, s.Hkv, N1, s.d, 1, 1, S.data(),
                                z.data(), 2);
                std::vector<double> qt((size_t)s.B * s.H * s.d), kt((size_t)s.B * s.Hkv * s.d), vt(kt.size()),
                    o(qt.size()), gz((size_t)s.B * s.Hkv, 0.0);
                for (int b = 0; b < s.B; ++b) {
                    for (int h = 0; h < s.H; ++h)
                        for (int i = 0; i < s.d; ++i)
                            qt[((size_t)b * s.H + h) * s.d + i] = q[(((size_t)b * s.H + h) * s.N + N1) * s.d + i];
                    for (int h = 0; h < s.Hkv; ++h)
                        for (int i = 0; i < s.d; ++i) {
                            kt[((size_t)b * s.Hkv + h) * s.d + i] = k[(((size_t)b * s.Hkv + h) * s.N + N1) * s.d + i];
                            vt[((size_t)b * s.Hkv + h) * s.d + i] = v[(((size_t)b * s.Hkv + h) * s.N + N1) * s.d + i];
                        }
                }
                std::vector<double> S2 = S, z2 = z, o2(o.size());
                check(linattn_ref_decode_step(S.data(), z.data(), qt.data(), kt.data(), vt.data(), o.data(), s.B, s.H,
                                              s.Hkv, s.d, 1) == 0, "decode");
                check(linattn_ref_decode_step_decay(S2.data(), z2.data(), qt.data(), kt.data(), vt.data(), gz.data(),
                                                    o2.data(), s.B, s.H, s.Hkv, s.d, 1) == 0, "decode decay");
                double worst = 0.0;
                for (int b = 0; b < s.B; ++b)
                    for (int h = 0; h < s.H; ++h)
                        for (int i = 0; i < s.d; ++i) {
                            const double r = full[(((size_t)b * s.H + h) * s.N + N1) * s.d + i];
                            worst = fmax(worst, fabs(o[((size_t)b * s.H + h) * s.d + i] - r) / (1.0 + fabs(r)));
                            worst = fmax(worst, fabs(o2[((size_t)b * s.H + h) * s.d + i] - r) / (1.0 + fabs(r)));
                        }
                check(worst < 1e-12, "decode after prefill equals the next prefill row");
            }
        }
    }
    linattn_ref_set_feature_map(0);
    // invalid arguments are refused, nothing read
    double x = 0.0;
    check(linattn_ref_fwd(nullptr, &x, &x, &x, 1, 1, 1, 1, 1, 1, 1, nullptr, nullptr, 1) == -1, "null q refused");
    check(linattn_ref_fwd(&x, &x, &x, &x, 1, 3, 2, 1, 1, 1, 1, nullptr, nullptr, 1) == -1, "H % Hkv refused");
    check(linattn_ref_decode_step(&x, nullptr, &x, &x, &x, &x, 1, 1, 1, 1, 1) == -1, "decode without z refused");
    check(linattn_ref_set_feature_map(7) != 0, "unknown feature map refused");
    // phi and phi' at edge values
    const double edge[] = {-1e308, -745.0, -1.0, -0.0, 0.0, 1e-300, 1.0, 700.0, 1e308};
    for (int fm = 0; fm < 3; ++fm) {
        linattn_ref_set_feature_map(fm);
        for (double e : edge) {
            const double p = linattn_ref_phi(e), dp = linattn_ref_dphi(e);
            check(p >= 0.0 && dp >= 0.0, "phi, phi' non-negative");
        }
    }
    linattn_ref_set_feature_map(0);
}

void plan_cases()
{
    const int dtypes[] = {LINATTN_F32, LINATTN_BF16, LINATTN_F16, LINATTN_DTYPE(LINATTN_BF16, LINATTN_PHI_RELU),
                          LINATTN_DTYPE(LINATTN_F32, LINATTN_PHI_SOFTPLUS), -1, 3, 1 << 9};
    const int ds[] = {0, 16, 32, 64, 96, 128, 256};
    const int chunks[] = {0, 16, 32, 64, 128, 256, 512};
    const int Ns[] = {-1, 0, 1, 31, 257, 4096, 65537, 1 << 22, 1 << 28};
    const int heads[][3] = {{1, 1, 1}, {2, 8, 8}, {1, 32, 8}, {3, 6, 2}, {1, 5, 3}, {0, 4, 4}, {64, 1, 1},
                            {1 << 20, 2, 2}, {-1, 1, 1}, {1, 0, 1}};
    long planned = 0;
    for (int dt : dtypes)
        for (int d : ds)
            for (int c : chunks)
                for (int N : Ns)
                    for (const auto &hh : heads)
                        for (int causal = 0; causal < 2; ++causal) {
                            linattn::Plan p;
                            const int rc = linattn::make_plan(hh[0], hh[1], hh[2], N, d, causal, dt, c, &p);
                            if (rc == LINATTN_OK) {
                                ++planned;
                                check(p.nseq == hh[0] * hh[2], "plan nseq");
                                if (hh[0] > 0 && N > 0) {
                                    check(p.segments >= 1 && p.seg_len % p.chunk == 0, "segments of whole chunks");
                                    check((long long)(p.segments - 1) * p.seg_len < N &&
                                              (long long)p.segments * p.seg_len >= N, "segments cover N");
                                }
                                if (causal) {
                                    (void)linattn::decay_ok(p);
                                    (void)linattn::decay_ws_bytes(p);
                                }
                            }
                            linattn::Plan pk;
                            (void)linattn::make_plan_packed(hh[0], hh[1], hh[2], N, d, causal, dt, c, &pk);
                        }
    check(planned > 1000, "some plans accepted");
    for (int G = 1; G <= 16; ++G)
        for (int d : {32, 64, 128})
            for (int dt : {LINATTN_F32, LINATTN_BF16}) {
                (void)linattn::heads_per_block(dt, d, 64, G);
                (void)linattn::auto_chunk(dt, d, G, 1);
            }
}

}  // namespace

int main()
{
    oracle_cases();
    plan_cases();
    if (fails) {
        fprintf(stderr, "%d failures\n", fails);
        return 1;
    }
    printf("sanitized oracle and planner: ok\n");
    return 0;
}
