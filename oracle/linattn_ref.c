/*
 * linattn_ref.c - fp64 CPU oracle for linear attention with the feature map
 * phi(x) = ELU(x) + 1.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plainly written checker
 * that the GPU library is compared against.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or helper with the HIP library, and nothing in the library
 * may call it.
 *
 * What it computes (source: the LinearTile 1.0.0 README on PyPI, section
 * "How It Works", and the paper it cites there, Katharopoulos et al. 2020,
 * "Transformers are RNNs"):
 *   - attention output O = phi(Q) (phi(K)^T V), i.e. the key/value product is
 *     formed first and then applied to the queries;
 *   - phi(x) = ELU(x) + 1 with the usual alpha = 1, so phi(x) = x + 1 for
 *     x > 0 and exp(x) otherwise (always positive); ReLU and softplus may be
 *     selected instead (README "Features", custom kernel plugins);
 *   - causal form (README "Features" list, the causal-masking item): query t
 *     only sees keys s <= t.  Written as a running state
 *         S_t = sum_{s<=t} phi(k_s) v_s^T   (d x d)
 *         z_t = sum_{s<=t} phi(k_s)         (d)
 *         o_t = phi(q_t)^T S_t / (phi(q_t) . z_t)   (normalised)
 *         o_t = phi(q_t)^T S_t                      (normalise == 0)
 *   - non-causal form: S and z summed over the whole sequence, then applied
 *     to every query;
 *   - grouped-query attention (README "Features" list, the GQA item): query
 *     head h reads key/value head floor(h / (H / Hkv)).
 *   - decode: one token appended to a carried (S, z); the state is updated
 *     first and then read, so the new token sees itself (s <= t).
 *   - continuation (README "Features", the KV-cache-reuse item: a prompt's
 *     state carried into later tokens): the same forward pass with S and z
 *     starting from given sums of earlier tokens instead of zero.
 *   - decayed state (a reading: the pages define decay only for the scan of
 *     the Stream efficiency essay, section 4.2, h_t = h_{t-1} a_t + b_t; for
 *     linear attention the running sums take the same form): with a log-decay
 *     g_t per (batch, kv head, token) and a_t = exp(g_t),
 *         S_t = a_t S_{t-1} + phi(k_t) v_t^T,   z_t = a_t z_{t-1} + phi(k_t),
 *     and o_t as above; causal only (linattn_ref_fwd_decay); decode likewise
 *     (linattn_ref_decode_step_decay).  g = 0 everywhere is the plain form.
 *   - sliding window (a reading of the README's "Features" list, the
 *     sliding-window item, which gives no definition): query t sees the keys
 *     of the band t - W < s <= t only,
 *         o_t = sum_{band} (phi(q_t) . phi(k_s)) v_s / sum_{band} phi(q_t) . phi(k_s)
 *     (numerator only when normalise == 0), written out per query as that
 *     sum (linattn_ref_fwd_window); W >= N is the causal form.
 *   - backward (the README's project layout names a backward module and its
 *     test without their content; the Stream efficiency essay, section 4.2,
 *     gives the pattern of a running-sum recurrence differentiated by a
 *     reverse-time scan): dQ, dK, dV of the forward above for a given output
 *     gradient dO, by the chain rule, written out at linattn_ref_bwd.
 *
 * Readings where the pages are silent: no 1/sqrt(d) scale, no epsilon in the
 * denominator, d_k = d_v = d, layouts q/out [B][H][N][d], k/v [B][Hkv][N][d],
 * state [B][Hkv][d][d] with S[i][j] = sum phi(k)_i v_j, z [B][Hkv][d].
 *
 * Everything is double precision and follows the recurrence one token at a
 * time; no blocking, no reordering beyond the definition above.  Threads
 * split the work over independent (batch, kv head, 16-wide value-column
 * block) items only; each item runs the plain recurrence for its columns.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define REF_COLBLOCK 16

/*
 * The feature map (README "Features", custom kernel plugins: phi can be
 * replaced).  0: ELU(x) + 1 with alpha = 1, the README's phi; 1: ReLU(x);
 * 2: softplus(x) = log(1 + e^x).  Selected for every later call with
 * linattn_ref_set_feature_map (the checker is driven from one thread).
 */
static int g_feature_map = 0;

int linattn_ref_set_feature_map(int kind)
{
    if (kind < 0 || kind > 2) return -1;
    g_feature_map = kind;
    return 0;
}

double linattn_ref_phi(double x)
{
    /* ReLU keeps a NaN input (non-finite inputs propagate through every map) */
    if (g_feature_map == 1) return x > 0.0 || x != x ? x : 0.0;
    if (g_feature_map == 2) return x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
    return x > 0.0 ? x + 1.0 : exp(x);
}

typedef struct {
    const double *q, *k, *v;
    const double *state_in, *z_in; /* starting sums, or NULL for zero */
    const double *g;               /* log-decay [B][Hkv][N], or NULL for none (causal only) */
    double *out, *state_out, *z_out;
    int B, H, Hkv, N, d, causal, normalise;
    int nitems, nthreads, tid;
} fwd_job;

/* One item: batch b, kv head g, value columns [j0, j0 + w). */
static void fwd_item(const fwd_job *J, int item)
{
    const int d = J->d, N = J->N, G = J->H / J->Hkv;
    const int ncb = (d + REF_COLBLOCK - 1) / REF_COLBLOCK;
    const int b = item / (J->Hkv * ncb);
    const int g = (item / ncb) % J->Hkv;
    const int j0 = (item % ncb) * REF_COLBLOCK;
    const int w = (d - j0) < REF_COLBLOCK ? (d - j0) : REF_COLBLOCK;

    double *S = calloc((size_t)d * w, sizeof(double)); /* S[i][jj] */
    double *z = calloc((size_t)d, sizeof(double));
    if (J->state_in) {
        const double *si = J->state_in + ((size_t)b * J->Hkv + g) * (size_t)d * d;
        for (int i = 0; i < d; ++i)
            for (int jj = 0; jj < w; ++jj) S[(size_t)i * w + jj] = si[(size_t)i * d + j0 + jj];
    }
    if (J->z_in) {
        const double *zi = J->z_in + ((size_t)b * J->Hkv + g) * (size_t)d;
        for (int i = 0; i < d; ++i) z[i] = zi[i];
    }
    double *f = malloc((size_t)d * sizeof(double));
    double *p = malloc((size_t)d * sizeof(double));

    const double *kb = J->k + ((size_t)b * J->Hkv + g) * (size_t)N * d;
    const double *vb = J->v + ((size_t)b * J->Hkv + g) * (size_t)N * d;

    if (!J->causal) {
        /* Pass over all keys first: S = sum_t phi(k_t) v_t^T, z = sum_t phi(k_t). */
        for (int t = 0; t < N; ++t) {
            for (int i = 0; i < d; ++i) f[i] = linattn_ref_phi(kb[(size_t)t * d + i]);
            for (int i = 0; i < d; ++i) {
                for (int jj = 0; jj < w; ++jj) S[(size_t)i * w + jj] += f[i] * vb[(size_t)t * d + j0 + jj];
                z[i] += f[i];
            }
        }
    }

    const double *gb = J->g ? J->g + ((size_t)b * J->Hkv + g) * (size_t)N : NULL;
    for (int t = 0; t < N; ++t) {
        if (J->causal) {
            /* Decay the sums of the earlier tokens by a_t = exp(g_t). */
            if (gb) {
                const double a = exp(gb[t]);
                for (int i = 0; i < d; ++i) {
                    for (int jj = 0; jj < w; ++jj) S[(size_t)i * w + jj] *= a;
                    z[i] *= a;
                }
            }
            /* Absorb token t before reading: query t sees keys s <= t. */
            for (int i = 0; i < d; ++i) f[i] = linattn_ref_phi(kb[(size_t)t * d + i]);
            for (int i = 0; i < d; ++i) {
                for (int jj = 0; jj < w; ++jj) S[(size_t)i * w + jj] += f[i] * vb[(size_t)t * d + j0 + jj];
                z[i] += f[i];
            }
        }
        for (int h = g * G; h < (g + 1) * G; ++h) {
            const double *qt = J->q + (((size_t)b * J->H + h) * N + t) * d;
            double *ot = J->out + (((size_t)b * J->H + h) * N + t) * d;
            for (int i = 0; i < d; ++i) p[i] = linattn_ref_phi(qt[i]);
            double den = 0.0;
            for (int i = 0; i < d; ++i) den += p[i] * z[i];
            for (int jj = 0; jj < w; ++jj) {
                double num = 0.0;
                for (int i = 0; i < d; ++i) num += p[i] * S[(size_t)i * w + jj];
                ot[j0 + jj] = J->normalise ? num / den : num;
            }
        }
    }

    if (J->state_out) {
        double *so = J->state_out + ((size_t)b * J->Hkv + g) * (size_t)d * d;
        for (int i = 0; i < d; ++i)
            for (int jj = 0; jj < w; ++jj) so[(size_t)i * d + j0 + jj] = S[(size_t)i * w + jj];
    }
    if (J->z_out && j0 == 0) {
        double *zo = J->z_out + ((size_t)b * J->Hkv + g) * (size_t)d;
        for (int i = 0; i < d; ++i) zo[i] = z[i];
    }
    free(S);
    free(z);
    free(f);
    free(p);
}

static void *fwd_worker(void *arg)
{
    const fwd_job *J = (const fwd_job *)arg;
    for (int item = J->tid; item < J->nitems; item += J->nthreads) fwd_item(J, item);
    return NULL;
}

/*
 * Forward pass continuing from state_in [B][Hkv][d][d] and z_in [B][Hkv][d]
 * (either may be NULL for zero).  All arrays are contiguous fp64 host arrays
 * in the layouts given above.  state_out / z_out may be NULL.  Returns 0, or
 * -1 on invalid arguments (nothing is written then).
 */
static int fwd_run(const double *q, const double *k, const double *v, const double *g, double *out,
                   int B, int H, int Hkv, int N, int d, int causal, int normalise,
                   const double *state_in, const double *z_in,
                   double *state_out, double *z_out, int nthreads)
{
    if (!q || !k || !v || !out) return -1;
    if (g && !causal) return -1;
    if (B < 0 || H <= 0 || Hkv <= 0 || N < 0 || d <= 0 || H % Hkv != 0) return -1;
    if (B == 0) return 0;
    const int ncb = (d + REF_COLBLOCK - 1) / REF_COLBLOCK;
    const int nitems = B * Hkv * ncb;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nitems) nthreads = nitems;

    fwd_job *jobs = malloc((size_t)nthreads * sizeof(fwd_job));
    pthread_t *th = malloc((size_t)nthreads * sizeof(pthread_t));
    for (int t = 0; t < nthreads; ++t) {
        fwd_job J = {q, k, v, state_in, z_in, g, out, state_out, z_out, B, H, Hkv, N, d, causal, normalise,
                     nitems, nthreads, t};
        jobs[t] = J;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, fwd_worker, &jobs[t]);
    fwd_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(jobs);
    free(th);
    return 0;
}

int linattn_ref_fwd_from(const double *q, const double *k, const double *v, double *out,
                         int B, int H, int Hkv, int N, int d, int causal, int normalise,
                         const double *state_in, const double *z_in,
                         double *state_out, double *z_out, int nthreads)
{
    return fwd_run(q, k, v, NULL, out, B, H, Hkv, N, d, causal, normalise, state_in, z_in, state_out, z_out,
                   nthreads);
}

/*
 * Causal forward pass with decayed sums: g [B][Hkv][N] holds the log-decay
 * of every token (a_t = exp(g_t) multiplies S and z before token t is
 * added).  Other arguments as linattn_ref_fwd_from.
 */
int linattn_ref_fwd_decay(const double *q, const double *k, const double *v, const double *g, double *out,
                          int B, int H, int Hkv, int N, int d, int normalise,
                          const double *state_in, const double *z_in,
                          double *state_out, double *z_out, int nthreads)
{
    if (!g) return -1;
    return fwd_run(q, k, v, g, out, B, H, Hkv, N, d, 1, normalise, state_in, z_in, state_out, z_out, nthreads);
}

/* Forward pass from zero sums (see linattn_ref_fwd_from). */
int linattn_ref_fwd(const double *q, const double *k, const double *v, double *out,
                    int B, int H, int Hkv, int N, int d, int causal, int normalise,
                    double *state_out, double *z_out, int nthreads)
{
    return linattn_ref_fwd_from(q, k, v, out, B, H, Hkv, N, d, causal, normalise, NULL, NULL, state_out, z_out,
                                nthreads);
}

/*
 * One decode step for a batch of B sequences, each with Hkv carried states.
 * state [B][Hkv][d][d] and z [B][Hkv][d] are updated in place (z may be NULL
 * when normalise == 0).  q/out are [B][H][d], k/v are [B][Hkv][d].
 * The state absorbs (k, v) first, then every query head of the group reads it.
 */
static int decode_run(double *state, double *z, const double *q, const double *k,
                      const double *v, const double *gd, double *out, int B, int H, int Hkv, int d,
                      int normalise)
{
    if (!state || !q || !k || !v || !out) return -1;
    if (normalise && !z) return -1;
    if (B < 0 || H <= 0 || Hkv <= 0 || d <= 0 || H % Hkv != 0) return -1;
    const int G = H / Hkv;
    double *f = malloc((size_t)d * sizeof(double));
    double *p = malloc((size_t)d * sizeof(double));
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            double *S = state + ((size_t)b * Hkv + g) * (size_t)d * d;
            double *zz = z ? z + ((size_t)b * Hkv + g) * (size_t)d : NULL;
            const double *kt = k + ((size_t)b * Hkv + g) * (size_t)d;
            const double *vt = v + ((size_t)b * Hkv + g) * (size_t)d;
            if (gd) {
                const double a = exp(gd[(size_t)b * Hkv + g]);
                for (int i = 0; i < d; ++i) {
                    for (int j = 0; j < d; ++j) S[(size_t)i * d + j] *= a;
                    if (zz) zz[i] *= a;
                }
            }
            for (int i = 0; i < d; ++i) f[i] = linattn_ref_phi(kt[i]);
            for (int i = 0; i < d; ++i) {
                for (int j = 0; j < d; ++j) S[(size_t)i * d + j] += f[i] * vt[j];
                if (zz) zz[i] += f[i];
            }
            for (int h = g * G; h < (g + 1) * G; ++h) {
                const double *qt = q + ((size_t)b * H + h) * (size_t)d;
                double *ot = out + ((size_t)b * H + h) * (size_t)d;
                for (int i = 0; i < d; ++i) p[i] = linattn_ref_phi(qt[i]);
                double den = 0.0;
                if (normalise)
                    for (int i = 0; i < d; ++i) den += p[i] * zz[i];
                for (int j = 0; j < d; ++j) {
                    double num = 0.0;
                    for (int i = 0; i < d; ++i) num += p[i] * S[(size_t)i * d + j];
                    ot[j] = normalise ? num / den : num;
                }
            }
        }
    }
    free(f);
    free(p);
    return 0;
}

int linattn_ref_decode_step(double *state, double *z, const double *q, const double *k,
                            const double *v, double *out, int B, int H, int Hkv, int d,
                            int normalise)
{
    return decode_run(state, z, q, k, v, NULL, out, B, H, Hkv, d, normalise);
}

/* One decode step with decayed sums: g [B][Hkv] is this token's log-decay;
 * S and z are multiplied by exp(g) before the token is added. */
int linattn_ref_decode_step_decay(double *state, double *z, const double *q, const double *k,
                                  const double *v, const double *g, double *out, int B, int H, int Hkv, int d,
                                  int normalise)
{
    if (!g) return -1;
    return decode_run(state, z, q, k, v, g, out, B, H, Hkv, d, normalise);
}

/* d phi / dx.  ELU + 1: 1 for x > 0, exp(x) otherwise (both sides give 1 at
 * 0); ReLU: 1 for x > 0, else 0; softplus: the logistic function. */
double linattn_ref_dphi(double x)
{
    if (g_feature_map == 1) return x > 0.0 ? 1.0 : (x != x ? x : 0.0);
    if (g_feature_map == 2) return 1.0 / (1.0 + exp(-x));
    return x > 0.0 ? 1.0 : exp(x);
}

typedef struct {
    const double *q, *k, *v, *out, *dout;
    double *dq, *dk, *dv;
    int B, H, Hkv, N, d, causal, normalise;
    int nitems, nthreads, tid;
} bwd_job;

/*
 * One item: batch b, kv head g with its G query heads.
 *
 * With a_t = phi(q_t), b_s = phi(k_s) and, for the normalised output
 * o_t = num_t / den_t (num_t = S_t^T a_t, den_t = a_t . z_t), the loss
 * gradient dO_t enters through
 *     g_t = dO_t / den_t              (gradient of num_t)
 *     h_t = -(dO_t . o_t) / den_t     (gradient of den_t)
 * (normalise == 0: g_t = dO_t, h_t = 0).  Then, with "t sees s" meaning
 * s <= t (causal) or every pair (non-causal):
 *     da_t = S_t g_t + h_t z_t                       (S_t, z_t as seen by t)
 *     dv_s = sum_{t sees s} (a_t . b_s) g_t     = R_s^T b_s
 *     db_s = sum_{t sees s} (g_t . v_s + h_t) a_t = R_s v_s + r_s
 * where R_s = sum_{t sees s} a_t g_t^T and r_s = sum_{t sees s} h_t a_t,
 * summed over the G query heads of the group as well.  Finally
 * dq = da * phi'(q), dk = db * phi'(k).  The forward walk gives da (and g,
 * h, which it keeps); a reverse walk accumulates R, r for dk and dv.
 */
static void bwd_item(const bwd_job *J, int item)
{
    const int d = J->d, N = J->N, G = J->H / J->Hkv;
    const int b = item / J->Hkv, g = item % J->Hkv;
    double *S = calloc((size_t)d * d, sizeof(double));
    double *z = calloc((size_t)d, sizeof(double));
    double *R = calloc((size_t)d * d, sizeof(double));
    double *r = calloc((size_t)d, sizeof(double));
    double *f = malloc((size_t)d * sizeof(double));
    double *p = malloc((size_t)d * sizeof(double));
    double *gs = malloc((size_t)G * N * d * sizeof(double) + 1);
    double *hs = malloc((size_t)G * N * sizeof(double) + 1);

    const double *kb = J->k + ((size_t)b * J->Hkv + g) * (size_t)N * d;
    const double *vb = J->v + ((size_t)b * J->Hkv + g) * (size_t)N * d;
    double *dkb = J->dk + ((size_t)b * J->Hkv + g) * (size_t)N * d;
    double *dvb = J->dv + ((size_t)b * J->Hkv + g) * (size_t)N * d;
#define ROW(base, hh, t) ((base) + (((size_t)b * J->H + (hh)) * N + (t)) * d)

    /* absorb key t into (S, z) */
#define ABSORB(t)                                                                                          \
    do {                                                                                                   \
        for (int i = 0; i < d; ++i) f[i] = linattn_ref_phi(kb[(size_t)(t) * d + i]);                     \
        for (int i = 0; i < d; ++i) {                                                                      \
            for (int j = 0; j < d; ++j) S[(size_t)i * d + j] += f[i] * vb[(size_t)(t) * d + j];          \
            z[i] += f[i];                                                                                  \
        }                                                                                                  \
    } while (0)

    if (!J->causal)
        for (int t = 0; t < N; ++t) ABSORB(t);
    /* forward walk: den, g, h and dq */
    for (int t = 0; t < N; ++t) {
        if (J->causal) ABSORB(t);
        for (int hh = 0; hh < G; ++hh) {
            const int h = g * G + hh;
            const double *qt = ROW(J->q, h, t), *dot = ROW(J->dout, h, t);
            double *gt = gs + ((size_t)hh * N + t) * d;
            for (int i = 0; i < d; ++i) p[i] = linattn_ref_phi(qt[i]);
            double hval = 0.0;
            if (J->normalise) {
                const double *ot = ROW(J->out, h, t);
                double den = 0.0, dov = 0.0;
                for (int i = 0; i < d; ++i) den += p[i] * z[i];
                for (int j = 0; j < d; ++j) dov += dot[j] * ot[j];
                for (int j = 0; j < d; ++j) gt[j] = dot[j] / den;
                hval = -dov / den;
            } else {
                for (int j = 0; j < d; ++j) gt[j] = dot[j];
            }
            hs[(size_t)hh * N + t] = hval;
            double *dqt = ROW(J->dq, h, t);
            for (int i = 0; i < d; ++i) {
                double da = hval * z[i];
                for (int j = 0; j < d; ++j) da += S[(size_t)i * d + j] * gt[j];
                dqt[i] = da * linattn_ref_dphi(qt[i]);
            }
        }
    }
#undef ABSORB

    /* gather every query of the group into (R, r) */
#define GATHER(t)                                                                                          \
    do {                                                                                                   \
        for (int hh = 0; hh < G; ++hh) {                                                                   \
            const double *qt = ROW(J->q, g * G + hh, (t));                                                 \
            const double *gt = gs + ((size_t)hh * N + (t)) * d;                                            \
            const double hval = hs[(size_t)hh * N + (t)];                                                  \
            for (int i = 0; i < d; ++i) p[i] = linattn_ref_phi(qt[i]);                                     \
            for (int i = 0; i < d; ++i) {                                                                  \
                for (int j = 0; j < d; ++j) R[(size_t)i * d + j] += p[i] * gt[j];                          \
                r[i] += hval * p[i];                                                                       \
            }                                                                                              \
        }                                                                                                  \
    } while (0)

    if (!J->causal)
        for (int t = 0; t < N; ++t) GATHER(t);
    /* reverse walk: key s is seen by queries t >= s */
    for (int s = N - 1; s >= 0; --s) {
        if (J->causal) GATHER(s);
        const double *ks = kb + (size_t)s * d, *vs = vb + (size_t)s * d;
        for (int i = 0; i < d; ++i) f[i] = linattn_ref_phi(ks[i]);
        for (int j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += R[(size_t)i * d + j] * f[i];
            dvb[(size_t)s * d + j] = acc;
        }
        for (int i = 0; i < d; ++i) {
            double acc = r[i];
            for (int j = 0; j < d; ++j) acc += R[(size_t)i * d + j] * vs[j];
            dkb[(size_t)s * d + i] = acc * linattn_ref_dphi(ks[i]);
        }
    }
#undef GATHER
#undef ROW
    free(S);
    free(z);
    free(R);
    free(r);
    free(f);
    free(p);
    free(gs);
    free(hs);
}

static void *bwd_worker(void *arg)
{
    const bwd_job *J = (const bwd_job *)arg;
    for (int item = J->tid; item < J->nitems; item += J->nthreads) bwd_item(J, item);
    return NULL;
}

/*
 * Backward pass: dq [B][H][N][d], dk and dv [B][Hkv][N][d] for the output
 * gradient dout [B][H][N][d].  out is the forward output (the normalised
 * gradient uses dO . o); it may be NULL when normalise == 0.  Returns 0, or
 * -1 on invalid arguments.
 */
int linattn_ref_bwd(const double *q, const double *k, const double *v, const double *out,
                    const double *dout, double *dq, double *dk, double *dv,
                    int B, int H, int Hkv, int N, int d, int causal, int normalise, int nthreads)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || (normalise && !out)) return -1;
    if (B < 0 || H <= 0 || Hkv <= 0 || N < 0 || d <= 0 || H % Hkv != 0) return -1;
    if (B == 0 || N == 0) return 0;
    const int nitems = B * Hkv;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nitems) nthreads = nitems;
    bwd_job *jobs = malloc((size_t)nthreads * sizeof(bwd_job));
    pthread_t *th = malloc((size_t)nthreads * sizeof(pthread_t));
    for (int t = 0; t < nthreads; ++t) {
        bwd_job J = {q, k, v, out, dout, dq, dk, dv, B, H, Hkv, N, d, causal, normalise, nitems, nthreads, t};
        jobs[t] = J;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, bwd_worker, &jobs[t]);
    bwd_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(jobs);
    free(th);
    return 0;
}

/*
 * Sliding-window forward pass (causal band of W keys): for every batch b,
 * query head h and token t, with g = h / (H / Hkv),
 *     num = sum_{s = max(0, t-W+1)}^{t} (phi(q_t) . phi(k_s)) v_s,
 *     den = sum over the same s of phi(q_t) . phi(k_s),
 *     out = num / den   (or num when normalise == 0).
 * The band's sum is formed directly for each query (no running state), one
 * key at a time.  Threads split the (batch, query head) pairs.  Returns 0, or
 * -1 on invalid arguments (W < 1 included).
 */
typedef struct {
    const double *q, *k, *v;
    double *out;
    int B, H, Hkv, N, d, W, normalise, nthreads, tid;
} win_job;

static void *win_worker(void *arg)
{
    const win_job *J = (const win_job *)arg;
    const int d = J->d, N = J->N, G = J->H / J->Hkv;
    double *pq = malloc((size_t)d * sizeof(double));
    double *pk = malloc((size_t)d * sizeof(double));
    double *num = malloc((size_t)d * sizeof(double));
    for (int item = J->tid; item < J->B * J->H; item += J->nthreads) {
        const int b = item / J->H, h = item % J->H, g = h / G;
        for (int t = 0; t < N; ++t) {
            const double *qt = J->q + (((size_t)b * J->H + h) * N + t) * d;
            for (int i = 0; i < d; ++i) pq[i] = linattn_ref_phi(qt[i]);
            for (int j = 0; j < d; ++j) num[j] = 0.0;
            double den = 0.0;
            const int s0 = t - J->W + 1 > 0 ? t - J->W + 1 : 0;
            for (int s = s0; s <= t; ++s) {
                const double *ks = J->k + (((size_t)b * J->Hkv + g) * N + s) * d;
                const double *vs = J->v + (((size_t)b * J->Hkv + g) * N + s) * d;
                for (int i = 0; i < d; ++i) pk[i] = linattn_ref_phi(ks[i]);
                double a = 0.0;
                for (int i = 0; i < d; ++i) a += pq[i] * pk[i];
                for (int j = 0; j < d; ++j) num[j] += a * vs[j];
                den += a;
            }
            double *ot = J->out + (((size_t)b * J->H + h) * N + t) * d;
            for (int j = 0; j < d; ++j) ot[j] = J->normalise ? num[j] / den : num[j];
        }
    }
    free(pq);
    free(pk);
    free(num);
    return NULL;
}

int linattn_ref_fwd_window(const double *q, const double *k, const double *v, double *out,
                           int B, int H, int Hkv, int N, int d, int W, int normalise, int nthreads)
{
    if (!q || !k || !v || !out) return -1;
    if (B < 0 || H <= 0 || Hkv <= 0 || N < 0 || d <= 0 || H % Hkv != 0 || W < 1) return -1;
    if (B == 0 || N == 0) return 0;
    const int nitems = B * H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nitems) nthreads = nitems;
    win_job *jobs = malloc((size_t)nthreads * sizeof(win_job));
    pthread_t *th = malloc((size_t)nthreads * sizeof(pthread_t));
    for (int t = 0; t < nthreads; ++t) {
        win_job J = {q, k, v, out, B, H, Hkv, N, d, W, normalise, nthreads, t};
        jobs[t] = J;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, win_worker, &jobs[t]);
    win_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(jobs);
    free(th);
    return 0;
}
