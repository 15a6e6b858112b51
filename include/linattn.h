/*
 * linattn.h - C ABI of liblinattn.so: linear attention with the feature map
 * phi(x) = ELU(x) + 1 on AMD Instinct MI355X (gfx950).
 *
 * Method (LinearTile 1.0.0 README on PyPI, section "How It Works"): the
 * attention output is O = phi(Q) (phi(K)^T V) with phi(x) = ELU(x) + 1
 * (alpha = 1, so phi(x) = x + 1 for x > 0 and exp(x) otherwise).  The causal
 * form (README "Features" list, causal-masking item; Katharopoulos et al. 2020,
 * "Transformers are RNNs", cited under the README's "Reference" section) is
 * the running state
 *     S_t = sum_{s<=t} phi(k_s) v_s^T,   z_t = sum_{s<=t} phi(k_s),
 *     o_t = phi(q_t)^T S_t / (phi(q_t) . z_t)      (normalise = 1)
 *     o_t = phi(q_t)^T S_t                         (normalise = 0)
 * No 1/sqrt(d) scale and no epsilon are applied.  Grouped-query attention
 * (README "Features" list, GQA item): query head h reads key/value head
 * floor(h / (H / Hkv)).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or synchronises; it keeps no state
 *     between calls and is reentrant.
 *   - Work is enqueued on `stream` (a hipStream_t; 0 = the null stream) and
 *     the call returns after enqueueing.  Buffers must stay alive until the
 *     stream has passed that point.
 *   - Layouts are dense row-major: q and out [B][H][N][d]; k and v
 *     [B][Hkv][N][d]; a state S [B][Hkv][d][d] with S[i][j] = sum phi(k)_i v_j;
 *     a normaliser z [B][Hkv][d].
 *   - q, k, v and out share `dtype` (LINATTN_F32, LINATTN_BF16 or
 *     LINATTN_F16; README "Features": mixed precision), except that fp8 rows
 *     (LINATTN_FP8_E4M3, LINATTN_FP8_E5M2: the OCP 8-bit formats, E4M3 with
 *     no infinities and largest value 448, E5M2 IEEE-like) are inputs only:
 *     with an fp8 dtype, q, k and v are fp8 and out is bf16.  fp8 rows are
 *     taken by linattn_fwd, linattn_fwd_from_state, linattn_fwd_packed,
 *     linattn_fwd_noalloc, linattn_fwd_window and linattn_decode_step (the
 *     backward and the decayed sums return LINATTN_ERR_UNSUPPORTED).  Arithmetic
 *     accumulates in fp32 and the state is always fp32.  fp16 rows are read
 *     and written as fp16 and enter the matrix cores as bf16, like bf16 rows
 *     (bf16 keeps fp32's exponent range, so the operand copies of the running
 *     sums, which grow with the sequence, cannot overflow as fp16 would); fp8
 *     rows likewise, widened exactly to bf16 when staged.  The output is
 *     rounded once, to nearest even, when stored.
 *   - Supported: d in {32, 64, 128}; H % Hkv == 0; every pointer 16-byte
 *     aligned; out must not alias q, k or v.
 *   - Errors: arguments are checked before anything is enqueued; a negative
 *     LINATTN_ERR_* code is returned and nothing is launched.  A failed
 *     kernel launch returns LINATTN_ERR_HIP.  The library never prints,
 *     aborts or throws.  NaN / Inf inputs are not checked and propagate: a
 *     non-finite query spoils its own row; a non-finite key or value at
 *     token s spoils the causal rows from s on (all rows when non-causal).
 *     Rows before s stay finite, except that a non-finite VALUE may also
 *     spoil the rows of its own 32-token tile (its pair of tiles, for chunk
 *     kernels that keep one state copy per pair) that come before it: the
 *     tile's values are multiplied by the masked (zero) scores.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LINATTN_ABI_VERSION 12

enum { LINATTN_F32 = 0, LINATTN_BF16 = 1, LINATTN_F16 = 2, LINATTN_FP8_E4M3 = 3, LINATTN_FP8_E5M2 = 4 };
/* Feature maps phi (README "Features": custom kernel plugins, phi
 * replaceable): ELU(x) + 1 (the README's, the default), ReLU(x) (a normalised
 * row whose query or keys are all <= 0 divides by zero), softplus(x) =
 * log(1 + e^x).  Every `dtype` argument below carries the element type in
 * bits 0-7 and the feature map in bits 8-15: LINATTN_DTYPE(elem, phi). */
enum { LINATTN_PHI_ELU1 = 0, LINATTN_PHI_RELU = 1, LINATTN_PHI_SOFTPLUS = 2 };
#define LINATTN_DTYPE(elem, phi) ((elem) | ((phi) << 8))

enum {
    LINATTN_OK = 0,
    LINATTN_ERR_NULL = -1,        /* a required pointer is NULL                       */
    LINATTN_ERR_SHAPE = -2,       /* B, H, Hkv, N or d out of range, or H % Hkv != 0  */
    LINATTN_ERR_DTYPE = -3,       /* unknown element type or feature map in dtype     */
    LINATTN_ERR_UNSUPPORTED = -4, /* d or chunk not supported by the kernels          */
    LINATTN_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required       */
    LINATTN_ERR_HIP = -6,         /* a HIP launch or runtime call failed              */
    LINATTN_ERR_ALIGN = -7,       /* a pointer is not 16-byte aligned                 */
    LINATTN_ERR_SCRATCH = -8      /* linattn_fwd_noalloc: the call needs more than the
                                     library's static scratch                          */
};

/*
 * linattn_fwd - forward pass over whole sequences.
 *
 * Computes `out` from q, k, v as stated at the top of this file: causal = 1
 * gives the running-state (s <= t) form; causal = 0 the non-causal form
 * O = phi(Q) (phi(K)^T V) over all N keys (README "How It Works"; the
 * normaliser is then phi(q_t) . sum_s phi(k_s)).
 *
 *   q, k, v     device, dtype, layouts above; read only.
 *   out         device, dtype, [B][H][N][d]; fully written.
 *   B, H, Hkv   batch, query heads, key/value heads (B >= 0, H % Hkv == 0).
 *   N           tokens per sequence (N >= 0; any N, ragged tails are masked).
 *   d           head dimension, 32, 64 or 128.
 *   causal      1 causal, 0 non-causal.
 *   normalise   1 divide by phi(q_t) . z_t, 0 return the numerator only.
 *   dtype       LINATTN_F32, LINATTN_BF16 or LINATTN_F16.
 *   state_out   nullable device fp32 [B][Hkv][d][d]: receives S_N (all N keys).
 *   z_out       nullable device fp32 [B][Hkv][d]: receives z_N.
 *   chunk       tokens per intra-chunk block: 0 = automatic, else 32, 64, 128
 *               or 256.  It changes only the order of summation.
 *   workspace   device scratch of at least linattn_fwd_workspace_bytes(...)
 *               bytes (may be NULL when that size is 0); its contents on
 *               entry do not matter and are clobbered.
 *   stream      HIP stream to enqueue on.
 * Returns LINATTN_OK or a LINATTN_ERR_* code.  B == 0 or N == 0 is a valid
 * no-op except that state_out / z_out, if given, are zero-filled.
 */
int linattn_fwd(const void *q, const void *k, const void *v, void *out,
                int B, int H, int Hkv, int N, int d, int causal, int normalise, int dtype,
                float *state_out, float *z_out, int chunk,
                void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * linattn_fwd_from_state - linattn_fwd for sequences that continue earlier
 * tokens (README "Features", the KV-cache-reuse item: a prompt's state
 * carried into the tokens that follow it; chunked prefill).  The running
 * sums start from the given ones instead of zero:
 *   S_t = state_in + sum_{s<=t} phi(k_s) v_s^T,  z_t = z_in + sum_{s<=t} phi(k_s)
 * (non-causal: the sums over all N keys are added to them).  Running a
 * sequence in pieces, each from the previous piece's state_out / z_out,
 * gives the rows of one call over the whole sequence (up to the order of
 * summation).
 *
 *   state_in    device fp32 [B][Hkv][d][d], required; read only.
 *   z_in        device fp32 [B][Hkv][d]; read only.  NULL means zero and is
 *               allowed only when normalise == 0.
 * All other arguments, the workspace size (linattn_fwd_workspace_bytes with
 * the same arguments) and the error behaviour are those of linattn_fwd;
 * state_out / z_out may alias neither state_in nor z_in.  With N == 0,
 * state_out / z_out receive copies of state_in / z_in.
 */
int linattn_fwd_from_state(const void *q, const void *k, const void *v, void *out,
                           int B, int H, int Hkv, int N, int d, int causal, int normalise, int dtype,
                           const float *state_in, const float *z_in,
                           float *state_out, float *z_out, int chunk,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * linattn_fwd_packed - linattn_fwd for a packed batch of sequences of
 * different lengths, with no padding (README "Features": variable sequence
 * length).  Sequence b owns tokens [cu_seqlens[b], cu_seqlens[b+1]) of
 * `total`, and every sequence is an independent forward pass (its own S and
 * z from zero; causal or not, normalised or not as for linattn_fwd).
 *
 *   q, out      device, dtype: the sequences' [H][n_b][d] blocks one after
 *               another (sequence b from element H * cu_seqlens[b] * d);
 *               H * total * d elements in all.
 *   k, v        device, dtype: likewise [Hkv][n_b][d] blocks, from element
 *               Hkv * cu_seqlens[b] * d.
 *   cu_seqlens  device int32 [nseqs + 1], non-decreasing, cu_seqlens[0] = 0,
 *               cu_seqlens[nseqs] = total.  Read on the device only (the
 *               call can be captured in a graph).  Offsets that break these
 *               rules give unspecified rows but no access outside the
 *               buffers: they are clamped to [0, total] and made
 *               non-decreasing.
 *   state_out, z_out  nullable: [nseqs][Hkv][d][d] and [nseqs][Hkv][d] fp32
 *               final sums per sequence (zero for an empty sequence).
 *   workspace   linattn_fwd_packed_workspace_bytes() bytes (depends on
 *               nseqs, total and the shape, not on the lengths).
 * Other arguments and errors as for linattn_fwd.
 */
size_t linattn_fwd_packed_workspace_bytes(int nseqs, int H, int Hkv, int total, int d, int causal, int dtype,
                                          int chunk);
int linattn_fwd_packed(const void *q, const void *k, const void *v, void *out, const int *cu_seqlens,
                       int nseqs, int total, int H, int Hkv, int d, int causal, int normalise, int dtype,
                       float *state_out, float *z_out, int chunk, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/*
 * linattn_fwd_timed - linattn_fwd with stage timing for profilers and
 * benchmarks.  Identical results; in addition it records events[0] on
 * `stream` before the first stage, events[1] before the second, events[2]
 * before the third and events[3] after the last.  The stages are:
 *   causal:     segment totals, segment prefix scan, chunked main pass;
 *   non-causal: segment totals, sum of the totals, application to the queries.
 * A stage the plan does not need is skipped (its two events coincide).
 * The last stage reads only the inputs and the workspace, so it is launched
 * `reps` (>= 1) times back to back between events[2] and events[3], with
 * the same result: (events[3] - events[2]) / reps is then its duration per
 * launch without the cost of recording an event around every launch.
 * reps == 0 launches the first two stages only (out is not written; events[2]
 * and events[3] coincide): a caller can then price the last stage as the
 * difference between timings of calls with and without it.
 * `events` points to n_events == 4 events created by the caller
 * (hipEventCreate); otherwise LINATTN_ERR_NULL is returned.  reps < 0 is
 * LINATTN_ERR_SHAPE.
 */
int linattn_fwd_timed(const void *q, const void *k, const void *v, void *out,
                      int B, int H, int Hkv, int N, int d, int causal, int normalise, int dtype,
                      float *state_out, float *z_out, int chunk,
                      void *workspace, size_t workspace_bytes, hipStream_t stream,
                      hipEvent_t *events, int n_events, int reps);

/*
 * linattn_fwd_workspace_bytes - scratch size linattn_fwd needs for these
 * arguments (0 when none).  Returns (size_t)-1 for invalid arguments.
 * The scratch holds one fp32 partial state and normaliser, d*(d+1) floats,
 * per (batch, kv head, sequence segment).
 */
size_t linattn_fwd_workspace_bytes(int B, int H, int Hkv, int N, int d, int causal, int dtype,
                                   int chunk);

/*
 * linattn_fwd_noalloc - linattn_fwd for callers that cannot allocate: code
 * under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc.  Same arguments, results and errors as linattn_fwd, without the
 * workspace: the call uses the library's static device scratch of
 * LINATTN_NOALLOC_SCRATCH_BYTES (64 MiB; one copy per GPU the library runs
 * on, held until the process ends) and calls no hipMalloc, hipFree or other
 * allocating routine.  A call whose linattn_fwd_workspace_bytes(...) exceeds
 * that size returns LINATTN_ERR_SCRATCH before anything is launched.  The
 * caller still provides q, k, v, out and the optional state_out / z_out.
 * Every call on one GPU shares that GPU's scratch, so calls that overlap in
 * time on one GPU (two streams, or two host threads) race and must be
 * ordered by the caller; calls ordered on one stream are safe.  The first
 * call on a device looks up the scratch's address there (a host-side
 * lookup, no allocation) under a lock.
 */
#define LINATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int linattn_fwd_noalloc(const void *q, const void *k, const void *v, void *out,
                        int B, int H, int Hkv, int N, int d, int causal, int normalise, int dtype,
                        float *state_out, float *z_out, int chunk, hipStream_t stream);

/*
 * linattn_fwd_plan - the launch plan linattn_fwd would use (host only, no
 * GPU work): chunk size and number of sequence segments per (batch, kv head).
 * Either output pointer may be NULL.  Returns LINATTN_OK or an error code.
 */
int linattn_fwd_plan(int B, int H, int Hkv, int N, int d, int causal, int dtype, int chunk,
                     int *chunk_out, int *segments_out);

/*
 * linattn_decode_step - append one token to every carried state and emit
 * the outputs for it (README "Features" list: KV cache reuse and fast
 * decoding; the fixed-size state replaces a growing key/value cache).
 *
 * For every batch b and kv head g, in place:
 *     S[b][g] += phi(k[b][g]) v[b][g]^T,   z[b][g] += phi(k[b][g]),
 * and then for every query head h of the group
 *     out[b][h] = phi(q[b][h])^T S[b][g] / (phi(q[b][h]) . z[b][g])
 * (or the numerator only when normalise == 0).  The update happens before
 * the read, so the new token attends to itself (s <= t), and a decode step
 * after a prefill of N tokens equals row N of a prefill of N + 1 tokens.
 *
 *   state   device fp32 [B][Hkv][d][d], read and written in place.
 *   z       device fp32 [B][Hkv][d], read and written in place.  May be NULL
 *           only when normalise == 0; when given it is always advanced
 *           (z += phi(k)), whatever normalise is, so a state carried through
 *           unnormalised steps can later be read normalised.
 *   q, out  device, dtype, [B][H][d];  k, v  device, dtype, [B][Hkv][d].
 *   out must not alias state, z, q, k or v.
 * Returns LINATTN_OK or a LINATTN_ERR_* code.
 */
int linattn_decode_step(float *state, float *z, const void *q, const void *k, const void *v,
                        void *out, int B, int H, int Hkv, int d, int normalise, int dtype,
                        hipStream_t stream);

/*
 * linattn_fwd_decay - causal forward pass with decayed running sums.  The
 * pages give decay only for the scan of the Stream efficiency essay
 * (section 4.2: h_t = h_{t-1} a_t + b_t); taken over to the sums of linear
 * attention with a log-decay g per (batch, kv head, token):
 *     S_t = exp(g_t) S_{t-1} + phi(k_t) v_t^T,   z_t = exp(g_t) z_{t-1} + phi(k_t),
 *     o_t = phi(q_t)^T S_t / (phi(q_t) . z_t)   (numerator only when normalise == 0),
 * with S and z starting from state_in / z_in (zero when NULL).  g = 0
 * everywhere gives linattn_fwd_from_state's rows; a query head reads its kv
 * head's sums, so the decay is per kv head.
 *
 *   g           device fp32 [B][Hkv][N], read only, 4-byte aligned.  Meant for
 *               g <= 0 (every factor in (0, 1]); larger values are not
 *               checked and can overflow.  Values below -20 (factors under
 *               2.1e-9) are taken as -20, so a reset (g = -inf) works; NaN
 *               propagates.
 *   state_in, z_in  device fp32 [B][Hkv][d][d] / [B][Hkv][d] or NULL (zero).
 * The other arguments are those of linattn_fwd with causal = 1.  Supported:
 * the default feature map (ELU + 1) in any element type, and every chunk
 * except one that makes an fp32 kernel shift its state copies (fp32,
 * d = 64, chunk 128): LINATTN_ERR_UNSUPPORTED otherwise.  chunk = 0 takes
 * linattn_fwd's automatic chunk, at most 64 tokens for 16-bit rows at
 * d <= 64.  The workspace is
 * linattn_fwd_decay_workspace_bytes(B, H, Hkv, N, d, dtype, chunk) bytes:
 * that of linattn_fwd plus one float per segment partial.  state_out /
 * z_out may alias neither state_in nor z_in.
 */
int linattn_fwd_decay(const void *q, const void *k, const void *v, const float *g, void *out,
                      int B, int H, int Hkv, int N, int d, int normalise, int dtype,
                      const float *state_in, const float *z_in, float *state_out, float *z_out, int chunk,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);
/* Workspace bytes linattn_fwd_decay needs; (size_t)-1 for arguments it rejects. */
size_t linattn_fwd_decay_workspace_bytes(int B, int H, int Hkv, int N, int d, int dtype, int chunk);

/*
 * linattn_decode_step_decay - linattn_decode_step with decayed sums: for
 * every batch b and kv head g the state and normaliser are first multiplied
 * by exp(gd[b][g]), then the token is added and read as in
 * linattn_decode_step.  gd: device fp32 [B][Hkv], read only, 4-byte aligned.
 */
int linattn_decode_step_decay(float *state, float *z, const void *q, const void *k, const void *v,
                              const float *gd, void *out, int B, int H, int Hkv, int d, int normalise,
                              int dtype, hipStream_t stream);

/*
 * linattn_fwd_window - causal forward pass over a sliding window of keys.
 * The pages name a sliding window (LinearTile 1.0.0 README, "Features" list,
 * sliding-window item: local context) without defining it; the reading taken
 * is the causal band of `window` keys: query t sees keys t - window < s <= t,
 *     o_t = sum_{band} (phi(q_t) . phi(k_s)) v_s / sum_{band} phi(q_t) . phi(k_s)
 * (the numerator only when normalise == 0).  window >= N gives linattn_fwd's
 * causal rows.  The band is formed directly (masked scores times values on the
 * matrix cores), so the cost is O(N * min(window, N) * d) per query head and
 * no running state is kept or returned.
 *
 *   q, out      device, dtype, [B][H][N][d];  k, v  device, dtype, [B][Hkv][N][d].
 *   window      keys per band, >= 1.
 * Other arguments, layouts and errors as for linattn_fwd; no workspace.
 */
int linattn_fwd_window(const void *q, const void *k, const void *v, void *out,
                       int B, int H, int Hkv, int N, int d, int window, int normalise, int dtype,
                       hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char *linattn_status_string(int status);

/* LINATTN_ABI_VERSION of the built library. */
int linattn_abi_version(void);

/*
 * linattn_bwd - gradients of linattn_fwd (the README's project layout names a
 * backward module; the gradient is the chain rule on the "How It Works"
 * definition, with the reverse-time walk of a running sum described in the
 * Stream efficiency essay, section 4.2).
 *
 * For the output gradient dout = dL/dout of o_t = num_t / den_t (or num_t
 * when normalise == 0), with a = phi(q), b = phi(k):
 *     g_t = dout_t / den_t,   h_t = -(dout_t . out_t) / den_t
 *     dq_t = (S_t g_t + h_t z_t) * phi'(q_t)
 *     dv_s = R_s^T b_s,   dk_s = (R_s v_s + r_s) * phi'(k_s)
 * where S_t, z_t are the forward's running sums seen by t and
 * R_s = sum a_t g_t^T, r_s = sum h_t a_t over the queries t that see key s
 * (t >= s causal, all t non-causal) and over the G query heads of the kv
 * group (GQA: dk, dv are summed over the group).  phi'(x) = 1 for x > 0,
 * exp(x) otherwise.
 *
 *   q, out, dout    device, dtype, [B][H][N][d]; out is the forward output
 *                   (used for h only; may be NULL when normalise == 0).
 *   k, v            device, dtype, [B][Hkv][N][d].
 *   dq              device, dtype, [B][H][N][d], written.
 *   dk, dv          device, dtype, [B][Hkv][N][d], written.
 *   causal, normalise, dtype   as in linattn_fwd (fp32 accumulation).
 *   workspace       device scratch of linattn_bwd_workspace_bytes() bytes,
 *                   16-byte aligned, owned by the caller; overwritten.
 * The outputs may not alias any input or each other.  All pointers 16-byte
 * aligned.  Asynchronous on `stream`; argument errors are returned before
 * any launch (LINATTN_ERR_*), launch failures as LINATTN_ERR_HIP.
 */
size_t linattn_bwd_workspace_bytes(int B, int H, int Hkv, int N, int d, int causal, int dtype);
int linattn_bwd(const void *q, const void *k, const void *v, const void *out, const void *dout,
                void *dq, void *dk, void *dv, int B, int H, int Hkv, int N, int d, int causal,
                int normalise, int dtype, void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
