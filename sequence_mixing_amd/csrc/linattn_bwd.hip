// linattn_bwd.hip - backward pass of phi = ELU+1 linear attention (gfx950).
//
// The forward pass (LinearTile 1.0.0 README, "How It Works", with the causal
// and GQA items of its "Features" list) is o_t = num_t / den_t with
// a_t = phi(q_t), b_s = phi(k_s), num_t = S_t^T a_t, den_t = a_t . z_t and the
// running sums S_t = sum_{s<=t} b_s v_s^T, z_t = sum_{s<=t} b_s.  Its gradient
// for an output gradient dO (the chain rule; the README's project layout
// names a backward module without its content, and the Stream efficiency
// essay, section 4.2, differentiates a running-sum recurrence by a
// reverse-time scan, the pattern used for dK and dV here):
//   g_t = dO_t / den_t,  h_t = -(dO_t . o_t) / den_t      (normalise == 0:
//                                                          g_t = dO_t, h_t = 0)
//   dq_t = (S_t g_t + h_t z_t) * phi'(q_t)
//   dv_s = R_s^T b_s,  dk_s = (R_s v_s + r_s) * phi'(k_s)
// with R_s = sum_{t>=s} a_t g_t^T and r_s = sum_{t>=s} h_t a_t over the query
// heads of the kv group (non-causal: every sum runs over the whole sequence).
// phi'(x) is taken from phi(x) (the feature map's df): for ELU + 1, 1 for
// x > 0 and exp(x) = phi(x) otherwise, i.e. min(1, phi(x)).
//
// Workgroups hand data over through LDS with lds_barrier(), which leaves the
// global loads of the next head or chunk in flight across the barrier.
//
// Launches (one workgroup = 4 wave64s, 8 for the dq walk at d = 128; chunks
// of 32 tokens):
//   seg_totals, seg_scan   the forward's segment sums of b v^T and b, giving
//                          each dq segment its starting S and z;
//   bwd_dq                 per (sequence, segment): walks the segment
//                          forwards, serving the G query heads of the group.
//                          Per chunk: z_t of every token (LDS prefix); per
//                          head: den = a . z_t, then on MFMA
//                          dA^T = B^T (M .* (V G^T + h)) + S G^T; writes dq,
//                          and den and h of every token (kept for the next
//                          passes, which then need not read the outputs);
//   bwd_dkv<totals>        per (sequence, segment): sum of a g^T and h a over
//                          the segment and the group's heads;
//   seg_scan (suffix)      gives each segment the sums of the later ones;
//   bwd_dkv                per (sequence, segment): walks the segment
//                          backwards.  Per chunk and head, on MFMA:
//                          dV^T += G^T (M .* A B^T), dB^T += A^T (M .* (G V^T + h)),
//                          R += A^T G; then dV^T += R^T B^T, dB^T += R V^T + r.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "linattn.h"
#include "linattn_kern.h"

namespace {

constexpr int kBC = 32;  // tokens per chunk (one 32-row MFMA tile)

// The dq walk runs 8 waves at d = 128 (two per SIMD): each wave carries half
// the state tiles of a 4-wave workgroup and the two waves on a SIMD hide each
// other's waits.  So does the dk/dv walk (its K-block loops unrolled by two,
// so that its accumulators fit); its totals pass keeps 4.
constexpr int DQ_WAVES(int d) { return d == 128 ? 8 : 4; }
constexpr int DKV_WAVES(int d, bool totals) { return d == 128 && !totals ? 8 : 4; }

// Shapes of the backward kernels for element type T and head dimension D.
template <typename T, int D, int NWAVES = 4>
struct BGeo {
    static constexpr int U = Vt<T>::U;          // elements per 16-byte group
    static constexpr int GPR = D / U;           // groups per token row
    static constexpr int NGRP = kBC * GPR;      // groups per chunk of one tensor
    static constexpr int NW = NWAVES;
    static constexpr int TH = 64 * NW;
    static constexpr int LDV = (NGRP + TH - 1) / TH;
    static constexpr int DT = D / 32;
    static constexpr int KBD = D / 16;          // K-blocks over features
    static constexpr int NST = DT * DT;
    static constexpr int MAXST = (NST + NW - 1) / NW;
    static constexpr int E = (int)sizeof(T);
    // Two workgroups per CU (two waves per SIMD hide each other's waits) where
    // the registers allow it without spilling vector registers: both walks up
    // to d = 64 (the fp32 dk/dv walk then needs 239 of the 256 registers).
    static constexpr int OCC_DQ = D <= 64 ? 2 : 1;
    static constexpr int OCC_DKV = D <= 64 ? 2 : 1;
    __device__ static int tile_of(int w, int i) { return w * MAXST + i; }
};

template <typename T> __device__ __forceinline__ typename Vt<T>::g16 to_g16(const float *x);
template <> __device__ __forceinline__ bf16x8 to_g16<bf16>(const float *x) { return cvt8<bf16>(x); }
template <> __device__ __forceinline__ f32x4 to_g16<float>(const float *x) { return f32x4{x[0], x[1], x[2], x[3]}; }

// Registers base..base+7 of an accumulator as one operand fragment (rows
// 16 kb + 4h + e and 16 kb + 8 + 4h + e for base = 8 kb): an accumulator
// fed back as the B operand of the next product.
template <typename T> __device__ __forceinline__ typename Vt<T>::v8 acc8(const f32x16 &m, int base)
{
    float x[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] = m[base + s];
    return cvt8<T>(x);
}

// Low part of a 16-bit operand: x - (float)round(x), rounded.  For bf16 the
// pair (hi, lo) carries x to about 2^-16 relative, so a product of two split
// operands taken as hi*hi + hi*lo + lo*hi is close to an fp32 product; fp32
// operands need no low part.
template <typename T> __device__ __forceinline__ typename Vt<T>::g16 to_g16_lo(const float *x)
{
    float r[Vt<T>::U];
#pragma unroll
    for (int i = 0; i < Vt<T>::U; ++i) r[i] = x[i] - (float)(T)x[i];
    return to_g16<T>(r);
}
template <typename T> __device__ __forceinline__ typename Vt<T>::v8 acc8_lo(const f32x16 &m, int base)
{
    float x[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) x[s] = m[base + s] - (float)(T)m[base + s];
    return cvt8<T>(x);
}

// Sum over the GPR consecutive lanes that hold one token row.
template <int GPR> __device__ __forceinline__ float row_sum(float x)
{
#pragma unroll
    for (int m = GPR / 2; m >= 1; m /= 2) x += __shfl_xor(x, m);
    return x;
}

// Row-major accumulator tile (it, jt) of a d x d sum, written to an LDS tile
// in the operand type: lane (h, n) register r holds row it*32 + 8(r/4) + 4h + r%4,
// column jt*32 + n.
template <typename T, int D>
__device__ __forceinline__ void publish_tile(const f32x16 &acc, Tile<T, D> t, int it, int jt, int lane)
{
    const int h = lane >> 5, n = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) t.p[t.at(it * 32 + 8 * (r / 4) + 4 * h + (r % 4), jt * 32 + n)] = (T)acc[r];
}

// Buffer descriptor from values that are the same in every lane (chunk start,
// row counts): read from the first lane, so the descriptor stays in scalar
// registers even where the compiler computed its fields with vector
// instructions (a descriptor in vector registers makes it loop over lanes).
__device__ __forceinline__ Rsrc make_rsrc_u(const void *base, int bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return make_rsrc(reinterpret_cast<const void *>(((uint64_t)hi << 32) | lo), __builtin_amdgcn_readfirstlane(bytes));
}

// Loads one chunk of a [N][D] row-major sequence (tokens t0 .. t0 + rows - 1;
// zeros elsewhere, also for rows <= 0, without touching memory).
template <typename T, int D, int TH, int L>
__device__ __forceinline__ void load_rows(typename Vt<T>::g16 (&r)[L], const T *base, int t0, int rows, int tid)
{
    using g16 = typename Vt<T>::g16;
    static_assert(L == BGeo<T, D, TH / 64>::LDV, "register array size");
    const Rsrc rs = make_rsrc_u(base + (size_t)t0 * D, rows > 0 ? rows * D * (int)sizeof(T) : 0);
#pragma unroll
    for (int l = 0; l < L; ++l) r[l] = buf_load16<g16>(rs, (unsigned)(tid + l * TH) * 16u);
}

// One float per staged group: x[t0 + row of the group] (zero past rows).
template <typename T, int D, int TH, int L>
__device__ __forceinline__ void load_row_scalars(float (&r)[L], const float *base, int t0, int rows, int tid)
{
    using BG = BGeo<T, D, TH / 64>;
    static_assert(L == BG::LDV, "register array size");
    const Rsrc rs = make_rsrc_u(base + t0, rows > 0 ? rows * 4 : 0);
#pragma unroll
    for (int l = 0; l < BG::LDV; ++l) {
        const int e = tid + l * BG::TH;
        r[l] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (unsigned)(e / BG::GPR) * 4u, 0, 0));
    }
}

// ----------------------------------------------------------------- bwd_dq
//
// One workgroup per (batch, kv head, segment) walks the segment forwards and
// serves the G query heads of the group.  Per chunk: phi(k), v to LDS, the
// state copy S (d x d, fp32 in MFMA accumulators over the four waves) and the
// inclusive z_t of every token.  Per head: den_t = phi(q_t) . z_t, g, h, then
// dA^T on MFMA.  The next head's (or chunk's) rows are requested into
// registers while the current one is computed.
template <typename T, int D, typename IO>
__global__ __launch_bounds__((BGeo<T, D, DQ_WAVES(D)>::TH), (BGeo<T, D, DQ_WAVES(D)>::OCC_DQ)) void k_bwd_dq(const T *__restrict__ q, const T *__restrict__ k,
                                                      const T *__restrict__ v, const T *__restrict__ o,
                                                      const T *__restrict__ dout, T *__restrict__ dq,
                                                      float *__restrict__ den_out, float *__restrict__ h_out,
                                                      const float *__restrict__ ws,
                                                      float *__restrict__ ws_r, int H, int Hkv, int N, int G, int P,
                                                      int seg_len, int causal, int normalise)
{
    using BG = BGeo<T, D, DQ_WAVES(D)>;
    using g16 = typename Vt<T>::g16;
    constexpr int U = BG::U, GPR = BG::GPR, LDV = BG::LDV;
    // bf16: low parts of b and g.  dq of the first tokens of a normalised
    // sequence is a small difference of the value and normaliser terms, so the
    // intra-chunk products take both operands split (see to_g16_lo).
    constexpr bool SPLIT = sizeof(T) == 2;
    __shared__ __attribute__((aligned(16))) T smB[kBC * D];
    __shared__ __attribute__((aligned(16))) T smV[kBC * D];
    __shared__ __attribute__((aligned(16))) T smS[D * D];
    __shared__ __attribute__((aligned(16))) T smA[kBC * D];
    __shared__ __attribute__((aligned(16))) T smG[kBC * D];
    // fp32 at d = 128 would exceed the 160 KiB of LDS with its own output
    // tile: the dq rows then go into the g tile, after a barrier.
    constexpr bool OWN_O = !(sizeof(T) == 4 && D == 128);
    __shared__ __attribute__((aligned(16))) T smO[OWN_O ? kBC * D : 8];
    __shared__ __attribute__((aligned(16))) T smBl[SPLIT ? kBC * D : 8];
    __shared__ __attribute__((aligned(16))) T smGl[SPLIT ? kBC * D : 8];
    // fp16 rows: v itself is rounded to bf16 on staging, so it is split too
    constexpr bool SPLITV = SPLIT && !std::is_same_v<T, typename IO::elem>;
    __shared__ __attribute__((aligned(16))) T smVl[SPLITV ? kBC * D : 8];
    __shared__ __attribute__((aligned(16))) float sZt[kBC * D];  // z_t of every token of the chunk, [t][i]
    __shared__ __attribute__((aligned(16))) float sZp[D];        // z before the chunk
    __shared__ float sZq[BGeo<T, D, DQ_WAVES(D)>::TH];            // z over each quarter of the chunk's tokens
    __shared__ float sH[kBC];
    // 16-bit rows at d <= 64: this walk also forms the segment's sums
    // R = sum a g^T and r = sum h a over its tokens and the group's heads (the
    // a, g and h tiles are in LDS here anyway), which the dk/dv walk needs
    // from the segments after its own; otherwise (the registers are short) a
    // pass of k_bwd_dkv<totals> forms them.
    constexpr bool RT = sizeof(T) == 2 && D <= 64;
    constexpr int RS = BG::TH / D;  // row slices of the r partial sums
    __shared__ float sRp[RT ? RS * D : 1];
    const Tile<T, D> sA{smA}, sB{smB}, sV{smV}, sG{smG}, sO{OWN_O ? smO : smG}, sS{smS}, sBl{smBl}, sGl{smGl};
    const Tile<T, D> sVl{smVl};

    const int sq = blockIdx.x / P, p = blockIdx.x % P;  // (batch, kv head) sequence, segment
    const int bb = sq / Hkv, g = sq % Hkv;
    const int qh0 = bb * H + g * G;                       // first query head of the group
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, n = lane & 31;
    const T *kb = k + (size_t)sq * N * D;
    const T *vb = v + (size_t)sq * N * D;
    const int s0 = p * seg_len, s1 = min(N, s0 + seg_len);
    const int nch = (s1 - s0 + kBC - 1) / kBC;
    auto rows_of = [&](int c) { return c < nch ? min(kBC, s1 - (s0 + c * kBC)) : 0; };

    // Starting sums: causal segment p > 0 reads the inclusive prefix of the
    // segments before it (slot p - 1); non-causal reads the total (slot 0).
    const float *init = nullptr;
    if (!causal) init = ws + (size_t)sq * P * D * (D + 1);
    else if (p > 0) init = ws + ((size_t)sq * (P - 1) + (p - 1)) * (size_t)D * (D + 1);
    f32x16 S[BG::MAXST];
#pragma unroll
    for (int i = 0; i < BG::MAXST; ++i) {
        S[i] = f32x16{};
        const int st = BG::tile_of(w, i);
        if (init && st < BG::NST) {
            const int it = st / BG::DT, jt = st % BG::DT;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                S[i][r] = init[(size_t)(it * 32 + 8 * (r / 4) + 4 * h + (r % 4)) * D + jt * 32 + n];
        }
    }
    float zrun = (init && tid < D) ? init[(size_t)D * D + tid] : 0.f;
    if (!causal) {
        // the sums are the same for every token: one copy of S, z_t = z
#pragma unroll
        for (int i = 0; i < BG::MAXST; ++i) {
            const int st = BG::tile_of(w, i);
            if (st < BG::NST) publish_tile<T, D>(S[i], sS, st / BG::DT, st % BG::DT, lane);
        }
        // one load per thread: every e it fills has e % D == tid % D
        static_assert(BG::TH % D == 0, "z element of a thread");
        const float zt = init[(size_t)D * D + tid % D];
        if (tid < D) sZp[tid] = zt;
        for (int e = tid; e < kBC * D; e += BG::TH) sZt[e] = zt;
    }

    f32x16 Rt[RT ? BG::MAXST : 1];
#pragma unroll
    for (int i = 0; i < (RT ? BG::MAXST : 1); ++i) Rt[i] = f32x16{};
    const int rcol = tid % D, rsl = tid / D;
    float rpart = 0.f;

    g16 kr[LDV], vr[LDV], qr[LDV], orr[LDV], dr[LDV];
    load_rows<T, D, BG::TH>(kr, kb, s0, rows_of(0), tid);
    load_rows<T, D, BG::TH>(vr, vb, s0, rows_of(0), tid);
    load_rows<T, D, BG::TH>(qr, q + (size_t)qh0 * N * D, s0, rows_of(0), tid);
    load_rows<T, D, BG::TH>(orr, o + (size_t)qh0 * N * D, s0, normalise ? rows_of(0) : 0, tid);
    load_rows<T, D, BG::TH>(dr, dout + (size_t)qh0 * N * D, s0, rows_of(0), tid);

    for (int c = 0; c < nch; ++c) {
        const int t0 = s0 + c * kBC, rows = rows_of(c);
        // ---- phi(k), v of the chunk to LDS; the next chunk's rows requested
#pragma unroll
        for (int l = 0; l < LDV; ++l) {
            const int e = tid + l * BG::TH, t = e / GPR, cq = (e % GPR) * U;
            if (BG::NGRP % BG::TH == 0 || e < BG::NGRP) {
                float bk[U];
#pragma unroll
                for (int i = 0; i < U; ++i) bk[i] = t < rows ? IO::phi::f(Io<T, IO>::fi(kr[l], i)) : 0.f;
                sB.write16(t, cq, to_g16<T>(bk));
                if constexpr (SPLIT) sBl.write16(t, cq, to_g16_lo<T>(bk));
                sV.write16(t, cq, op16<T, IO>(vr[l]));
                if constexpr (SPLITV) {
                    float vf[U];
#pragma unroll
                    for (int ii = 0; ii < U; ++ii) vf[ii] = Io<T, IO>::fi(vr[l], ii);
                    sVl.write16(t, cq, to_g16_lo<T>(vf));
                }
            }
        }
        load_rows<T, D, BG::TH>(kr, kb, t0 + kBC, rows_of(c + 1), tid);
        load_rows<T, D, BG::TH>(vr, vb, t0 + kBC, rows_of(c + 1), tid);
        if (causal) {
#pragma unroll
            for (int i = 0; i < BG::MAXST; ++i) {
                const int st = BG::tile_of(w, i);
                if (st < BG::NST) publish_tile<T, D>(S[i], sS, st / BG::DT, st % BG::DT, lane);
            }
        }
        lds_barrier();
        // ---- z before the chunk and z_t after each of its tokens: thread
        // (quarter zq, feature zf) sums its quarter of the chunk's tokens,
        // then adds the quarters before it and z before the chunk
        if (causal) {
            constexpr int ZQ = BG::TH / D, ZT = kBC / ZQ;  // token quarters, tokens per quarter
            const int zf = tid % D, zq = tid / D;
            float loc[ZT];
            float z = 0.f;
#pragma unroll
            for (int i = 0; i < ZT; ++i) {
                const int t = zq * ZT + i;
                z += (float)sB.p[sB.at(t, zf)];
                if constexpr (SPLIT) z += (float)sBl.p[sBl.at(t, zf)];
                loc[i] = z;
            }
            sZq[zq * D + zf] = z;
            if (zq == 0) sZp[zf] = zrun;
            lds_barrier();
            float off = sZp[zf], all = 0.f;
#pragma unroll
            for (int q2 = 0; q2 < ZQ; ++q2) {
                const float x = sZq[q2 * D + zf];
                if (q2 < zq) off += x;
                all += x;
            }
#pragma unroll
            for (int i = 0; i < ZT; ++i) sZt[(zq * ZT + i) * D + zf] = off + loc[i];
            if (zq == 0) zrun += all;
        }
        lds_barrier();
        for (int hh = 0; hh < G; ++hh) {
            const int qh = qh0 + hh;
            // ---- a, den, g, h of this head; the next head's rows requested
            {
                const Rsrc rden = make_rsrc_u(den_out + (size_t)qh * N + t0, normalise ? rows * 4 : 0);
                const Rsrc rh = make_rsrc_u(h_out + (size_t)qh * N + t0, normalise ? rows * 4 : 0);
#pragma unroll
                for (int l = 0; l < LDV; ++l) {
                    const int e = tid + l * BG::TH, t = e / GPR, cq = (e % GPR) * U;
                    const bool grp = BG::NGRP % BG::TH == 0 || e < BG::NGRP;
                    float a[U], den = 0.f, dov = 0.f;
#pragma unroll
                    for (int i = 0; i < U; ++i) {
                        a[i] = IO::phi::f(Io<T, IO>::fi(qr[l], i));
                        dov += Io<T, IO>::fi(dr[l], i) * Io<T, IO>::fi(orr[l], i);
                    }
                    if (grp) {
#pragma unroll
                        for (int i = 0; i < U; ++i) den += a[i] * sZt[t * D + cq + i];
                    }
                    den = row_sum<GPR>(den);
                    dov = row_sum<GPR>(dov);
                    const float inv = t < rows ? (normalise ? 1.f / den : 1.f) : 0.f;
                    float gg[U];
#pragma unroll
                    for (int i = 0; i < U; ++i) gg[i] = Io<T, IO>::fi(dr[l], i) * inv;
                    const float hv = normalise ? -dov * inv : 0.f;
                    if (grp) {
                        sA.write16(t, cq, to_g16<T>(a));
                        sG.write16(t, cq, to_g16<T>(gg));
                        if constexpr (SPLIT) sGl.write16(t, cq, to_g16_lo<T>(gg));
                        if (e % GPR == 0) sH[t] = hv;
                    }
                    // den and h for the dk/dv passes (one lane per row; the others' offsets are out of range)
                    const unsigned roff = (grp && e % GPR == 0) ? (unsigned)t * 4u : kOutOfRange;
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, den), rden, roff, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, hv), rh, roff, 0, 0);
                }
                const int nh = hh + 1 < G ? hh + 1 : 0, nc = hh + 1 < G ? c : c + 1;
                const size_t nq = (size_t)(qh0 + nh) * N * D;
                const int nt0 = s0 + nc * kBC, nrows = rows_of(nc);
                load_rows<T, D, BG::TH>(qr, q + nq, nt0, nrows, tid);
                load_rows<T, D, BG::TH>(orr, o + nq, nt0, normalise ? nrows : 0, tid);
                load_rows<T, D, BG::TH>(dr, dout + nq, nt0, nrows, tid);
            }
            lds_barrier();
            // ---- dA^T tiles (one 32-feature block per unit); the state update after the last head
            constexpr int MAXI = (BG::DT + BG::NW - 1) / BG::NW;
            f32x16 dacc[MAXI];
#pragma unroll
            for (int ui = 0; ui < MAXI; ++ui) {
                const int it = w + BG::NW * ui;
                if (it >= BG::DT) break;
                f32x16 acc = f32x16{};
                const float hn = sH[n];
                if (causal) {
                    f32x16 M = f32x16{};  // M[s][t] = v_s . g_t + h_t for s <= t
#pragma unroll
                    for (int kk = 0; kk < BG::KBD; ++kk) {
                        const auto vf = sV.read8(n, kk * 16 + 8 * h);
                        mma(M, vf, sG.read8(n, kk * 16 + 8 * h));
                        if constexpr (SPLIT) mma(M, vf, sGl.read8(n, kk * 16 + 8 * h));
                        if constexpr (SPLITV) mma(M, sVl.read8(n, kk * 16 + 8 * h), sG.read8(n, kk * 16 + 8 * h));
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) M[r] = (8 * (r / 4) + 4 * h + (r % 4)) <= n ? M[r] + hn : 0.f;
#pragma unroll
                    for (int kb2 = 0; kb2 < 2; ++kb2) {
                        const int ra = 16 * kb2 + 4 * h;
                        const auto bh = colfrag(sB, ra, ra + 8, it * 32, lane);
                        mma(acc, bh, acc8<T>(M, 8 * kb2));
                        if constexpr (SPLIT) {
                            mma(acc, bh, acc8_lo<T>(M, 8 * kb2));
                            mma(acc, colfrag(sBl, ra, ra + 8, it * 32, lane), acc8<T>(M, 8 * kb2));
                        }
                    }
                }
#pragma unroll
                for (int kk = 0; kk < BG::KBD; ++kk)
                    mma(acc, sS.read8(it * 32 + n, kk * 16 + 8 * h), sG.read8(n, kk * 16 + 8 * h));
                dacc[ui] = acc;
            }
            if constexpr (!OWN_O) lds_barrier();  // every read of the g tile is done
            // registers 4 q4 .. 4 q4 + 3 are four consecutive features of
            // token n: written (and a, z read) four at a time
#pragma unroll
            for (int ui = 0; ui < MAXI; ++ui) {
                const int it = w + BG::NW * ui;
                if (it >= BG::DT) break;
                const float hn = sH[n];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int i0 = it * 32 + 8 * q4 + 4 * h;
                    const auto av = sA.read4(n, i0);
                    const f32x4 zp = *reinterpret_cast<const f32x4 *>(sZp + i0);
                    f32x4 x;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x[e] = (dacc[ui][4 * q4 + e] + hn * zp[e]) * IO::phi::df((float)av[e]);
                    sO.write4(n, i0, out4<T, IO>(x));
                }
            }
            if constexpr (RT) {
                // R += A^T G, r += A^T h over this head's tokens of the chunk
#pragma unroll
                for (int i = 0; i < BG::MAXST; ++i) {
                    const int st = BG::tile_of(w, i);
                    if (st < BG::NST) tile_state_update<T, D>(Rt[i], false, st / BG::DT, st % BG::DT, 0, sA, sG, lane);
                }
#pragma unroll
                for (int t = rsl * (kBC / RS); t < (rsl + 1) * (kBC / RS); ++t)
                    rpart += sH[t] * (float)sA.p[sA.at(t, rcol)];
            }
            if (causal && hh == G - 1) {
#pragma unroll
                for (int i = 0; i < BG::MAXST; ++i) {
                    const int st = BG::tile_of(w, i);
                    if (st < BG::NST) tile_state_update<T, D>(S[i], false, st / BG::DT, st % BG::DT, 0, sB, sV, lane);
                }
            }
            lds_barrier();
            // ---- dq rows of this head
            {
                const Rsrc rdq = make_rsrc_u(dq + ((size_t)qh * N + t0) * D, rows * D * (int)sizeof(T));
#pragma unroll
                for (int l = 0; l < LDV; ++l) {
                    const int e = tid + l * BG::TH, t = e / GPR, cq = (e % GPR) * U;
                    if (BG::NGRP % BG::TH == 0 || e < BG::NGRP)
                        buf_store16_nt<g16>(rdq, (unsigned)e * 16u, *reinterpret_cast<const g16 *>(sO.p + sO.at(t, cq)));
                }
            }
        }
    }
    if constexpr (RT) {
        // the segment's R, r: slot p - 1 of the causal suffix sums (segment 0
        // is no later segment's), slot p of the non-causal total
        if (!causal || p > 0) {
            const int nsl = causal ? P - 1 : P;
            float *dst = ws_r + ((size_t)sq * nsl + (causal ? p - 1 : p)) * (size_t)D * (D + 1);
#pragma unroll
            for (int i = 0; i < BG::MAXST; ++i) {
                const int st = BG::tile_of(w, i);
                if (st < BG::NST) {
                    const int it = st / BG::DT, jt = st % BG::DT;
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        dst[(size_t)(it * 32 + 8 * (r / 4) + 4 * h + (r % 4)) * D + jt * 32 + n] = Rt[i][r];
                }
            }
            sRp[rsl * D + rcol] = rpart;
            lds_barrier();
            if (tid < D) {
                float rf = 0.f;
                for (int sl = 0; sl < RS; ++sl) rf += sRp[sl * D + tid];
                dst[(size_t)D * D + tid] = rf;
            }
        }
    }
}

// ---------------------------------------------------------------- bwd_dkv
//
// TOTALS: per (sequence, segment) the sums R = sum a g^T and r = sum h a over
// the segment's tokens and the group's query heads, written to ws_r.
// Otherwise: the segment walked backwards from the sums of the later
// segments; per chunk the intra-chunk terms of every head, then the carried
// terms, then dk and dv are stored.  R lives in MFMA accumulators over the
// waves; r in per-thread partial sums (column tid % D, a slice of the rows).
template <typename T, int D, bool TOTALS, typename IO>
__global__ __launch_bounds__((BGeo<T, D, DKV_WAVES(D, TOTALS)>::TH), (BGeo<T, D, DKV_WAVES(D, TOTALS)>::OCC_DKV)) void k_bwd_dkv(const T *__restrict__ q, const T *__restrict__ k,
                                                       const T *__restrict__ v, const float *__restrict__ hrow,
                                                       const T *__restrict__ dout, const float *__restrict__ den,
                                                       T *__restrict__ dk, T *__restrict__ dv, float *__restrict__ ws_r,
                                                       int H, int Hkv, int N, int G, int P, int seg_len, int causal,
                                                       int normalise, int nslots, int first_seg)
{
    using BG = BGeo<T, D, DKV_WAVES(D, TOTALS)>;
    using g16 = typename Vt<T>::g16;
    constexpr int U = BG::U, GPR = BG::GPR, LDV = BG::LDV;
    constexpr int RS = BG::TH / D;  // row slices of the r partial sums
    __shared__ __attribute__((aligned(16))) T smA[kBC * D];
    __shared__ __attribute__((aligned(16))) T smG[kBC * D];
    __shared__ __attribute__((aligned(16))) T smB[TOTALS ? 16 / sizeof(T) : kBC * D];
    __shared__ __attribute__((aligned(16))) T smV[TOTALS ? 16 / sizeof(T) : kBC * D];
    __shared__ __attribute__((aligned(16))) T smR[TOTALS ? 16 / sizeof(T) : D * D];
    __shared__ float sH[kBC], sRp[RS * D];
    __shared__ __attribute__((aligned(16))) float sRf[D];  // the r partials summed, per feature
    const Tile<T, D> sA{smA}, sG{smG}, sB{smB}, sV{smV}, sR{smR};
    const Tile<T, D> sOK{smA}, sOV{smG};  // dk, dv rows, once the heads are done

    const int sq = blockIdx.x / nslots;                // (batch, kv head) sequence
    const int pseg = blockIdx.x % nslots + first_seg;  // segment
    const int bb = sq / Hkv, g = sq % Hkv;
    const int qh0 = bb * H + g * G;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, n = lane & 31;
    const int s0 = pseg * seg_len, s1 = min(N, s0 + seg_len);
    const int nch = (s1 - s0 + kBC - 1) / kBC;
    const T *kb = k + (size_t)sq * N * D;
    const T *vb = v + (size_t)sq * N * D;
    // chunks are visited last to first: step j is chunk nch - 1 - j
    auto t0_of = [&](int j) { return s0 + (nch - 1 - j) * kBC; };
    auto rows_of = [&](int j) { return j < nch ? min(kBC, s1 - t0_of(j)) : 0; };

    const float *init = nullptr;
    if (!TOTALS) {
        if (!causal) init = ws_r + (size_t)sq * P * D * (D + 1);
        else if (pseg < P - 1) init = ws_r + ((size_t)sq * (P - 1) + pseg) * (size_t)D * (D + 1);
    }
    f32x16 R[BG::MAXST];
#pragma unroll
    for (int i = 0; i < BG::MAXST; ++i) {
        R[i] = f32x16{};
        const int st = BG::tile_of(w, i);
        if (init && st < BG::NST) {
            const int it = st / BG::DT, jt = st % BG::DT;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                R[i][r] = init[(size_t)(it * 32 + 8 * (r / 4) + 4 * h + (r % 4)) * D + jt * 32 + n];
        }
    }
    // r partial: column tid % D over rows (tid / D) * (kBC / RS) ..; slice 0 holds the start value
    const int rcol = tid % D, rsl = tid / D;
    float rpart = (init && rsl == 0) ? init[(size_t)D * D + rcol] : 0.f;

    constexpr int NU = 2 * BG::DT, MAXU = (NU + BG::NW - 1) / BG::NW;
    f32x16 out[MAXU];
    const int nheads = (!TOTALS && !causal) ? 0 : G;

    // h of every token comes from the dq walk (it formed h from dO and the
    // outputs already), so the outputs are not read again here
    g16 kr[LDV], vr[LDV], qr[LDV], dr[LDV];
    float dn[LDV], hn[LDV];
    if (!TOTALS) {
        load_rows<T, D, BG::TH>(kr, kb, t0_of(0), rows_of(0), tid);
        load_rows<T, D, BG::TH>(vr, vb, t0_of(0), rows_of(0), tid);
    }
    {
        const int r0 = nheads > 0 ? rows_of(0) : 0;
        load_rows<T, D, BG::TH>(qr, q + (size_t)qh0 * N * D, t0_of(0), r0, tid);
        load_rows<T, D, BG::TH>(dr, dout + (size_t)qh0 * N * D, t0_of(0), r0, tid);
        load_row_scalars<T, D, BG::TH>(dn, den + (size_t)qh0 * N, t0_of(0), normalise ? r0 : 0, tid);
        load_row_scalars<T, D, BG::TH>(hn, hrow + (size_t)qh0 * N, t0_of(0), normalise ? r0 : 0, tid);
    }

    for (int j = 0; j < nch; ++j) {
        const int t0 = t0_of(j), rows = rows_of(j);
        if (!TOTALS) {
#pragma unroll
            for (int u = 0; u < MAXU; ++u) out[u] = f32x16{};
#pragma unroll
            for (int l = 0; l < LDV; ++l) {
                const int e = tid + l * BG::TH, t = e / GPR, cq = (e % GPR) * U;
                if (BG::NGRP % BG::TH == 0 || e < BG::NGRP) {
                    float bk[U];
#pragma unroll
                    for (int i = 0; i < U; ++i) bk[i] = t < rows ? IO::phi::f(Io<T, IO>::fi(kr[l], i)) : 0.f;
                    sB.write16(t, cq, to_g16<T>(bk));
                    sV.write16(t, cq, op16<T, IO>(vr[l]));
                }
            }
            load_rows<T, D, BG::TH>(kr, kb, t0_of(j + 1), rows_of(j + 1), tid);
            load_rows<T, D, BG::TH>(vr, vb, t0_of(j + 1), rows_of(j + 1), tid);
            // the carried sums of the later tokens, as they stand before this chunk
            if (causal || j == 0) {
#pragma unroll
                for (int i = 0; i < BG::MAXST; ++i) {
                    const int st = BG::tile_of(w, i);
                    if (st < BG::NST) publish_tile<T, D>(R[i], sR, st / BG::DT, st % BG::DT, lane);
                }
                sRp[rsl * D + rcol] = rpart;
            }
            lds_barrier();
            // r as it stands before this chunk, summed over the slices once
            // (read by the outputs after the heads' barriers; without heads,
            // non-causal, it is fixed and summed at the first chunk)
            if (causal || j == 0) {
                if (tid < D) {
                    float rs = 0.f;
#pragma unroll
                    for (int sl = 0; sl < RS; ++sl) rs += sRp[sl * D + tid];
                    sRf[tid] = rs;
                }
                if (nheads == 0) lds_barrier();
            }
        }
        for (int hh = 0; hh < nheads; ++hh) {
            // ---- a, g, h of this head; the next head's (or chunk's) rows requested
#pragma unroll
            for (int l = 0; l < LDV; ++l) {
                const int e = tid + l * BG::TH, t = e / GPR, cq = (e % GPR) * U;
                const bool real = t < rows;
                const float inv = real ? (normalise ? 1.f / dn[l] : 1.f) : 0.f;
                float a[U], gg[U];
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    a[i] = real ? IO::phi::f(Io<T, IO>::fi(qr[l], i)) : 0.f;
                    gg[i] = Io<T, IO>::fi(dr[l], i) * inv;
                }
                if (BG::NGRP % BG::TH == 0 || e < BG::NGRP) {
                    sA.write16(t, cq, to_g16<T>(a));
                    sG.write16(t, cq, to_g16<T>(gg));
                    if (e % GPR == 0) sH[t] = real && normalise ? hn[l] : 0.f;
                }
            }
            {
                const int nh = hh + 1 < G ? hh + 1 : 0, nj = hh + 1 < G ? j : j + 1;
                const size_t nq = (size_t)(qh0 + nh);
                const int nt0 = t0_of(nj), nrows = rows_of(nj);
                load_rows<T, D, BG::TH>(qr, q + nq * N * D, nt0, nrows, tid);
                load_rows<T, D, BG::TH>(dr, dout + nq * N * D, nt0, nrows, tid);
                load_row_scalars<T, D, BG::TH>(dn, den + nq * N, nt0, normalise ? nrows : 0, tid);
                load_row_scalars<T, D, BG::TH>(hn, hrow + nq * N, nt0, normalise ? nrows : 0, tid);
            }
            lds_barrier();
            // ---- intra-chunk terms (causal), then R += A^T G, r += A^T h
            if (!TOTALS && causal) {
#pragma unroll
                for (int u = 0; u < MAXU; ++u) {
                    const int unit = w + BG::NW * u;
                    if (unit < NU) {
                        f32x16 M = f32x16{};
                        if (unit < BG::DT) {
                            // M[t][s] = a_t . b_s for t >= s
#pragma unroll 2
                            for (int kk = 0; kk < BG::KBD; ++kk)
                                mma(M, sA.read8(n, kk * 16 + 8 * h), sB.read8(n, kk * 16 + 8 * h));
#pragma unroll
                            for (int r = 0; r < 16; ++r) M[r] = (8 * (r / 4) + 4 * h + (r % 4)) >= n ? M[r] : 0.f;
                        } else {
                            // M[t][s] = g_t . v_s + h_t for t >= s
#pragma unroll 2
                            for (int kk = 0; kk < BG::KBD; ++kk)
                                mma(M, sG.read8(n, kk * 16 + 8 * h), sV.read8(n, kk * 16 + 8 * h));
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int t = 8 * (r / 4) + 4 * h + (r % 4);
                                M[r] = t >= n ? M[r] + sH[t] : 0.f;
                            }
                        }
                        // dv^T[j][s] += sum_t g_t[j] M[t][s];  dk^T[i][s] += sum_t a_t[i] M[t][s]
                        const Tile<T, D> &src = unit < BG::DT ? sG : sA;
                        const int col = (unit < BG::DT ? unit : unit - BG::DT) * 32;
#pragma unroll
                        for (int kb2 = 0; kb2 < 2; ++kb2) {
                            const int ra = 16 * kb2 + 4 * h;
                            mma(out[u], colfrag(src, ra, ra + 8, col, lane), acc8<T>(M, 8 * kb2));
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < BG::MAXST; ++i) {
                const int st = BG::tile_of(w, i);
                if (st < BG::NST) tile_state_update<T, D>(R[i], false, st / BG::DT, st % BG::DT, 0, sA, sG, lane);
            }
#pragma unroll
            for (int t = rsl * (kBC / RS); t < (rsl + 1) * (kBC / RS); ++t) rpart += sH[t] * (float)sA.p[sA.at(t, rcol)];
            lds_barrier();
        }
        if (!TOTALS) {
            // ---- carried terms and the outputs of this chunk
#pragma unroll
            for (int u = 0; u < MAXU; ++u) {
                const int unit = w + BG::NW * u;
                if (unit < NU) {
                    if (unit < BG::DT) {
                        // dv^T[j][s] += sum_i R[i][j] b_s[i]
#pragma unroll 2
                        for (int kk = 0; kk < BG::KBD; ++kk) {
                            const int ra = kk * 16 + 8 * h;
                            mma(out[u], colfrag(sR, ra, ra + 4, unit * 32, lane), sB.read8(n, ra));
                        }
                    } else {
                        // dk^T[i][s] += sum_j R[i][j] v_s[j]
#pragma unroll 2
                        for (int kk = 0; kk < BG::KBD; ++kk)
                            mma(out[u], sR.read8((unit - BG::DT) * 32 + n, kk * 16 + 8 * h), sV.read8(n, kk * 16 + 8 * h));
                    }
                }
            }
            // registers 4 q4 .. 4 q4 + 3 of a unit are four consecutive
            // features of token n: written (and phi(k) read) four at a time
#pragma unroll
            for (int u = 0; u < MAXU; ++u) {
                const int unit = w + BG::NW * u;
                if (unit < NU) {
                    const int fb = (unit < BG::DT ? unit : unit - BG::DT) * 32;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int f0 = fb + 8 * q4 + 4 * h;
                        f32x4 x{out[u][4 * q4], out[u][4 * q4 + 1], out[u][4 * q4 + 2], out[u][4 * q4 + 3]};
                        if (unit < BG::DT) {
                            sOV.write4(n, f0, out4<T, IO>(x));
                        } else {
                            const auto bv = sB.read4(n, f0);
                            const f32x4 rf = *reinterpret_cast<const f32x4 *>(sRf + f0);
#pragma unroll
                            for (int e = 0; e < 4; ++e) x[e] = (x[e] + rf[e]) * IO::phi::df((float)bv[e]);
                            sOK.write4(n, f0, out4<T, IO>(x));
                        }
                    }
                }
            }
            lds_barrier();
            const Rsrc rdk = make_rsrc_u(dk + ((size_t)sq * N + t0) * D, rows * D * (int)sizeof(T));
            const Rsrc rdv = make_rsrc_u(dv + ((size_t)sq * N + t0) * D, rows * D * (int)sizeof(T));
#pragma unroll
            for (int l = 0; l < LDV; ++l) {
                const int e = tid + l * BG::TH, t = e / GPR, cq = (e % GPR) * U;
                if (BG::NGRP % BG::TH == 0 || e < BG::NGRP) {
                    buf_store16_nt<g16>(rdk, (unsigned)e * 16u, *reinterpret_cast<const g16 *>(sOK.p + sOK.at(t, cq)));
                    buf_store16_nt<g16>(rdv, (unsigned)e * 16u, *reinterpret_cast<const g16 *>(sOV.p + sOV.at(t, cq)));
                }
            }
        }
    }
    if (TOTALS) {
        float *dst = ws_r + ((size_t)sq * nslots + (blockIdx.x % nslots)) * (size_t)D * (D + 1);
#pragma unroll
        for (int i = 0; i < BG::MAXST; ++i) {
            const int st = BG::tile_of(w, i);
            if (st < BG::NST) {
                const int it = st / BG::DT, jt = st % BG::DT;
#pragma unroll
                for (int r = 0; r < 16; ++r) dst[(size_t)(it * 32 + 8 * (r / 4) + 4 * h + (r % 4)) * D + jt * 32 + n] = R[i][r];
            }
        }
        sRp[rsl * D + rcol] = rpart;
        lds_barrier();
        if (tid < D) {
            float rf = 0.f;
            for (int sl = 0; sl < RS; ++sl) rf += sRp[sl * D + tid];
            dst[(size_t)D * D + tid] = rf;
        }
    }
}

// ------------------------------------------------------------------ plan

struct BwdPlan {
    int nseq, G, P, seg_len, fwd_slots, r_slots;
    size_t off_den, off_h, off_r, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int bwd_plan(int B, int H, int Hkv, int N, int d, int causal, int dtype, BwdPlan *pl)
{
    if (B < 0 || H <= 0 || Hkv <= 0 || N < 0 || H % Hkv != 0) return LINATTN_ERR_SHAPE;
    if (!valid_dtype(dtype)) return LINATTN_ERR_DTYPE;
    if (d != 32 && d != 64 && d != 128) return LINATTN_ERR_UNSUPPORTED;
    // fp8 rows are forward inputs only (their gradients would be written as fp8)
    if ((dtype & 0xff) == LINATTN_FP8_E4M3 || (dtype & 0xff) == LINATTN_FP8_E5M2) return LINATTN_ERR_UNSUPPORTED;
    const int e = (dtype & 0xff) != LINATTN_F32 ? 2 : 4;
    if ((long long)N * d * e > 0x7fffffffLL) return LINATTN_ERR_SHAPE;
    BwdPlan p{};
    p.nseq = B * Hkv;
    p.G = H / Hkv;
    // Segments: about 512 workgroups for the walks (one per sequence and
    // segment), segments whole chunks of 32 tokens.
    const int nchunks = (N + kBC - 1) / kBC;
    int P = p.nseq > 0 ? (512 + p.nseq - 1) / p.nseq : 1;
    if (P > nchunks) P = nchunks;
    if (P < 1) P = 1;
    p.seg_len = ((nchunks + P - 1) / P) * kBC;
    p.P = N > 0 ? (N + p.seg_len - 1) / p.seg_len : 1;
    p.fwd_slots = causal ? p.P - 1 : p.P;
    p.r_slots = p.fwd_slots;
    const size_t part = (size_t)d * (d + 1) * 4;
    const size_t fwd = align256((size_t)p.nseq * p.fwd_slots * part);
    p.off_den = fwd;
    p.off_h = p.off_den + align256((size_t)B * H * N * 4);
    p.off_r = p.off_h + align256((size_t)B * H * N * 4);
    p.bytes = p.off_r + align256((size_t)p.nseq * p.r_slots * part);
    *pl = p;
    return LINATTN_OK;
}

template <typename T, int D, typename IO>
int run_bwd(const BwdPlan &pl, int H, int Hkv, int N, const void *q, const void *k, const void *v, const void *o,
            const void *dout, void *dq, void *dk, void *dv, int causal, int normalise, char *ws, hipStream_t st)
{
    const T *qq = static_cast<const T *>(q), *kk = static_cast<const T *>(k), *vv = static_cast<const T *>(v);
    const T *oo = static_cast<const T *>(o ? o : q);  // not read when normalise == 0
    const T *dd = static_cast<const T *>(dout);
    float *wf = reinterpret_cast<float *>(ws);
    float *wden = reinterpret_cast<float *>(ws + pl.off_den);
    float *wh = reinterpret_cast<float *>(ws + pl.off_h);
    float *wr = reinterpret_cast<float *>(ws + pl.off_r);
    const int P = pl.P, E = D * D + D;
    const int c1 = totals_chunk<T, D>(pl.seg_len);
    // 1. forward sums at the segment starts (or their total)
    if (causal) {
        if (P > 1 && launch_totals<T, D, IO>(c1, pl.nseq * (P - 1), st, in_ptr<IO>(kk), in_ptr<IO>(vv), wf, N,
                                              pl.seg_len, P - 1))
            return LINATTN_ERR_UNSUPPORTED;
        if (P > 2)
            hipLaunchKernelGGL(k_seg_scan, scan_grid(D, pl.nseq), dim3(kThreads), 0, st, wf,
                               P - 1, D, 0, (float *)nullptr, (float *)nullptr, (const float *)nullptr,
                               (const float *)nullptr);
    } else {
        if (launch_totals<T, D, IO>(c1, pl.nseq * P, st, in_ptr<IO>(kk), in_ptr<IO>(vv), wf, N, pl.seg_len, P))
            return LINATTN_ERR_UNSUPPORTED;
        hipLaunchKernelGGL(k_seg_scan, scan_grid(D, pl.nseq), dim3(kThreads), 0, st, wf, P, D,
                           1, (float *)nullptr, (float *)nullptr, (const float *)nullptr, (const float *)nullptr);
    }
    // 2. dq (and den)
    // (16-bit rows, d <= 64: the dq walk also writes each segment's sums of a g^T and h a)
    constexpr bool RT = sizeof(T) == 2 && D <= 64;
    hipLaunchKernelGGL((k_bwd_dq<T, D, IO>), dim3(pl.nseq * P), dim3(BGeo<T, D, DQ_WAVES(D)>::TH), 0, st, qq, kk, vv, oo, dd,
                       static_cast<T *>(dq), wden, wh, (const float *)wf, RT ? wr : (float *)nullptr, H, Hkv, N, pl.G, P,
                       pl.seg_len, causal, normalise);
    // 3. sums of a g^T and h a per segment (otherwise their own pass):
    // causal segments 1..P-1 with a suffix scan, non-causal all and their sum
    if (causal) {
        if (P > 1) {
            if (!RT)
                hipLaunchKernelGGL((k_bwd_dkv<T, D, true, IO>), dim3(pl.nseq * (P - 1)), dim3(BGeo<T, D, DKV_WAVES(D, true)>::TH), 0, st, qq, kk, vv,
                                   (const float *)wh, dd, (const float *)wden, (T *)nullptr, (T *)nullptr, wr, H, Hkv, N, pl.G, P,
                                   pl.seg_len, causal, normalise, P - 1, 1);
            if (P > 2)
                hipLaunchKernelGGL(k_seg_scan, scan_grid(D, pl.nseq), dim3(kThreads), 0, st,
                                   wr, P - 1, D, 2, (float *)nullptr, (float *)nullptr, (const float *)nullptr,
                                   (const float *)nullptr);
        }
    } else {
        if (!RT)
            hipLaunchKernelGGL((k_bwd_dkv<T, D, true, IO>), dim3(pl.nseq * P), dim3(BGeo<T, D, DKV_WAVES(D, true)>::TH), 0, st, qq, kk, vv, (const float *)wh, dd,
                               (const float *)wden, (T *)nullptr, (T *)nullptr, wr, H, Hkv, N, pl.G, P, pl.seg_len,
                               causal, normalise, P, 0);
        hipLaunchKernelGGL(k_seg_scan, scan_grid(D, pl.nseq), dim3(kThreads), 0, st, wr, P, D,
                           1, (float *)nullptr, (float *)nullptr, (const float *)nullptr, (const float *)nullptr);
    }
    // 4. dk, dv
    hipLaunchKernelGGL((k_bwd_dkv<T, D, false, IO>), dim3(pl.nseq * P), dim3(BGeo<T, D, DKV_WAVES(D, false)>::TH), 0, st, qq, kk, vv, (const float *)wh, dd,
                       (const float *)wden, static_cast<T *>(dk), static_cast<T *>(dv), wr, H, Hkv, N, pl.G, P,
                       pl.seg_len, causal, normalise, P, 0);
    return launch_status();
}

template <typename T, typename IO = Fmt<T, PhiElu1>>
int dispatch_bwd(const BwdPlan &pl, int d, int H, int Hkv, int N, const void *q, const void *k, const void *v,
                 const void *o, const void *dout, void *dq, void *dk, void *dv, int causal, int normalise, char *ws,
                 hipStream_t st)
{
    switch (d) {
    case 32: return run_bwd<T, 32, IO>(pl, H, Hkv, N, q, k, v, o, dout, dq, dk, dv, causal, normalise, ws, st);
    case 64: return run_bwd<T, 64, IO>(pl, H, Hkv, N, q, k, v, o, dout, dq, dk, dv, causal, normalise, ws, st);
    case 128: return run_bwd<T, 128, IO>(pl, H, Hkv, N, q, k, v, o, dout, dq, dk, dv, causal, normalise, ws, st);
    }
    return LINATTN_ERR_UNSUPPORTED;
}

}  // namespace

extern "C" {

size_t linattn_bwd_workspace_bytes(int B, int H, int Hkv, int N, int d, int causal, int dtype)
{
    BwdPlan pl;
    if (bwd_plan(B, H, Hkv, N, d, causal ? 1 : 0, dtype, &pl) != LINATTN_OK) return (size_t)-1;
    return pl.bytes;
}

int linattn_bwd(const void *q, const void *k, const void *v, const void *out, const void *dout, void *dq, void *dk,
                void *dv, int B, int H, int Hkv, int N, int d, int causal, int normalise, int dtype, void *workspace,
                size_t workspace_bytes, hipStream_t stream)
{
    BwdPlan pl;
    causal = causal ? 1 : 0;
    normalise = normalise ? 1 : 0;
    const int rc = bwd_plan(B, H, Hkv, N, d, causal, dtype, &pl);
    if (rc != LINATTN_OK) return rc;
    if (B == 0 || N == 0) return LINATTN_OK;
    if (!q || !k || !v || !dout || !dq || !dk || !dv || (normalise && !out)) return LINATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
        return LINATTN_ERR_ALIGN;
    if (!workspace || workspace_bytes < pl.bytes) return LINATTN_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    return with_format(dtype, [&](auto kind) {
        using K = decltype(kind);
        return dispatch_bwd<typename K::T, typename K::IO>(pl, d, H, Hkv, N, q, k, v, out, dout, dq, dk, dv, causal,
                                                           normalise, ws, stream);
    });
}

}  // extern "C"
