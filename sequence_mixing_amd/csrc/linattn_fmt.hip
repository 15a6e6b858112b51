// linattn_fmt.hip - gfx950 (MI355X) forward and decode kernels of
// liblinattn.so and their launchers.  Built once per (feature map, element
// type), selected by -DLINATTN_FMT_PHI / -DLINATTN_FMT_ELEM, so that the
// library's objects compile in parallel; the C ABI in linattn.hip calls the
// matching fwd_format / decode_format.
//
// Linear attention with phi(x) = ELU(x) + 1 (LinearTile 1.0.0 README, "How It
// Works": O = phi(Q) (phi(K)^T V), key/value product first).  Causal rows use
// the running state S_t = sum_{s<=t} phi(k_s) v_s^T and z_t = sum_{s<=t}
// phi(k_s) (README "Features": causal masking without a quadratic buffer;
// Katharopoulos et al. 2020, cited in the README's "Reference" section).
//
// Kernel family (workgroups of 4 wave64s = 256 threads; the chunk kernel's
// shapes that run one workgroup per CU use 8):
//   seg_totals    per (sequence, segment): T_p = phi(K_p)^T V_p and sum phi(K_p)
//                 on MFMA, written as fp32 partials (causal: all segments but
//                 the last; non-causal: all segments).
//   seg_scan      inclusive prefix of the partials along the segments (causal),
//                 or their sum (non-causal).
//   causal_chunks per (sequence, segment): walks the segment in chunks of C
//                 tokens.  Per chunk, for every query tile of 32 rows:
//                   O^T = V^T (M . phi(K) phi(Q)^T) + S_prev^T phi(Q)^T
//                 (intra-chunk masked term plus the carried-state term, both
//                 on MFMA), then S += phi(K)^T V on MFMA.  The d x d fp32 state
//                 lives in MFMA accumulators spread over the waves; the waves
//                 see it through LDS copies refreshed every key tile (or pair).
//   noncausal_apply  O = phi(Q) S / phi(Q) . z with the summed S, z.
//   decode_step   one token: S += phi(k) v^T, z += phi(k), then G query heads
//                 read the updated state.  Bandwidth bound, plain fp32 VALU.
//
// MFMA shapes: bf16 uses v_mfma_f32_32x32x16_bf16, fp32 uses
// v_mfma_f32_32x32x2_f32 (true fp32 products).  Every operand fragment holds,
// per lane, 8 values of one row/column for one "K-block" of 16 reduction
// indices; which reduction index a (half-wave, slot) pair holds is free as
// long as both operands agree, and the kernels exploit that to feed one
// product's accumulator layout straight into the next product.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "linattn.h"
#include "linattn_fwd.h"
#include "linattn_kern.h"
#include "linattn_plan.h"
#include "linattn_window.h"

#if !defined(LINATTN_FMT_PHI) || !defined(LINATTN_FMT_ELEM)
#error "built once per format: -DLINATTN_FMT_PHI=<LINATTN_PHI_*> -DLINATTN_FMT_ELEM=<LINATTN_F32|BF16|F16>"
#endif

namespace {

using linattn::record;
using linattn::Start;
using linattn::Timing;

// ----------------------------------------------------------- causal_chunks
//
// One workgroup per (sequence, block of GT query heads, segment), walking the
// segment in chunks of C tokens.  Per chunk:
//   staging  phi(K), V and phi(Q) of the chunk go to LDS (row-major).  The
//            output of the previous chunk, parked in the phi(Q) rows, is
//            stored to HBM just before those rows are overwritten.
//   phase 1  every state tile's owner wave publishes S^T and z to LDS before
//            every RPC-th 32-token key tile and adds each tile's phi(K)^T V
//            (MFMA): copy j is the state seen by query tiles j*RPC ..
//            j*RPC + RPC - 1 (all keys before key tile j*RPC).
//   phase 2  every unit (query head g, query tile r) computes
//            O^T = V^T (M . phi(K) phi(Q)^T) on the diagonal 32x32 tile, plus
//            the unmasked tiles between its state copy and the diagonal
//            (none when RPC = 1, at most one when RPC = 2), plus S_j^T phi(Q)^T,
//            and the denominator; it parks O in its own phi(Q) rows.
// Global memory is touched only during staging: one wait there covers loads
// and stores issued a whole chunk earlier, and the compute phases never wait
// on memory.  With staging waves (MainShape::pipe) half of the waves stage
// chunk c+1 while the other half run phase 2 of chunk c (see below).
template <typename T, int D, int C, int GT>
struct Main {
    static constexpr linattn::MainShape SH = linattn::main_shape((int)sizeof(T), D, C, GT);
    static constexpr int NW = SH.nw, TH = 64 * NW;   // waves and threads per workgroup
    static constexpr int U = Vt<T>::U;
    static constexpr int CT = C / 32, DT = D / 32, KBD = D / 16;
    static constexpr int NST = DT * DT, MAXST = (NST + NW - 1) / NW;
    static constexpr int GPR = D / U;                // 16-byte groups per row
    static constexpr int KVG = C * GPR;              // groups of one K (or V) chunk
    static constexpr int QG = GT * C * GPR;          // groups of the chunk's q rows
    static constexpr int LK = (KVG + TH - 1) / TH;
    static constexpr int LQ = (QG + TH - 1) / TH;
    static constexpr int NU = GT * CT;               // units (query head, 32-row query tile) per chunk
    // Waves that take phase-2 items: all, or the first half with staging waves.
    static constexpr int NWC = SH.pipe ? NW / 2 : NW;
    // With fewer units than those waves, a unit's output columns are split
    // over PARTS waves (each recomputes the unit's scores and denominator).
    static constexpr int PARTS = NU >= NWC ? 1 : (NWC / NU < DT ? NWC / NU : DT);
    static constexpr int NWI = NU * PARTS;           // phase-2 work items
    static constexpr int CTP = DT / PARTS;           // 32-column output tiles per item
    static constexpr int NSC = SH.nsc;
    static constexpr bool SHIFT = SH.shift;          // copy j = state after key tile j (fp32 only)
    static constexpr int RPC = SHIFT ? 1 : CT / NSC;
    static constexpr bool FITS = SH.fits;
    static constexpr int OCC = SH.occ;
    static constexpr bool PIPE = SH.pipe;            // phase-2 items on waves 0 .. NW/2-1, staging on the rest
    static_assert(SH.lk == LK && SH.lq == LQ, "staging shape");
    static_assert(!SHIFT || (sizeof(T) == 4 && NSC == CT - 1), "shifted copies");
    static_assert(DT % PARTS == 0 && (PARTS == 1 || NWI <= NWC), "phase-2 split");
    static_assert(DT % MAXST == 0 || NST <= NW, "z owner: every column-0 state tile is some wave's first");
    __device__ static int tile_of(int w, int i) { return w * MAXST + i; }
};

// DK: decayed sums (dense batches): gd [seq][N] holds the log-decay of every
// token; the chunk's tile sums of g (DecayTab) scale the state update, the
// scores within and next to the diagonal, and the state copy each query reads.
template <typename T, int D, int C, int GT, typename IO, bool DK = false>
__global__ __launch_bounds__((Main<T, D, C, GT>::TH), (Main<T, D, C, GT>::OCC)) void k_causal_chunks(
    const typename IO::elem *__restrict__ q, const typename IO::elem *__restrict__ k,
    const typename IO::elem *__restrict__ v, T *__restrict__ out,
    const float *__restrict__ ws, float *__restrict__ state_out, float *__restrict__ z_out,
    int H, int Hkv, int N, int G, int P, int seg_len, int normalise, const float *__restrict__ s_in,
    const float *__restrict__ z_in, Packed pk, const float *__restrict__ gd = nullptr)
{
    using M = Main<T, D, C, GT>;
    using v8 = typename Vt<T>::v8;
    using g16 = typename Vt<T>::g16;
    constexpr bool BF = sizeof(T) == 2;
    constexpr int U = M::U, CT = M::CT, DT = M::DT, KBD = M::KBD, GPR = M::GPR, NSC = M::NSC, RPC = M::RPC;
    constexpr int NW = M::NW, TH = M::TH;

    // PIPE: K, V and q double-buffered (staging waves fill one buffer while
    // the compute waves work on the other)
    constexpr bool PIPE = M::PIPE && !DK;
    constexpr int NB = PIPE ? 2 : 1;
    __shared__ __attribute__((aligned(16))) T smK[NB][C * D];
    __shared__ __attribute__((aligned(16))) T smV[NB][C * D];
    __shared__ __attribute__((aligned(16))) T smQ[NB][GT * C * D];
    __shared__ __attribute__((aligned(16))) T smST[NSC][D * D];
    __shared__ __attribute__((aligned(16))) T smZ[NSC][D];
    __shared__ __attribute__((aligned(16))) DecayTab<C> smDT;  // DK only
    static_assert(!(DK && M::SHIFT), "decayed sums need one state copy per key tile or pair");
    const Tile<T, D> sQ{smQ[0]};

    const int HB = G / GT;
    // Dense batch: blocks run over (sequence, head block, segment).  Packed
    // batch: over (kv head, head block, segment of all sequences), with the
    // sequence's length in place of N and its segment count in place of P.
    int p, hb, seq, np = P;
    size_t kbase, qbase, slot0;
    if (!pk.tab) {
        p = blockIdx.x % P;
        hb = (blockIdx.x / P) % HB;
        seq = blockIdx.x / (P * HB);
        const int b = seq / Hkv, gk = seq % Hkv;
        kbase = (size_t)seq * N * D;
        qbase = ((size_t)b * H + (size_t)gk * G + (size_t)hb * GT) * N * D;  // first query head of the block
        slot0 = (size_t)seq * (P - 1);
    } else {
        SegLoc r;
        const int rest = blockIdx.x / pk.nsmax;
        hb = rest % HB;
        const int gk = rest / HB;
        if (!packed_locate(pk, blockIdx.x % pk.nsmax, r)) return;
        p = r.p;
        np = r.np;
        N = r.n;
        seq = r.b * Hkv + gk;
        kbase = ((size_t)r.off * Hkv + (size_t)gk * r.n) * D;
        qbase = ((size_t)r.off * H + (size_t)(gk * G + hb * GT) * r.n) * D;
        slot0 = packed_slot0(r, gk, Hkv, 1);
    }
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, n = lane & 31;
    using In = typename IO::elem;
    const In *kb = k + kbase;
    const In *vb = v + kbase;
    const In *qb = q + qbase;
    T *ob = out + qbase;
    const int s0 = p * seg_len, s1 = min(N, s0 + seg_len);
    const int nch = (s1 - s0 + C - 1) / C;

    // ---- the state this segment starts from (state tile i of wave w is w*MAXST + i)
    f32x16 S[M::MAXST];
    float zr = 0.f;
    // segment p > 0: the scanned sums in slot p - 1; segment 0: the start
    // sums of a continuation, or zero
    const float *init = p > 0 ? ws + (slot0 + (p - 1)) * (size_t)D * (D + 1)
                              : (s_in ? s_in + (size_t)seq * D * D : nullptr);
    const float *initz = p > 0 ? init + (size_t)D * D : (z_in ? z_in + (size_t)seq * D : nullptr);
#pragma unroll
    for (int i = 0; i < M::MAXST; ++i) {
        S[i] = f32x16{};
        const int st = M::tile_of(w, i);
        if (st < M::NST) {
            const int it = st / DT, jt = st % DT;
            if (init) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    S[i][r] = init[(size_t)(it * 32 + 8 * (r / 4) + 4 * h + (r % 4)) * D + jt * 32 + n];
            }
            if (initz && i == 0 && jt == 0) zr = initz[it * 32 + n];
        }
    }
    // ---- staging: raw K, V, q of a chunk in registers, one chunk ahead
    // Raw K, V, q of the next chunk in registers: loaded one chunk ahead.
    // E: bytes of an output element; IE, GB: of an input element and of a raw
    // input group (they differ for fp8 rows, whose output is bf16).
    constexpr int E = (int)sizeof(T), IE = Io<T, IO>::EB, GB = Io<T, IO>::GB;
    struct Regs {
        g16 k[M::LK], v[M::LK], q[M::LQ];
        float g;  // DK: log-decay of token t0 + tid
    };
    const float *gb = DK ? gd + (size_t)seq * N : nullptr;
    Regs ra;
    // q / out group l of this thread: element offset from (head block, token
    // t0) and its token row within the chunk (qt = C marks a group past the block).
    unsigned qel[M::LQ];
    int qt[M::LQ];
#pragma unroll
    for (int l = 0; l < M::LQ; ++l) {
        const int e = tid + l * TH;
        const int row = e / GPR, qq = e % GPR;
        const int g = row / C, t = row % C;
        const bool in = M::QG % TH == 0 || e < M::QG;
        qel[l] = (unsigned)((g * N + t) * D + qq * U);
        qt[l] = in ? t : C;
    }
    const int qspan = GT * N * D;  // elements of the head block's q (and out)
    // Loads chunk [t0, t0 + C) of K, V and q; nothing (zeros) when the chunk
    // lies past the segment (t0 >= s1), zeros for tokens past N.
    auto rows_at = [&](int t0) { return t0 < s1 ? min(C, N - t0) : 0; };
    auto load_kv = [&](Regs &r, int t0) {
        const int rows = rows_at(t0);
        const Rsrc rk = make_rsrc(kb + (size_t)t0 * D, rows * D * IE);
        const Rsrc rv = make_rsrc(vb + (size_t)t0 * D, rows * D * IE);
#pragma unroll
        for (int l = 0; l < M::LK; ++l) {
            const unsigned off = (unsigned)(tid + l * TH) * GB;
            r.k[l] = load_in<T, IO>(rk, off);
            r.v[l] = load_in<T, IO>(rv, off);
        }
    };
    auto load_q = [&](Regs &r, int t0) {
        const int rows = rows_at(t0);
        const Rsrc rq = make_rsrc(qb + (size_t)t0 * D, rows ? (qspan - t0 * D) * IE : 0);
#pragma unroll
        for (int l = 0; l < M::LQ; ++l) r.q[l] = load_in_nt<T, IO>(rq, qt[l] < rows ? qel[l] * IE : kOutOfRange);
    };
    auto load_all = [&](Regs &r, int t0) {
        load_kv(r, t0);
        load_q(r, t0);
        if constexpr (DK) r.g = tid < rows_at(t0) ? gb[t0 + tid] : 0.f;
    };
    // The output parked in the q rows: read into registers before phi(q) of
    // the next chunk overwrites them, stored after the next loads are issued
    // (so the stores may still be in flight when those loads are consumed).
    auto read_out = [&](g16 (&o)[M::LQ]) {
#pragma unroll
        for (int l = 0; l < M::LQ; ++l) {
            const int e = tid + l * TH;
            const int row = (M::QG % TH == 0 || e < M::QG) ? e / GPR : 0, qq = e % GPR;
            o[l] = *reinterpret_cast<const g16 *>(sQ.p + sQ.at(row, qq * U));
        }
    };
    auto store_out = [&](const g16 (&o)[M::LQ], int t_prev) {
        const int rows = min(C, N - t_prev);
        const Rsrc ro = make_rsrc(ob + (size_t)t_prev * D, (qspan - t_prev * D) * E);
#pragma unroll
        for (int l = 0; l < M::LQ; ++l) buf_store16_nt<g16>(ro, qt[l] < rows ? qel[l] * E : kOutOfRange, o[l]);
    };
    // phi(q) of the staged chunk into the q rows.
    auto stage_q = [&](const Regs &r) {
#pragma unroll
        for (int l = 0; l < M::LQ; ++l) {
            const int e = tid + l * TH;
            if (M::QG % TH == 0 || e < M::QG) {
                const int row = e / GPR, qq = e % GPR;
                g16 fq;
#pragma unroll
                for (int i = 0; i < U; ++i) fq[i] = (T)IO::phi::f(Io<T, IO>::fi(r.q[l], i));
                sQ.write16(row, qq * U, fq);
            }
        }
    };

    const bool carry_out = p == np - 1 && (state_out || z_out);
    // Key tiles of the chunk at t0 holding tokens < N; tiles past them add
    // nothing and no query reads a copy published there.  In the last chunk
    // of a segment the state after the last published copy is needed only
    // when it is returned to the caller.
    auto kt_valid_of = [&](int t0) { return min(CT, (N - t0 + 31) / 32); };
    auto kt_upd_of = [&](int c, int t0) {
        const int kv = kt_valid_of(t0);
        return (c + 1 < nch || carry_out) ? kv : min(kv, M::SHIFT ? CT - 1 : RPC * (NSC - 1));
    };
    // ---- phase 1 of chunk c (tokens from t0): every state tile's owner
    // publishes the state before every RPC-th key tile (after each of tiles
    // 0 .. CT-2 with shifted copies) and absorbs each tile of sK, sV.
    auto phase1 = [&](int c, int t0, Tile<T, D> sK, Tile<T, D> sV) {
        const int kt_valid = kt_valid_of(t0), kt_upd = kt_upd_of(c, t0);
#pragma unroll
        for (int i = 0; i < M::MAXST; ++i) {
            const int st = M::tile_of(w, i);
            if (st < M::NST) {
                const int it = st / DT, jt = st % DT;
                const bool zown = i == 0 && jt == 0;
                const int row = jt * 32 + n;
                float zs = 0.f;
                auto publish = [&](int slot) {
                    const Tile<T, D> sST{smST[slot]};
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        f32x4 x{S[i][4 * q4], S[i][4 * q4 + 1], S[i][4 * q4 + 2], S[i][4 * q4 + 3]};
                        sST.write4(row, it * 32 + 8 * q4 + 4 * h, cvt4<T>(x));
                    }
                    if (zown && h == 0) smZ[slot][it * 32 + n] = (T)(zr + zs);
                };
#pragma unroll
                for (int kt = 0; kt < CT; ++kt) {
                    if (!M::SHIFT && kt % RPC == 0 && kt < kt_valid) publish(kt / RPC);
                    if (kt < kt_upd) {
                        if constexpr (DK) {
                            // the sums fade over the tile, then its keys are added with their weights
                            const float a = __builtin_amdgcn_exp2f(smDT.TL[kt] * kLog2e);
                            S[i] *= a;
                            const float dz = tile_state_update<T, D>(S[i], zown, it, jt, kt, sK, sV, lane, smDT.W);
                            if (zown) zr = a * zr + (BF ? dz : dz + __shfl_xor(dz, 32));
                        } else {
                            const float dz = tile_state_update<T, D>(S[i], zown, it, jt, kt, sK, sV, lane);
                            if (zown) zs += BF ? dz : dz + __shfl_xor(dz, 32);
                        }
                    }
                    if (M::SHIFT && kt < CT - 1 && kt < kt_valid) publish(kt);
                }
                if (zown) zr += zs;
            }
        }
    };

    // ---- phase 2: query tiles
    // phi(q) fragments of unit u: lane (h, n) holds query n, features kq*16 + 8h + s.
    auto unit_qf = [&](int u, v8 (&qf)[KBD], Tile<T, D> sQ) {
        const int qrow = (u / CT) * C + (u % CT) * 32 + n;
#pragma unroll
        for (int kq = 0; kq < KBD; ++kq) qf[kq] = sQ.read8(qrow, kq * 16 + h * 8);
    };
    // Output columns ct0 .. ct0 + CTP - 1 of unit u, parked in its q rows of
    // sQ; the chunk's keys and values in sK, sV.
    auto unit_run = [&](int u, int ct0, const v8 (&qf)[KBD], Tile<T, D> sK, Tile<T, D> sV, Tile<T, D> sQ) {
        const int g = u / CT, r = u % CT;
        // Shifted copies: tile r >= 1 reads copy r - 1 (keys before tile r);
        // tile 0 reads copy 0 (keys of tile 0 included) and subtracts the
        // keys of its diagonal tile that come after the query.
        const int j = M::SHIFT ? (r > 0 ? r - 1 : 0) : r / RPC;
        const bool sub = M::SHIFT && r == 0;
        const bool off = r % RPC != 0;   // one unmasked key tile r-1 before the diagonal
        const int qrow = g * C + r * 32 + n;
        // DK: L of this query and of the 16 keys its lane holds (below),
        // and the fade qs from the state copy to the query.
        float lq = 0.f, qs = 1.f;
        if constexpr (DK) {
            lq = smDT.L[r * 32 + n];
            qs = __builtin_amdgcn_exp2f((lq + (off ? smDT.TL[r - 1] : 0.f)) * kLog2e);
        }
        auto key_l = [&](int tile, float (&lk)[16]) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(&smDT.L[tile * 32 + 8 * q4 + 4 * h]);
#pragma unroll
                for (int e = 0; e < 4; ++e) lk[4 * q4 + e] = x[e];
            }
        };
        // Pt[key][query] = phi(K) phi(Q)^T; accumulator reg i holds key
        // 8(i/4) + 4h + i%4 of the tile for query n.
        v8 pb0, pb1, po0 = v8{}, po1 = v8{};
        {
            f32x16 Pt = f32x16{};
#pragma unroll
            for (int kq = 0; kq < KBD; ++kq) mma(Pt, sK.read8(r * 32 + n, kq * 16 + h * 8), qf[kq]);
            // Causal mask: accumulator reg i holds key 8(i/4) + 4h + i%4 of the
            // tile for query n; keep keys <= n (or, subtracting, -Pt for keys > n).
            const int kmax = n - 4 * h;
            float pv[16];
            if constexpr (DK) {
                // kept scores fade by exp(L[query] - L[key]) (<= 1)
                float lk[16];
                key_l(r, lk);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const bool le = 8 * (i / 4) + (i % 4) <= kmax;
                    pv[i] = le ? Pt[i] * __builtin_amdgcn_exp2f((lq - lk[i]) * kLog2e) : 0.f;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const bool le = 8 * (i / 4) + (i % 4) <= kmax;
                    pv[i] = sub ? (le ? 0.f : -Pt[i]) : (le ? Pt[i] : 0.f);
                }
            }
            pb0 = cvt8<T>(pv);
            pb1 = cvt8<T>(pv + 8);
        }
        if (off) {
            f32x16 Po = f32x16{};
#pragma unroll
            for (int kq = 0; kq < KBD; ++kq) mma(Po, sK.read8(r * 32 - 32 + n, kq * 16 + h * 8), qf[kq]);
            float ov[16];
            if constexpr (DK) {
                // keys of the tile before: exp(L[query] + TL[r-1] - L[key])
                float lk[16];
                key_l(r - 1, lk);
                const float lt = lq + smDT.TL[r - 1];
#pragma unroll
                for (int i = 0; i < 16; ++i) ov[i] = Po[i] * __builtin_amdgcn_exp2f((lt - lk[i]) * kLog2e);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) ov[i] = Po[i];
            }
            po0 = cvt8<T>(ov);
            po1 = cvt8<T>(ov + 8);
        }
        float den;
        if constexpr (BF) {
            // den = 1^T (masked Pt) + 1^T Po + z_j . phi(q), on the matrix core:
            // every row of the product equals the denominator of query n.
            f32x16 Dn = f32x16{};
            mma(Dn, ones8<T>(), pb0);
            mma(Dn, ones8<T>(), pb1);
            if (off) {
                mma(Dn, ones8<T>(), po0);
                mma(Dn, ones8<T>(), po1);
            }
            if constexpr (DK) {
                // the copy's z fades by qs: its own accumulator
                f32x16 Dz = f32x16{};
#pragma unroll
                for (int kq = 0; kq < KBD; ++kq)
                    mma(Dz, *reinterpret_cast<const v8 *>(&smZ[j][kq * 16 + h * 8]), qf[kq]);
                den = Dn[0] + qs * Dz[0];
            } else {
#pragma unroll
                for (int kq = 0; kq < KBD; ++kq)
                    mma(Dn, *reinterpret_cast<const v8 *>(&smZ[j][kq * 16 + h * 8]), qf[kq]);
                den = Dn[0];
            }
        } else {
            float ds = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s) ds += (float)pb0[s] + (float)pb1[s] + (float)po0[s] + (float)po1[s];
            float dzs = 0.f;
#pragma unroll
            for (int kq = 0; kq < KBD; ++kq)
#pragma unroll
                for (int s = 0; s < 8; ++s) (DK ? dzs : ds) += (float)qf[kq][s] * (float)smZ[j][kq * 16 + h * 8 + s];
            if constexpr (DK) ds += qs * dzs;
            den = ds + __shfl_xor(ds, 32);
        }
        const float inv = normalise ? 1.f / den : 1.f;
        const Tile<T, D> sST{smST[j]};
#pragma unroll
        for (int ct = ct0; ct < ct0 + M::CTP; ++ct) {
            // O^T[feature][query] = V^T Pt (slot s of K-block kb2 holds key
            // 16 kb2 + 8 (s/4) + 4h + s%4) + V^T Po + S_j^T phi(Q)^T.
            f32x16 O = f32x16{};
            if constexpr (DK) {
                // the copy's part first, faded by qs, then the keys of the chunk
#pragma unroll
                for (int kq = 0; kq < KBD; ++kq) mma(O, sST.read8(ct * 32 + n, kq * 16 + h * 8), qf[kq]);
                O *= qs;
            }
            mma(O, colfrag(sV, r * 32 + 4 * h, r * 32 + 8 + 4 * h, ct * 32, lane), pb0);
            mma(O, colfrag(sV, r * 32 + 16 + 4 * h, r * 32 + 24 + 4 * h, ct * 32, lane), pb1);
            if (off) {
                mma(O, colfrag(sV, r * 32 - 32 + 4 * h, r * 32 - 24 + 4 * h, ct * 32, lane), po0);
                mma(O, colfrag(sV, r * 32 - 16 + 4 * h, r * 32 - 8 + 4 * h, ct * 32, lane), po1);
            }
            if constexpr (!DK) {
#pragma unroll
                for (int kq = 0; kq < KBD; ++kq) mma(O, sST.read8(ct * 32 + n, kq * 16 + h * 8), qf[kq]);
            }
            // Park O in this unit's own q rows (every reader of them has read its phi(q)).
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 x{O[4 * q4] * inv, O[4 * q4 + 1] * inv, O[4 * q4 + 2] * inv, O[4 * q4 + 3] * inv};
                sQ.write4(qrow, ct * 32 + 8 * q4 + 4 * h, out4<T, IO>(x));
            }
        }
    };
    // Half-query items (HQ: the fp32 d = 64 staging-wave shapes whose units
    // are split over two waves): item (u, qh) takes queries 16 qh .. 16 qh + 15
    // of unit u and every output column, on the 16x16x4 fp32 instruction
    // (lane (j, kq), j = lane % 16, kq = lane / 16, supplies A[j][kq] and
    // B[kq][j]; register r of its result is row 4 kq + r, column j).  Split
    // by queries, the two items of a unit share no scores: split by output
    // columns, as unit_run does, each recomputed the unit's whole 32 x 32
    // score tile.  Instruction (s, e) takes feature 16 s + 4 kq + e in slot
    // kq, so phi(q), phi(k) and the state copy are read four features (16
    // bytes) at a time; scores come out with key 16 kt + 4 kq + r in register
    // r of lane (query j, kq), which is the B operand of O^T += V^T P as it
    // stands.
    constexpr bool HQ = sizeof(T) == 4 && D == 64 && PIPE && M::PARTS == 2 && RPC == 1 && !M::SHIFT && !DK;
    auto unit_run_hq = [&](int u, int qh, Tile<T, D> sK, Tile<T, D> sV, Tile<T, D> sQ) {
        const int g = u / CT, r = u % CT, j = r;
        const int jq = lane & 15, kq = lane >> 4;
        const int qrow = g * C + r * 32 + 16 * qh + jq;  // the query of this lane's column
        constexpr int NS = D / 16;
        const Tile<T, D> sST{smST[j]};
        // Every LDS operand is requested ahead of the matrix instructions that
        // use it: phi(q) and the diagonal tile's keys first; the value words
        // and state-copy rows of output tile ct + 1 while tile ct is computed
        // (scheduling barriers keep the compiler from sinking those reads
        // next to their first use, where each group of four instructions
        // waited for its own read).
        f32x4 bq[NS], ak[2][NS];
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) bq[s2] = *reinterpret_cast<const f32x4 *>(sQ.p + sQ.at(qrow, 16 * s2 + 4 * kq));
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2)
                ak[kt][s2] = *reinterpret_cast<const f32x4 *>(sK.p + sK.at(r * 32 + 16 * kt + jq, 16 * s2 + 4 * kq));
        float av[2][2][4];
        f32x4 as[2][NS];
        auto load_o = [&](int ct, int b) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) av[b][kt][rr] = sV.p[sV.at(r * 32 + 16 * kt + 4 * kq + rr, 16 * ct + jq)];
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2)
                as[b][s2] = *reinterpret_cast<const f32x4 *>(sST.p + sST.at(16 * ct + jq, 16 * s2 + 4 * kq));
        };
        load_o(0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // scores of the diagonal key tile, masked (key <= query), and their sum
        float pm[2][4], ds = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            f32x4 P = f32x4{};
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
                for (int e = 0; e < 4; ++e) P = __builtin_amdgcn_mfma_f32_16x16x4f32(ak[kt][s2][e], bq[s2][e], P, 0, 0, 0);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                pm[kt][rr] = 16 * kt + 4 * kq + rr <= 16 * qh + jq ? P[rr] : 0.f;
                ds += pm[kt][rr];
            }
        }
        // the state copy's part of the denominator: phi(q) . z_j
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) {
            const f32x4 zz = *reinterpret_cast<const f32x4 *>(&smZ[j][16 * s2 + 4 * kq]);
#pragma unroll
            for (int e = 0; e < 4; ++e) ds += bq[s2][e] * zz[e];
        }
        ds += __shfl_xor(ds, 16);
        ds += __shfl_xor(ds, 32);
        const float inv = normalise ? 1.f / ds : 1.f;
#pragma unroll
        for (int ct = 0; ct < NS; ++ct) {
            const int b = ct & 1;
            if (ct + 1 < NS) load_o(ct + 1, b ^ 1);
            __builtin_amdgcn_sched_barrier(0);
            // O^T[column][query]: V^T P over the diagonal tile's keys, then S_j^T phi(q)^T
            f32x4 O = f32x4{};
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) O = __builtin_amdgcn_mfma_f32_16x16x4f32(av[b][kt][rr], pm[kt][rr], O, 0, 0, 0);
#pragma unroll
            for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
                for (int e = 0; e < 4; ++e) O = __builtin_amdgcn_mfma_f32_16x16x4f32(as[b][s2][e], bq[s2][e], O, 0, 0, 0);
            // register rr is column 16 ct + 4 kq + rr of query jq: park four columns at once
            sQ.write4(qrow, 16 * ct + 4 * kq, out4<T, IO>(f32x4{O[0] * inv, O[1] * inv, O[2] * inv, O[3] * inv}));
        }
    };

    if constexpr (!PIPE) {
        const Tile<T, D> sK{smK[0]}, sV{smV[0]};
        // ---- prologue: chunk 0 staged, chunk 1 in flight
        load_all(ra, s0);
        stage_rows<T, D, C, TH, IO>(ra.k, ra.v, sK, sV, min(C, N - s0), tid);
        stage_q(ra);
        if constexpr (DK) decay_stage<C>(smDT, ra.g, tid);
        load_all(ra, s0 + C);
        lds_barrier();

        for (int c = 0; c < nch; ++c) {
            const int t0 = s0 + c * C;
            // ---- with output columns split over waves (one item per wave), the
            // item's phi(q) fragments are read now: the barrier after phase 1
            // then orders every such read before any part parks output there.
            const int u_split = w / M::PARTS;
            const bool has_split = M::PARTS > 1 && w < M::NWI && t0 + (u_split % CT) * 32 < N;
            v8 qf_split[KBD];
            if constexpr (M::PARTS > 1) {
                if (has_split) {
                    const int qrow = (u_split / CT) * C + (u_split % CT) * 32 + n;
#pragma unroll
                    for (int kq = 0; kq < KBD; ++kq) qf_split[kq] = sQ.read8(qrow, kq * 16 + h * 8);
                }
            }

            phase1(c, t0, sK, sV);
            lds_barrier();

            if constexpr (M::PARTS == 1) {
                for (int u = w; u < M::NU; u += NW) {
                    if (t0 + (u % CT) * 32 >= N) continue;  // tile entirely past the end
                    v8 qf[KBD];
                    unit_qf(u, qf, sQ);
                    unit_run(u, 0, qf, sK, sV, sQ);
                }
            } else {
                if (has_split) unit_run(u_split, (w % M::PARTS) * M::CTP, qf_split, sK, sV, sQ);
            }
            lds_barrier();

            // ---- staging of the next chunk (and the stores of this one); the
            // registers are refilled with the chunk after it
            g16 o[M::LQ];
            read_out(o);
            if (c + 1 < nch) {
                stage_rows<T, D, C, TH, IO>(ra.k, ra.v, sK, sV, min(C, N - t0 - C), tid);
                stage_q(ra);
                if constexpr (DK) decay_stage<C>(smDT, ra.g, tid);
                load_all(ra, t0 + 2 * C);  // past the segment: no access
                store_out(o, t0);
                lds_barrier();
            } else {
                store_out(o, t0);
            }
        }
    } else {
        // Staging waves (MainShape::pipe): every wave runs phase 1 for its
        // state tiles; waves 0 .. NC-1 then take the phase-2 items of chunk c
        // (from buffer c & 1), while waves NC .. NW-1 stage chunk c+1 into
        // the other buffer, store the outputs of chunk c-1 and keep chunk c+2
        // in flight (16-bit rows: chunks c+2 and c+3, in two register sets;
        // the fp32 shape measured slower with the second set).  Each role
        // runs its own loop (one pair of barriers per chunk in both), so the
        // staging registers are not live in the phase-2 code.
        constexpr int NC = M::NWC, PTH = TH - 64 * NC;
        constexpr int LKP = (M::KVG + PTH - 1) / PTH, LQP = (M::QG + PTH - 1) / PTH;
        if (__builtin_amdgcn_readfirstlane(w) >= NC) {
            const int pt = tid - 64 * NC;
            struct PSet {
                g16 k[LKP], v[LKP], q[LQP];
            };
            constexpr int NSET = sizeof(T) == 2 ? 2 : 1;  // register sets of chunks in flight
            static_assert(NSET == 2 || M::NST <= NC * M::MAXST, "one set: the state tiles sit on the first half");
            PSet sa, sb;  // two sets: sa holds the even chunks, sb the odd ones
            unsigned pqel[LQP];  // element offsets, as qel above
            int pqt[LQP];
#pragma unroll
            for (int l = 0; l < LQP; ++l) {
                const int e = pt + l * PTH;
                const int row = e / GPR, qq = e % GPR;
                pqel[l] = (unsigned)(((row / C) * N + row % C) * D + qq * U);
                pqt[l] = (M::QG % PTH == 0 || e < M::QG) ? row % C : C;
            }
            auto p_load = [&](PSet &r, int t0) {
                const int rows = rows_at(t0);
                const Rsrc rk = make_rsrc(kb + (size_t)t0 * D, rows * D * IE);
                const Rsrc rv = make_rsrc(vb + (size_t)t0 * D, rows * D * IE);
#pragma unroll
                for (int l = 0; l < LKP; ++l) {
                    const unsigned off = (unsigned)(pt + l * PTH) * GB;
                    r.k[l] = load_in<T, IO>(rk, off);
                    r.v[l] = load_in<T, IO>(rv, off);
                }
                const Rsrc rq = make_rsrc(qb + (size_t)t0 * D, rows ? (qspan - t0 * D) * IE : 0);
#pragma unroll
                for (int l = 0; l < LQP; ++l) r.q[l] = load_in_nt<T, IO>(rq, pqt[l] < rows ? pqel[l] * IE : kOutOfRange);
            };
            auto p_stage_kv = [&](const PSet &r, int b, int rows) {
                stage_rows<T, D, C, PTH, IO>(r.k, r.v, Tile<T, D>{smK[b]}, Tile<T, D>{smV[b]}, rows, pt);
            };
            auto p_stage_q = [&](const PSet &r, int b) {
                const Tile<T, D> tq{smQ[b]};
#pragma unroll
                for (int l = 0; l < LQP; ++l) {
                    const int e = pt + l * PTH;
                    if (M::QG % PTH == 0 || e < M::QG) {
                        g16 fq;
#pragma unroll
                        for (int i = 0; i < U; ++i) fq[i] = (T)IO::phi::f(Io<T, IO>::fi(r.q[l], i));
                        tq.write16(e / GPR, (e % GPR) * U, fq);
                    }
                }
            };
            // the outputs parked in the q rows of buffer b, stored as rows of chunk t_prev
            auto p_out = [&](int b, int t_prev) {
                const Tile<T, D> tq{smQ[b]};
                g16 o[LQP];
#pragma unroll
                for (int l = 0; l < LQP; ++l) {
                    const int e = pt + l * PTH;
                    const int row = (M::QG % PTH == 0 || e < M::QG) ? e / GPR : 0;
                    o[l] = *reinterpret_cast<const g16 *>(tq.p + tq.at(row, (e % GPR) * U));
                }
                const int rows = min(C, N - t_prev);
                const Rsrc ro = make_rsrc(ob + (size_t)t_prev * D, (qspan - t_prev * D) * E);
#pragma unroll
                for (int l = 0; l < LQP; ++l) buf_store16_nt<g16>(ro, pqt[l] < rows ? pqel[l] * E : kOutOfRange, o[l]);
            };
            // One chunk step (two sets); r holds chunk c+1 and is refilled
            // with chunk c+3.  The one-set loop below is the same step with
            // chunk c+2 requested, the outputs of chunk c-1 written beside
            // phase 1 (balancing the two halves), and no phase 1 (its state
            // tiles all sit on the first half: the fp32 shape).
            auto step = [&](int c, PSet &r) {
                const int t0 = s0 + c * C, nb = (c + 1) & 1;
                phase1(c, t0, Tile<T, D>{smK[c & 1]}, Tile<T, D>{smV[c & 1]});
                lds_barrier();
                // while the other waves run phase 2 (from buffer c & 1): the
                // outputs of chunk c-1 (parked in buffer nb) out, K, V and
                // phi(q) of chunk c+1 into buffer nb, chunk c+3 requested.
                // K and V are staged here rather than beside phase 1, which
                // these waves also run: per-wave clocks put the staging half
                // on the critical path of the first half-step.
                if (c >= 1) p_out(nb, t0 - C);
                if (c + 1 < nch) {
                    p_stage_kv(r, nb, min(C, N - t0 - C));
                    p_stage_q(r, nb);
                }
                p_load(r, t0 + 3 * C);  // past the segment: no access
                lds_barrier();
            };
            // ---- prologue: chunk 0 staged into buffer 0, chunks 1 .. NSET requested
            p_load(sa, s0);
            if constexpr (NSET == 2) p_load(sb, s0 + C);
            p_stage_kv(sa, 0, min(C, N - s0));
            p_stage_q(sa, 0);
            p_load(sa, s0 + NSET * C);
            lds_barrier();
            if constexpr (NSET == 2) {
                for (int c = 0; c < nch; c += 2) {
                    step(c, sb);
                    if (c + 1 < nch) step(c + 1, sa);
                }
            } else {
                for (int c = 0; c < nch; ++c) {
                    const int t0 = s0 + c * C, nb = (c + 1) & 1;
                    // beside phase 1: the outputs of chunk c-1 out, K, V of chunk c+1 in
                    if (c >= 1) p_out(nb, t0 - C);
                    if (c + 1 < nch) p_stage_kv(sa, nb, min(C, N - t0 - C));
                    lds_barrier();
                    // beside phase 2: phi(q) of chunk c+1 in, chunk c+2 requested
                    if (c + 1 < nch) {
                        p_stage_q(sa, nb);
                        p_load(sa, t0 + 2 * C);
                    }
                    lds_barrier();
                }
            }
            if (nch > 0) p_out((nch - 1) & 1, s0 + (nch - 1) * C);
        } else {
            lds_barrier();  // chunk 0 staged
            for (int c = 0; c < nch; ++c) {
                const int t0 = s0 + c * C, b = c & 1;
                const Tile<T, D> tk{smK[b]}, tv{smV[b]}, tq{smQ[b]};
                // with output columns split over waves, an item's phi(q)
                // fragments are read before the barrier after phase 1 (no part
                // parks output in the rows before then)
                const int u_split = w / M::PARTS;
                const bool has_split = M::PARTS > 1 && w < M::NWI && t0 + (u_split % CT) * 32 < N;
                v8 qf_split[KBD];
                if constexpr (M::PARTS > 1 && !HQ) {
                    if (has_split) unit_qf(u_split, qf_split, tq);
                }
                phase1(c, t0, tk, tv);
                lds_barrier();
                if constexpr (M::PARTS == 1) {
                    for (int u = w; u < M::NU; u += NC) {
                        if (t0 + (u % CT) * 32 >= N) continue;  // tile entirely past the end
                        v8 qf[KBD];
                        unit_qf(u, qf, tq);
                        unit_run(u, 0, qf, tk, tv, tq);
                    }
                } else if constexpr (HQ) {
                    // each item reads and parks only its own 16 query rows
                    if (has_split) unit_run_hq(u_split, w % 2, tk, tv, tq);
                } else {
                    if (has_split) unit_run(u_split, (w % M::PARTS) * M::CTP, qf_split, tk, tv, tq);
                }
                lds_barrier();
            }
        }
    }
    if (p == np - 1 && state_out) {
        float *so = state_out + (size_t)seq * D * D;
#pragma unroll
        for (int i = 0; i < M::MAXST; ++i) {
            const int st = M::tile_of(w, i);
            if (hb == 0 && st < M::NST) {
                const int it = st / DT, jt = st % DT;
#pragma unroll
                for (int r = 0; r < 16; ++r) so[(size_t)(it * 32 + 8 * (r / 4) + 4 * h + (r % 4)) * D + jt * 32 + n] = S[i][r];
            }
        }
    }
    if (p == np - 1 && z_out && hb == 0) {
        const int st = M::tile_of(w, 0);
        if (st < M::NST && st % DT == 0 && h == 0) z_out[(size_t)seq * D + (st / DT) * 32 + n] = zr;
    }
}

// --------------------------------------------------------- noncausal_apply
//
// One workgroup per (sequence, block of 128 tokens).  S and z are the sums
// left in slot 0 of ws; S^T goes to LDS once.  Per query head of the group,
// the block's 128 q rows are loaded as whole 16-byte row groups (coalesced),
// phi(q) is written to an LDS tile, wave w computes O^T = S^T phi(Q)^T on
// MFMA for rows 32 w .. 32 w + 31 and parks the outputs in its own rows of
// the tile, and the tile is stored as whole rows with the non-temporal hint.
// The next head's q rows are requested while the current head is computed.
template <typename T, int D, typename IO>
__global__ __launch_bounds__(kThreads) void k_noncausal_apply(const typename IO::elem *__restrict__ q,
                                                              T *__restrict__ out,
                                                              const float *__restrict__ ws, int nslots, int H,
                                                              int Hkv, int N, int G, int nblk, int normalise,
                                                              Packed pk, int seg_len)
{
    constexpr int TQ = 128;
    using Gm = Geo<T, D, 32>;
    using v8 = typename Vt<T>::v8;
    using g16 = typename Vt<T>::g16;
    constexpr int U = Gm::U, GPR = D / U;
    constexpr int QG = TQ * GPR, LQ = QG / kThreads;  // 16-byte groups of a 128-row tile, per thread
    static_assert(QG % kThreads == 0, "whole groups per thread");
    constexpr int E = (int)sizeof(T), IE = Io<T, IO>::EB, GB = Io<T, IO>::GB;  // output, input bytes
    __shared__ __attribute__((aligned(16))) T smST[D * D];
    __shared__ __attribute__((aligned(16))) T smQ[TQ * D];
    __shared__ float smZ[D];
    const Tile<T, D> sST{smST}, sQ{smQ};

    // Dense batch: blocks run over (sequence, 128-token block).  Packed batch
    // (segments of seg_len tokens, a multiple of 128): over (kv head, segment
    // of all sequences, 128-token block of the segment).
    int blk;
    size_t qbase, slot0;
    if (!pk.tab) {
        const int seq = blockIdx.x / nblk, b = seq / Hkv, gk = seq % Hkv;
        blk = blockIdx.x % nblk;
        qbase = ((size_t)b * H + (size_t)gk * G) * N * D;
        slot0 = (size_t)seq * nslots;
    } else {
        const int bps = seg_len / TQ, j = blockIdx.x % bps, rest = blockIdx.x / bps;
        const int gk = rest / pk.nsmax;
        SegLoc r;
        if (!packed_locate(pk, rest % pk.nsmax, r)) return;
        blk = r.p * bps + j;
        N = r.n;
        if (blk * TQ >= N) return;
        qbase = ((size_t)r.off * H + (size_t)gk * G * r.n) * D;
        slot0 = packed_slot0(r, gk, Hkv, 0);
    }
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, n = lane & 31;
    const int t0 = blk * TQ, rows = min(TQ, N - t0);
    const typename IO::elem *qb = q + qbase + (size_t)t0 * D;
    T *ob = out + qbase + (size_t)t0 * D;

    // raw q groups of head g's tile (rows past N, and heads past G, read zeros)
    g16 xr[LQ];
    auto load_tile = [&](int g) {
        const Rsrc rq = make_rsrc(qb + (size_t)g * N * D, g < G ? rows * D * IE : 0);
#pragma unroll
        for (int l = 0; l < LQ; ++l) xr[l] = load_in_nt<T, IO>(rq, (unsigned)(tid + l * kThreads) * GB);
    };
    load_tile(0);

    // S^T into LDS: element (row j, col i) = S[i][j].  Every thread's 16-byte
    // groups of S (and z) are requested at once, then written transposed.
    const float *S = ws + slot0 * (size_t)D * (D + 1);
    constexpr int S4 = D * D / 4, SPT = S4 / kThreads;
    static_assert(S4 % kThreads == 0 && D <= kThreads, "S in whole 16-byte groups per thread");
    f32x4 sg[SPT];
#pragma unroll
    for (int l = 0; l < SPT; ++l) sg[l] = *reinterpret_cast<const f32x4 *>(S + 4 * (tid + l * kThreads));
    const float zv = tid < D ? S[(size_t)D * D + tid] : 0.f;
#pragma unroll
    for (int l = 0; l < SPT; ++l) {
        const int e = 4 * (tid + l * kThreads), i = e / D, j0 = e % D;
#pragma unroll
        for (int x = 0; x < 4; ++x) smST[sST.at(j0 + x, i)] = (T)sg[l][x];
    }
    if (tid < D) smZ[tid] = zv;

    const Rsrc ro0 = make_rsrc(ob, rows * D * E);
    for (int g = 0; g < G; ++g) {
        // phi(q) of this head's tile into LDS, then the next head's rows requested
#pragma unroll
        for (int l = 0; l < LQ; ++l) {
            const int e = tid + l * kThreads;
            g16 f;
#pragma unroll
            for (int i = 0; i < U; ++i) f[i] = (T)IO::phi::f(Io<T, IO>::fi(xr[l], i));
            sQ.write16(e / GPR, (e % GPR) * U, f);
        }
        load_tile(g + 1);
        lds_barrier();  // (the first time also S^T and z)
        v8 qf[Gm::KBD];
        float dq = 0.f;
#pragma unroll
        for (int kb = 0; kb < Gm::KBD; ++kb) {
            qf[kb] = sQ.read8(32 * w + n, kb * 16 + h * 8);
#pragma unroll
            for (int s = 0; s < 8; ++s) dq += (float)qf[kb][s] * smZ[kb * 16 + h * 8 + s];
        }
        f32x16 O[Gm::DT];
#pragma unroll
        for (int ct = 0; ct < Gm::DT; ++ct) {
            O[ct] = f32x16{};
            const int j = ct * 32 + n;
#pragma unroll
            for (int kb = 0; kb < Gm::KBD; ++kb) mma(O[ct], sST.read8(j, kb * 16 + h * 8), qf[kb]);
        }
        dq += __shfl_xor(dq, 32);
        const float inv = normalise ? 1.f / dq : 1.f;
        // outputs into this wave's own rows of the tile (its phi(q) is in registers)
#pragma unroll
        for (int ct = 0; ct < Gm::DT; ++ct)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                f32x4 x{O[ct][4 * q4] * inv, O[ct][4 * q4 + 1] * inv, O[ct][4 * q4 + 2] * inv,
                        O[ct][4 * q4 + 3] * inv};
                sQ.write4(32 * w + n, ct * 32 + 8 * q4 + 4 * h, out4<T, IO>(x));
            }
        lds_barrier();
        // whole output rows (rows past N are out of range: not stored)
        const Rsrc ro = g == 0 ? ro0 : make_rsrc(ob + (size_t)g * N * D, rows * D * E);
#pragma unroll
        for (int l = 0; l < LQ; ++l) {
            const int e = tid + l * kThreads;
            const g16 o = *reinterpret_cast<const g16 *>(sQ.p + sQ.at(e / GPR, (e % GPR) * U));
            buf_store16_nt<g16>(ro, (unsigned)e * 16u, o);
        }
        lds_barrier();  // the tile is written again for the next head
    }
}

// ------------------------------------------------------------- decode_step
//
// One workgroup per (batch, kv head).  Thread tid owns the float4 column
// group tid % (D/4) of rows tid / (D/4) + RG * i.  All global loads are
// issued first (the state block, then k, v, z and the G query rows), so a
// step costs one memory round trip: the state is updated with phi(k)_i v_j
// in registers and written back, partial phi(q)^T S sums for 4 query heads
// at a time are reduced through LDS, and each head's denominator is one
// wave reduction.  NT: the state rows are read and written with the
// non-temporal hint (chosen when the whole state is larger than the
// memory-side cache, so that it streams rather than thrashing the cache).
template <typename T, int D, typename IO, bool NT = false>
__global__ __launch_bounds__(kThreads) void k_decode_step(float *__restrict__ state, float *__restrict__ z,
                                                          const typename IO::elem *__restrict__ q,
                                                          const typename IO::elem *__restrict__ k,
                                                          const typename IO::elem *__restrict__ v, T *__restrict__ out, int H,
                                                          int Hkv, int G, int normalise,
                                                          const float *__restrict__ gd = nullptr)
{
    constexpr int C4 = D / 4;            // float4 groups per row
    constexpr int RG = kThreads / C4;    // row groups
    constexpr int NV = D / RG;           // rows per thread
    constexpr int HB = 4;                // query heads per reduction pass
    constexpr int GMAX = 32;             // query heads staged per pass of the outer loop
    constexpr int QGR = (GMAX * D / Vt<T>::U + kThreads - 1) / kThreads;  // q groups per thread per pass
    constexpr int QPAD = QGR * kThreads * Vt<T>::U > GMAX * D ? QGR * kThreads * Vt<T>::U : GMAX * D;
    // Padded so that every thread writes its loaded group (the compiler would
    // otherwise sink a load into the branch that guards its write, behind the
    // state loads): only the first D (or G * D) entries are read.
    constexpr int KPAD = kThreads * Vt<T>::U;
    __shared__ float sk[KPAD], sv[KPAD], sz[kThreads * 4];
    __shared__ float sqf[QPAD];  // phi(q) of head g at sqf[g * D + i]
    __shared__ float sden[GMAX];
    __shared__ __attribute__((aligned(16))) float red[RG][HB][D];

    const int seq = blockIdx.x;
    const int b = seq / Hkv, gk = seq % Hkv;
    const int tid = threadIdx.x, c4 = tid % C4, rg = tid / C4, lane = tid & 63, wv = tid >> 6;
    float *Sb = state + (size_t)seq * D * D;
    const typename IO::elem *qb = q + ((size_t)b * H + (size_t)gk * G) * D;

    // The small operands first (k, v, z, the first query heads, as 16-byte
    // buffer loads that read zeros past their end), then the state rows:
    // waiting for the small ones leaves every state load in flight, and each
    // state row is updated and stored as soon as it lands, so the stores
    // overlap the remaining loads.
    using g16 = typename Vt<T>::g16;
    constexpr int U = Vt<T>::U;                             // elements per 16 bytes
    constexpr int E = Io<T, IO>::EB, GB = Io<T, IO>::GB;   // input element and raw group bytes
    const int g_first = G < GMAX ? G : GMAX;
    const unsigned off = (unsigned)tid * GB;
    const g16 kg = load_in<T, IO>(make_rsrc(k + (size_t)seq * D, D * E), off);
    const g16 vg = load_in<T, IO>(make_rsrc(v + (size_t)seq * D, D * E), off);
    // z is advanced whenever it is given, also when the output is not
    // normalised, so a state carried through such steps stays whole.
    const f32x4 zg = buf_load16<f32x4>(make_rsrc(z ? z + (size_t)seq * D : nullptr, z ? D * 4 : 0), (unsigned)tid * 16u);
    g16 qg[QGR];
    const Rsrc rq = make_rsrc(qb, g_first * D * E);
#pragma unroll
    for (int j = 0; j < QGR; ++j) qg[j] = load_in<T, IO>(rq, off + (unsigned)j * kThreads * GB);
    __builtin_amdgcn_sched_barrier(0);  // small loads stay ahead of the state loads
    f32x4 Sr[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(Sb + (size_t)(rg + RG * i) * D + 4 * c4);
        if constexpr (NT) Sr[i] = __builtin_nontemporal_load(src);
        else Sr[i] = *src;
        __builtin_amdgcn_sched_barrier(0);  // state rows issued in the order they are consumed
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
        sk[tid * U + i] = IO::phi::f(Io<T, IO>::fi(kg, i));
        sv[tid * U + i] = Io<T, IO>::fi(vg, i);
    }
#pragma unroll
    for (int j = 0; j < QGR; ++j) {
        const int e0 = (tid + j * kThreads) * U;
#pragma unroll
        for (int i = 0; i < U; ++i) sqf[e0 + i] = IO::phi::f(Io<T, IO>::fi(qg[j], i));
    }
    lds_barrier();
    // decayed sums: S and z fade by exp(g) before the token is added
    const float fade = gd ? __builtin_amdgcn_exp2f(clamp_log_decay(gd[seq]) * kLog2e) : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) sz[tid * 4 + i] = (gd ? fade * zg[i] : zg[i]) + sk[tid * 4 + i];

    const f32x4 vv{sv[4 * c4], sv[4 * c4 + 1], sv[4 * c4 + 2], sv[4 * c4 + 3]};
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (gd) Sr[i] *= fade;
        Sr[i] += sk[rg + RG * i] * vv;
        f32x4 *dst = reinterpret_cast<f32x4 *>(Sb + (size_t)(rg + RG * i) * D + 4 * c4);
        if constexpr (NT) __builtin_nontemporal_store(Sr[i], dst);
        else *dst = Sr[i];
        __builtin_amdgcn_sched_barrier(0);  // rows in load order: each store waits for its own row only
    }
    lds_barrier();
    if (z && tid < D) z[(size_t)seq * D + tid] = sz[tid];

    for (int g0 = 0; g0 < G; g0 += GMAX) {
        const int gn = G - g0 < GMAX ? G - g0 : GMAX;
        if (g0 > 0) {
            // the next GMAX query heads, requested at once as in the first pass
            const Rsrc rq2 = make_rsrc(qb + (size_t)g0 * D, gn * D * E);
#pragma unroll
            for (int j = 0; j < QGR; ++j) qg[j] = load_in<T, IO>(rq2, off + (unsigned)j * kThreads * GB);
            lds_barrier();
#pragma unroll
            for (int j = 0; j < QGR; ++j) {
                const int e0 = (tid + j * kThreads) * U;
#pragma unroll
                for (int i = 0; i < U; ++i) sqf[e0 + i] = IO::phi::f(Io<T, IO>::fi(qg[j], i));
            }
            __syncthreads();
        }
        // Denominators: wave wv reduces phi(q_g) . z for heads g = wv, wv + 4, ...
        if (normalise) {
            for (int g = wv; g < gn; g += 4) {
                float a = 0.f;
                for (int i = lane; i < D; i += 64) a += sqf[g * D + i] * sz[i];
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o);
                if (lane == 0) sden[g] = a;
            }
        }
        for (int h0 = 0; h0 < gn; h0 += HB) {
            const int nh = gn - h0 < HB ? gn - h0 : HB;
#pragma unroll
            for (int hh = 0; hh < HB; ++hh) {
                if (hh < nh) {
                    f32x4 acc{};
#pragma unroll
                    for (int i = 0; i < NV; ++i) acc += sqf[(h0 + hh) * D + rg + RG * i] * Sr[i];
                    *reinterpret_cast<f32x4 *>(&red[rg][hh][4 * c4]) = acc;
                }
            }
            __syncthreads();
            for (int e = tid; e < nh * D; e += kThreads) {
                const int hh = e / D, j = e % D;
                float num = 0.f;
#pragma unroll
                for (int r = 0; r < RG; ++r) num += red[r][hh][j];
                const float o = normalise ? num / sden[h0 + hh] : num;
                out[((size_t)b * H + (size_t)gk * G + g0 + h0 + hh) * D + j] = Io<T, IO>::out(o);
            }
            __syncthreads();
        }
    }
}


// -------------------------------------------------------------- launchers





template <typename T, int D, int C, typename IO, bool DK = false>
int run_fwd(const linattn::Plan &pl, const void *q, const void *k, const void *v, void *out, float *state_out,
            float *z_out, float *ws, int normalise, hipStream_t st, const Timing *ev, const Start &s0)
{
    // Totals pass: its own chunk size, the largest that divides the segments
    // (up to 128 tokens), independent of the main pass's chunk.
    const int c1 = totals_chunk<T, D>(pl.seg_len);
    using In = typename IO::elem;
    const In *qq = static_cast<const In *>(q);
    const In *kk = static_cast<const In *>(k);
    const In *vv = static_cast<const In *>(v);
    T *oo = static_cast<T *>(out);
    const int P = pl.segments;  // packed: the segments the launches are sized for
    const int E = D * D + D;
    const dim3 sgrid = scan_grid(D, pl.nseq);
    Packed pk{nullptr, 0, 0};
    if (record(ev, 0, st)) return LINATTN_ERR_HIP;
    if (pl.packed) {
        int *tab = reinterpret_cast<int *>(reinterpret_cast<char *>(ws) + pl.tab_off);
        hipLaunchKernelGGL(k_pack_plan, dim3(1), dim3(kThreads), 0, st, pl.cu, pl.nb, pl.N, pl.seg_len, P, tab);
        pk = Packed{tab, pl.nb, P};
    }
    // decayed sums: each slot's summed log-decay, after the slots
    float *gs = DK ? ws + (size_t)pl.nseq * pl.ws_slots * E : nullptr;
    if (pl.causal) {
        if (pl.packed) {
            if (launch_totals<T, D, IO>(c1, pl.Hkv * P, st, kk, vv, ws, pl.N, pl.seg_len, 1, pk, pl.Hkv, 1))
                return LINATTN_ERR_UNSUPPORTED;
        } else if (P > 1 && launch_totals<T, D, IO, DK>(c1, pl.nseq * (P - 1), st, kk, vv, ws, pl.N, pl.seg_len, P - 1,
                                                          Packed{nullptr, 0, 0}, 1, 1, s0.g, gs)) {
            return LINATTN_ERR_UNSUPPORTED;
        }
        if (record(ev, 1, st)) return LINATTN_ERR_HIP;
        // the scan also adds the start sums of a continuation into every slot
        if (pl.packed || P > 2 || (P == 2 && (s0.S || s0.z)))
            hipLaunchKernelGGL(k_seg_scan, sgrid, dim3(kThreads), 0, st, ws, P - 1, D, 0, (float *)nullptr,
                               (float *)nullptr, s0.S, s0.z, pk, pl.Hkv, (const float *)gs);
        if (record(ev, 2, st)) return LINATTN_ERR_HIP;
        const dim3 grid((pl.packed ? pl.Hkv : pl.nseq) * (pl.G / pl.gt) * P);
        for (int rep = 0; rep < (ev ? ev->reps : 1); ++rep) switch (pl.gt) {
#define LINATTN_MAIN(GT)                                                                                            \
    case GT:                                                                                                       \
        if constexpr (Main<T, D, C, GT>::FITS && !(DK && Main<T, D, C, GT>::SHIFT)) {                               \
            hipLaunchKernelGGL((k_causal_chunks<T, D, C, GT, IO, DK>), grid, dim3(Main<T, D, C, GT>::TH), 0, st, qq,   \
                               kk, vv, oo, (const float *)ws, state_out, z_out, pl.H, pl.Hkv, pl.N, pl.G, P,       \
                               pl.seg_len, normalise, s0.S, s0.z, pk, s0.g);                                       \
            break;                                                                                                 \
        } else {                                                                                                   \
            return LINATTN_ERR_UNSUPPORTED;                                                                        \
        }
            LINATTN_MAIN(1)
            LINATTN_MAIN(2)
            LINATTN_MAIN(4)
            LINATTN_MAIN(8)
#undef LINATTN_MAIN
        default: return LINATTN_ERR_UNSUPPORTED;
        }
    } else if constexpr (DK) {
        return LINATTN_ERR_UNSUPPORTED;  // decayed sums are causal only
    } else {
        if (launch_totals<T, D, IO>(c1, (pl.packed ? pl.Hkv : pl.nseq) * P, st, kk, vv, ws, pl.N, pl.seg_len, P, pk,
                                pl.Hkv, 0))
            return LINATTN_ERR_UNSUPPORTED;
        if (record(ev, 1, st)) return LINATTN_ERR_HIP;
        hipLaunchKernelGGL(k_seg_scan, sgrid, dim3(kThreads), 0, st, ws, P, D, 1, state_out, z_out, s0.S, s0.z, pk,
                           pl.Hkv);
        if (record(ev, 2, st)) return LINATTN_ERR_HIP;
        const int nblk = (pl.N + 127) / 128;
        const unsigned grid = pl.packed ? (unsigned)(pl.Hkv * P * (pl.seg_len / 128)) : (unsigned)(pl.nseq * nblk);
        for (int rep = 0; rep < (ev ? ev->reps : 1); ++rep)
            hipLaunchKernelGGL((k_noncausal_apply<T, D, IO>), dim3(grid), dim3(kThreads), 0, st, qq, oo,
                               (const float *)ws, P, pl.H, pl.Hkv, pl.N, pl.G, nblk, normalise, pk, pl.seg_len);
    }
    if (record(ev, 3, st)) return LINATTN_ERR_HIP;
    return launch_status();
}

template <typename T, int D, int C>
constexpr bool chunk_ok()
{
    return Main<T, D, C, 1>::FITS || Main<T, D, C, 2>::FITS || Main<T, D, C, 4>::FITS || Main<T, D, C, 8>::FITS;
}

template <typename T, int D, typename IO, bool DK = false>
int dispatch_chunk(const linattn::Plan &pl, const void *q, const void *k, const void *v, void *out,
                   float *state_out, float *z_out, float *ws, int normalise, hipStream_t st, const Timing *ev,
                   const Start &s0)
{
    switch (pl.chunk) {
    case 32:
        if constexpr (chunk_ok<T, D, 32>()) return run_fwd<T, D, 32, IO, DK>(pl, q, k, v, out, state_out, z_out, ws, normalise, st, ev, s0);
        break;
    case 64:
        if constexpr (chunk_ok<T, D, 64>()) return run_fwd<T, D, 64, IO, DK>(pl, q, k, v, out, state_out, z_out, ws, normalise, st, ev, s0);
        break;
    case 128:
        if constexpr (chunk_ok<T, D, 128>()) return run_fwd<T, D, 128, IO, DK>(pl, q, k, v, out, state_out, z_out, ws, normalise, st, ev, s0);
        break;
    case 256:
        if constexpr (chunk_ok<T, D, 256>()) return run_fwd<T, D, 256, IO, DK>(pl, q, k, v, out, state_out, z_out, ws, normalise, st, ev, s0);
        break;
    }
    return LINATTN_ERR_UNSUPPORTED;
}

template <typename T, typename IO = Fmt<T, PhiElu1>, bool DK = false>
int dispatch_d(const linattn::Plan &pl, const void *q, const void *k, const void *v, void *out,
               float *state_out, float *z_out, float *ws, int normalise, hipStream_t st, const Timing *ev,
               const Start &s0)
{
    switch (pl.d) {
    case 32: return dispatch_chunk<T, 32, IO, DK>(pl, q, k, v, out, state_out, z_out, ws, normalise, st, ev, s0);
    case 64: return dispatch_chunk<T, 64, IO, DK>(pl, q, k, v, out, state_out, z_out, ws, normalise, st, ev, s0);
    case 128: return dispatch_chunk<T, 128, IO, DK>(pl, q, k, v, out, state_out, z_out, ws, normalise, st, ev, s0);
    }
    return LINATTN_ERR_UNSUPPORTED;
}


template <typename T, typename IO = Fmt<T, PhiElu1>>
int run_decode(float *state, float *z, const void *q, const void *k, const void *v, const float *g, void *out, int B,
               int H, int Hkv, int d, int normalise, hipStream_t st)
{
    const int G = H / Hkv;
    const dim3 grid(B * Hkv), block(kThreads);
    using In = typename IO::elem;
    const In *qq = static_cast<const In *>(q);
    const In *kk = static_cast<const In *>(k);
    const In *vv = static_cast<const In *>(v);
    T *oo = static_cast<T *>(out);
    // A state larger than the 256 MiB memory-side cache cannot stay there
    // between steps: it is streamed with the non-temporal hint (batch 1024 of
    // 8 kv heads at d = 128: 220 -> 190 us per step), a smaller one is read
    // and written plainly so that it stays cached (the hint cost batch 64
    // 10.7 -> 13.0 us per step).
    const bool nt = (size_t)B * Hkv * d * d * 4 > ((size_t)256 << 20);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, block, 0, st, state, z, qq, kk, vv, oo, H, Hkv, G, normalise, g);
    };
    switch (d) {
    case 32: nt ? go(k_decode_step<T, 32, IO, true>) : go(k_decode_step<T, 32, IO>); break;
    case 64: nt ? go(k_decode_step<T, 64, IO, true>) : go(k_decode_step<T, 64, IO>); break;
    case 128: nt ? go(k_decode_step<T, 128, IO, true>) : go(k_decode_step<T, 128, IO>); break;
    default: return LINATTN_ERR_UNSUPPORTED;
    }
    return launch_status();
}

}  // namespace

// ----------------------------------------------- this object's format
namespace {
template <int PHI> struct PhiOf;
template <> struct PhiOf<LINATTN_PHI_ELU1> { using type = PhiElu1; };
template <> struct PhiOf<LINATTN_PHI_RELU> { using type = PhiRelu; };
template <> struct PhiOf<LINATTN_PHI_SOFTPLUS> { using type = PhiSoftplus; };
// element type in memory -> (operand type, row format)
template <int ELEM, typename P> struct ElemOf;
template <typename P> struct ElemOf<LINATTN_F32, P> { using T = float; using IO = Fmt<float, P>; };
template <typename P> struct ElemOf<LINATTN_BF16, P> { using T = bf16; using IO = Fmt<bf16, P>; };
template <typename P> struct ElemOf<LINATTN_F16, P> { using T = bf16; using IO = Fmt<f16, P>; };
template <typename P> struct ElemOf<LINATTN_FP8_E4M3, P> { using T = bf16; using IO = Fmt<fp8e4m3, P>; };
template <typename P> struct ElemOf<LINATTN_FP8_E5M2, P> { using T = bf16; using IO = Fmt<fp8e5m2, P>; };
using Phi = PhiOf<LINATTN_FMT_PHI>::type;
using K = ElemOf<LINATTN_FMT_ELEM, Phi>;
}  // namespace

namespace linattn {

template <>
int fwd_format<LINATTN_FMT_PHI, LINATTN_FMT_ELEM>(const FwdCall &c)
{
    if (c.s0.g) {
        // decayed sums are built for the default feature map only (decay_ok)
        if constexpr (std::is_same_v<Phi, PhiElu1>)
            return dispatch_d<K::T, K::IO, true>(*c.pl, c.q, c.k, c.v, c.out, c.state_out, c.z_out, c.ws,
                                                 c.normalise, c.stream, c.ev, c.s0);
        else
            return LINATTN_ERR_UNSUPPORTED;
    }
    return dispatch_d<K::T, K::IO>(*c.pl, c.q, c.k, c.v, c.out, c.state_out, c.z_out, c.ws, c.normalise, c.stream,
                                   c.ev, c.s0);
}

template <>
int decode_format<LINATTN_FMT_PHI, LINATTN_FMT_ELEM>(const DecodeCall &c)
{
    return run_decode<K::T, K::IO>(c.state, c.z, c.q, c.k, c.v, c.g, c.out, c.B, c.H, c.Hkv, c.d, c.normalise,
                                   c.stream);
}

template <>
int window_format<LINATTN_FMT_PHI, LINATTN_FMT_ELEM>(const WindowCall &c)
{
    return run_window<K::T, K::IO>(c.q, c.k, c.v, c.out, c.B, c.H, c.Hkv, c.N, c.d, c.window, c.normalise,
                                   c.stream);
}

}  // namespace linattn
