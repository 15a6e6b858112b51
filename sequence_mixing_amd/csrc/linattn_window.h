// linattn_window.h - sliding-window causal linear attention on gfx950.
//
// Reading of the LinearTile 1.0.0 README's "Features" list, sliding-window
// item (the pages give no definition): query t sees the keys of the causal
// band t - W < s <= t,
//     o_t = sum_{band} (phi(q_t) . phi(k_s)) v_s / sum_{band} phi(q_t) . phi(k_s)
// (numerator only when not normalised).  The band is computed as it stands,
// masked scores times values on the matrix cores, like the intra-chunk term
// of the chunked pass: there is no running state to subtract from (S_t -
// S_{t-W} of two running sums would cancel in fp32 once t >> W), and no
// carry between workgroups, so every (query head, 128-row query tile) is an
// independent workgroup.  The cost is O(N * min(W, N) * d) per head.
#pragma once
#include "linattn_kern.h"

namespace {

template <typename T, int D>
struct Win {
    static constexpr int TQ = 128;                     // query rows per workgroup: one 32-row tile per wave
    static constexpr int U = Vt<T>::U, GPR = D / U, DT = D / 32, KBD = D / 16;
    static constexpr int QG = TQ * GPR;                // 16-byte q groups of the query tile
    static constexpr int LQ = (QG + kThreads - 1) / kThreads;
    static constexpr int KG = 32 * GPR;                // 16-byte groups of one 32-key tile
    static constexpr int LK = (KG + kThreads - 1) / kThreads;
    // key tiles in flight in registers (16-bit rows: three at d <= 64, two
    // at d = 128, with the registers of 4, 3 and 2 workgroups per CU at d = 32,
    // 64 and 128; fp32 rows: two, occupancy left to the compiler)
    static constexpr bool B16 = sizeof(T) == 2;
    static constexpr int NS = B16 && D <= 64 ? 3 : 2;
    static constexpr int OCC = !B16 ? 1 : D <= 32 ? 4 : D <= 64 ? 3 : 2;
};

// One workgroup per (batch, query head, 128-query tile).  Key tiles of 32
// tokens covering the workgroup's band are staged (phi(K), V) into LDS, two
// buffers, the next tile's loads in flight while the current one is used.
// Wave w owns queries q0 = t0 + 32 w .. q0 + 31 and skips key tiles outside
// its band.  Per key tile: Pt = phi(K) phi(Q)^T (MFMA), the band mask (a
// select, so masked non-finite scores do not leak), the denominator's row
// sums, and O^T += V^T Pt (MFMA).  The outputs are parked in the wave's own
// q rows and stored as whole rows.
template <typename T, int D, typename IO>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(Win<T, D>::OCC))) void k_window(const typename IO::elem *__restrict__ q,
                                                     const typename IO::elem *__restrict__ k,
                                                     const typename IO::elem *__restrict__ v, T *__restrict__ out,
                                                     int H, int Hkv, int N, int W, int normalise, int nqt)
{
    using Wn = Win<T, D>;
    using v8 = typename Vt<T>::v8;
    using g16 = typename Vt<T>::g16;
    constexpr bool BF = sizeof(T) == 2;
    constexpr int U = Wn::U, GPR = Wn::GPR, DT = Wn::DT, KBD = Wn::KBD, TQ = Wn::TQ;
    constexpr int E = (int)sizeof(T), IE = Io<T, IO>::EB, GB = Io<T, IO>::GB;  // output, input bytes
    __shared__ __attribute__((aligned(16))) T smQ[TQ * D];
    __shared__ __attribute__((aligned(16))) T smK[2][32 * D];
    __shared__ __attribute__((aligned(16))) T smV[2][32 * D];
    const Tile<T, D> sQ{smQ};

    const int bh = blockIdx.x / nqt, qt = blockIdx.x % nqt;
    const int b = bh / H, hq = bh % H, g = hq / (H / Hkv);
    using In = typename IO::elem;
    const In *qb = q + (size_t)bh * N * D;
    T *ob = out + (size_t)bh * N * D;
    const size_t kvb = ((size_t)b * Hkv + g) * N * D;
    const In *kb = k + kvb, *vb = v + kvb;
    const int t0 = qt * TQ, qrows = min(TQ, N - t0);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, n = lane & 31;

    // phi(q) of the query tile into LDS (rows past N read zeros)
    {
        const Rsrc rq = make_rsrc(qb + (size_t)t0 * D, qrows * D * IE);
        g16 r[Wn::LQ];
#pragma unroll
        for (int l = 0; l < Wn::LQ; ++l) {
            const int e = tid + l * kThreads;
            r[l] = load_in<T, IO>(rq, (Wn::QG % kThreads == 0 || e < Wn::QG) ? (unsigned)e * GB : kOutOfRange);
        }
#pragma unroll
        for (int l = 0; l < Wn::LQ; ++l) {
            const int e = tid + l * kThreads;
            if (Wn::QG % kThreads == 0 || e < Wn::QG) {
                g16 f;
#pragma unroll
                for (int i = 0; i < U; ++i) f[i] = (T)IO::phi::f(Io<T, IO>::fi(r[l], i));
                sQ.write16(e / GPR, (e % GPR) * U, f);
            }
        }
    }

    // key tiles of the workgroup's band: keys max(0, t0 - W + 1) .. t0 + qrows - 1
    const int kt0 = max(0, t0 - W + 1) / 32, kt1 = (t0 + qrows - 1) / 32;
    auto rows_of = [&](int kt) { return kt <= kt1 ? min(32, N - kt * 32) : 0; };
    // NS register sets: key tile kt waits in set (kt - kt0) % NS from NS
    // steps before its staging (one step left the loads' round trip exposed).
    constexpr int NS = Wn::NS;
    g16 kr[NS][Wn::LK], vr[NS][Wn::LK];
    auto load_kv = [&](int u, int kt) {  // past the band: nothing is read
        const int rows = rows_of(kt);
        const Rsrc rk = make_rsrc(kb + (size_t)kt * 32 * D, rows * D * IE);
        const Rsrc rv = make_rsrc(vb + (size_t)kt * 32 * D, rows * D * IE);
#pragma unroll
        for (int l = 0; l < Wn::LK; ++l) {
            const int e = tid + l * kThreads;
            const unsigned off = (Wn::KG % kThreads == 0 || e < Wn::KG) ? (unsigned)e * GB : kOutOfRange;
            kr[u][l] = load_in<T, IO>(rk, off);
            vr[u][l] = load_in<T, IO>(rv, off);
        }
    };
#pragma unroll
    for (int u = 0; u < NS; ++u) load_kv(u, kt0 + u);
    stage_rows<T, D, 32, kThreads, IO>(kr[0], vr[0], Tile<T, D>{smK[0]}, Tile<T, D>{smV[0]}, rows_of(kt0), tid);
    load_kv(0, kt0 + NS);
    lds_barrier();

    const int q0 = t0 + 32 * w;
    const bool live = q0 < t0 + qrows;
    v8 qf[KBD];
#pragma unroll
    for (int kq = 0; kq < KBD; ++kq) qf[kq] = sQ.read8(32 * w + n, kq * 16 + h * 8);
    f32x16 O[DT];
#pragma unroll
    for (int ct = 0; ct < DT; ++ct) O[ct] = f32x16{};
    f32x16 Dn = f32x16{};
    float ds = 0.f;
    const int t = q0 + n;  // this lane's query

    // Step kt uses LDS buffer (kt - kt0) & 1 and stages tile kt + 1 from
    // register set (kt + 1 - kt0) % NS into the other; steps in groups of
    // lcm(NS, 2) so that both indices are fixed.
    auto step = [&](int kt, const int buf, const int nset) {
        const Tile<T, D> tK{smK[buf]}, tV{smV[buf]};
        const int ks = kt * 32;
        if (live && ks <= q0 + 31 && ks + 31 > q0 - W) {
            f32x16 Pt = f32x16{};
#pragma unroll
            for (int kq = 0; kq < KBD; ++kq) mma(Pt, tK.read8(n, kq * 16 + h * 8), qf[kq]);
            // accumulator reg i holds key ks + 8(i/4) + 4h + i%4 for query t
            float pv[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int s = ks + 8 * (i / 4) + 4 * h + (i % 4);
                pv[i] = (s <= t && s > t - W) ? Pt[i] : 0.f;
            }
            const v8 pb0 = cvt8<T>(pv), pb1 = cvt8<T>(pv + 8);
            if constexpr (BF) {
                mma(Dn, ones8<T>(), pb0);
                mma(Dn, ones8<T>(), pb1);
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s) ds += pb0[s] + pb1[s];
            }
#pragma unroll
            for (int ct = 0; ct < DT; ++ct) {
                mma(O[ct], colfrag(tV, 4 * h, 8 + 4 * h, ct * 32, lane), pb0);
                mma(O[ct], colfrag(tV, 16 + 4 * h, 24 + 4 * h, ct * 32, lane), pb1);
            }
        }
        if (kt < kt1) {
            // the next tile into the other buffer (last read before the previous barrier)
            stage_rows<T, D, 32, kThreads, IO>(kr[nset], vr[nset], Tile<T, D>{smK[buf ^ 1]},
                                               Tile<T, D>{smV[buf ^ 1]}, rows_of(kt + 1), tid);
            load_kv(nset, kt + 1 + NS);
        }
        lds_barrier();
    };
    constexpr int GRP = NS % 2 ? 2 * NS : NS;
    for (int kt = kt0; kt <= kt1; kt += GRP) {
#pragma unroll
        for (int j = 0; j < GRP; ++j)
            if (kt + j <= kt1) step(kt + j, j & 1, (j + 1) % NS);
    }

    // outputs into this wave's own q rows, then whole rows out
    const float den = BF ? Dn[0] : ds + __shfl_xor(ds, 32);
    const float inv = normalise && live ? 1.f / den : 1.f;
#pragma unroll
    for (int ct = 0; ct < DT; ++ct)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 x{O[ct][4 * q4] * inv, O[ct][4 * q4 + 1] * inv, O[ct][4 * q4 + 2] * inv, O[ct][4 * q4 + 3] * inv};
            sQ.write4(32 * w + n, ct * 32 + 8 * q4 + 4 * h, out4<T, IO>(x));
        }
    lds_barrier();
    const Rsrc ro = make_rsrc(ob + (size_t)t0 * D, qrows * D * E);
#pragma unroll
    for (int l = 0; l < Wn::LQ; ++l) {
        const int e = tid + l * kThreads;
        const bool in = Wn::QG % kThreads == 0 || e < Wn::QG;
        const g16 o = *reinterpret_cast<const g16 *>(sQ.p + sQ.at(in ? e / GPR : 0, (e % GPR) * U));
        buf_store16<g16>(ro, in ? (unsigned)e * 16u : kOutOfRange, o);
    }
}

template <typename T, typename IO>
int run_window(const void *q, const void *k, const void *v, void *out, int B, int H, int Hkv, int N, int d, int W,
               int normalise, hipStream_t st)
{
    const int nqt = (N + Win<T, 64>::TQ - 1) / Win<T, 64>::TQ;
    const dim3 grid((unsigned)((size_t)B * H * nqt)), block(kThreads);
    using In = typename IO::elem;
    const In *qq = static_cast<const In *>(q), *kk = static_cast<const In *>(k), *vv = static_cast<const In *>(v);
    T *oo = static_cast<T *>(out);
    switch (d) {
    case 32: hipLaunchKernelGGL((k_window<T, 32, IO>), grid, block, 0, st, qq, kk, vv, oo, H, Hkv, N, W, normalise, nqt); break;
    case 64: hipLaunchKernelGGL((k_window<T, 64, IO>), grid, block, 0, st, qq, kk, vv, oo, H, Hkv, N, W, normalise, nqt); break;
    case 128: hipLaunchKernelGGL((k_window<T, 128, IO>), grid, block, 0, st, qq, kk, vv, oo, H, Hkv, N, W, normalise, nqt); break;
    default: return LINATTN_ERR_UNSUPPORTED;
    }
    return launch_status();
}

}  // namespace
