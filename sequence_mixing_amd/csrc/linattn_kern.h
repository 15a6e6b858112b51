// linattn_kern.h - device building blocks shared by the forward and the
// backward kernels of liblinattn.so (gfx950): buffer accesses, MFMA operand
// fragments, swizzled LDS tiles, phi, and the segment totals / scan passes
// that carry a d x d running sum across workgroups.  Internal header: every
// definition has internal linkage in each translation unit that includes it.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "linattn.h"

namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// ------------------------------------------------------- buffer accesses
//
// Raw buffer loads/stores through a scalar descriptor (base, size in bytes).
// The hardware checks every lane's byte offset against the size: loads out
// of range return zero and stores out of range are dropped.  Tails and
// masked lanes therefore need no branches, every staging step issues the
// same instructions, and the compiler can wait for exactly the loads a step
// consumes while later ones stay in flight.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr unsigned kOutOfRange = 0x80000000u;  // beyond every size used here (< 2^31)

__device__ __forceinline__ Rsrc make_rsrc(const void *base, int bytes)
{
    // Word 3: 32-bit data format (raw access, no swizzle, no format conversion).
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}
template <typename G> __device__ __forceinline__ G buf_load16(Rsrc r, unsigned off)
{
    static_assert(sizeof(G) == 16, "16-byte group");
    return __builtin_bit_cast(G, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
template <typename G> __device__ __forceinline__ void buf_store16(Rsrc r, unsigned off, G x)
{
    static_assert(sizeof(G) == 16, "16-byte group");
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}

// The same with the non-temporal hint (cache policy bit nt): for rows that
// are written once and not read again by the kernels that follow.
template <typename G> __device__ __forceinline__ void buf_store16_nt(Rsrc r, unsigned off, G x)
{
    static_assert(sizeof(G) == 16, "16-byte group");
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 2);
}

// Workgroup barrier for LDS hand-offs only.  __syncthreads() also drains
// every outstanding global load (vmcnt), which would stall the register
// prefetch of the next chunk at each barrier; here only LDS traffic
// (lgkmcnt) is waited for, and the prefetched loads stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ----------------------------------------------------------- feature maps
//
// phi is a template functor of every kernel (README "Features": custom
// kernel plugins, phi replaceable): f(x), and phi'(x) written as a function of
// phi(x) (df), which is what the backward keeps.  A new map is a struct with
// these two members plus a code in the dispatch.
//
// ELU(x) + 1 (alpha = 1), the README's phi: x + 1 for x > 0, exp(x) otherwise,
// as a select between the two (one v_exp_f32, no branch); phi' = 1 for x > 0,
// exp(x) = phi otherwise, i.e. min(1, phi).  Both are written so that NaN
// propagates (a NaN input gives NaN: fmaxf / fminf would turn it into 0).
struct PhiElu1 {
    static __device__ __forceinline__ float f(float x)
    {
        const float e = __builtin_amdgcn_exp2f(x * 1.44269504088896340736f);
        return x > 0.f ? x + 1.f : e;
    }
    static __device__ __forceinline__ float df(float y) { return y >= 1.f ? 1.f : y; }
};
// ReLU: max(x, 0); phi' = 1 where phi > 0.  (A normalised row whose query or
// keys are all <= 0 divides by zero.)  NaN propagates through both.
struct PhiRelu {
    static __device__ __forceinline__ float f(float x) { return x > 0.f || x != x ? x : 0.f; }
    static __device__ __forceinline__ float df(float y) { return y > 0.f ? 1.f : (y == y ? 0.f : y); }
};
// softplus: log(1 + e^x) = max(x, 0) + log1p(e^-|x|); phi' = the logistic
// function = 1 - e^-phi (written -expm1(-phi), exact for small phi).
struct PhiSoftplus {
    static __device__ __forceinline__ float f(float x) { return fmaxf(x, 0.f) + log1pf(__expf(-fabsf(x))); }
    static __device__ __forceinline__ float df(float y) { return -expm1f(-y); }
};

// Row format and feature map of a kernel instance: element type in memory
// (float, bf16 or fp16) and phi.
template <typename E, typename P> struct Fmt {
    using elem = E;
    using phi = P;
};

// ------------------------------------------------------------------ types

template <typename E> struct Vt;
template <> struct Vt<bf16> {
    using v8 = bf16x8;  // 8 consecutive elements: one MFMA operand fragment
    using v4 = bf16x4;
    using g16 = bf16x8; // one 16-byte group
    static constexpr int U = 8;  // elements per 16 bytes
};
template <> struct Vt<float> {
    using v8 = f32x8;
    using v4 = f32x4;
    using g16 = f32x4;
    static constexpr int U = 4;
};

// acc += A(32 x 16) * B(16 x 32) for one K-block of 16.
__device__ __forceinline__ void mma(f32x16 &acc, const bf16x8 &a, const bf16x8 &b)
{
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x16 &acc, const f32x8 &a, const f32x8 &b)
{
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 cat(const bf16x4 &a, const bf16x4 &b)
{
    return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f32x8 cat(const f32x4 &a, const f32x4 &b)
{
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ------------------------------------------------------------ input/output
//
// Rows in memory may be fp16 or fp8 while the matrix-core operands of the
// 16-bit kernels are bf16 (T = bf16, IO = fp16 or fp8): bf16 keeps fp32's
// exponent range, so the operand copies of the running sums (which grow with
// the sequence) stay finite where fp16 would overflow, and it holds every fp8
// value exactly.  Registers hold the raw input groups (one load each: 16 bytes
// of 2- or 4-byte elements, 8 bytes of fp8, U elements either way); these
// convert them at the staging that writes them to LDS.  IO is a Fmt (below);
// its element type equal to T is the plain case.
typedef _Float16 f16;
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// fp8 rows (README "Features": mixed precision; the OCP 8-bit formats MI355X
// uses): E4M3 (bias 7, no infinities, S.1111.111 is NaN, largest 448) and
// E5M2 (bias 15, IEEE-like infinities and NaN).  One byte each.
struct fp8e4m3 {
    unsigned char b;
};
struct fp8e5m2 {
    unsigned char b;
};
template <typename E> constexpr bool is_fp8 = std::is_same_v<E, fp8e4m3> || std::is_same_v<E, fp8e5m2>;

// The value of an fp8 code, exactly, from the formats' definitions.
__device__ __forceinline__ float fp8_value(unsigned b, fp8e4m3)
{
    const unsigned e = (b >> 3) & 15u, m = b & 7u;
    // normal: (1 + m/8) 2^(e-7), i.e. fp32 exponent e + 120; subnormal (e = 0): m 2^-9
    const float normal = __uint_as_float(((e + 120u) << 23) | (m << 20));
    const float sub = (float)m * 0x1p-9f;
    float x = e ? normal : sub;
    x = (e == 15u && m == 7u) ? __builtin_nanf("") : x;
    return __uint_as_float(__float_as_uint(x) | ((b & 0x80u) << 24));
}
__device__ __forceinline__ float fp8_value(unsigned b, fp8e5m2)
{
    // E5M2 is the upper byte of an IEEE fp16 (same exponent width and bias)
    return (float)__builtin_bit_cast(f16, (unsigned short)(b << 8));
}

template <typename T, typename IO> struct Io {
    using E = typename IO::elem;
    static_assert(std::is_same_v<T, E> || (std::is_same_v<T, bf16> && (std::is_same_v<E, f16> || is_fp8<E>)),
                  "I/O type");
    static constexpr bool SAME = std::is_same_v<T, E>;
    static constexpr bool FP8 = is_fp8<E>;
    static constexpr int EB = (int)sizeof(E);       // bytes of one input element in memory
    static constexpr int GB = Vt<T>::U * EB;         // bytes of one raw input group
    // output elements: the input format, except bf16 for fp8 rows
    using OutE = std::conditional_t<FP8, bf16, E>;
    static constexpr int OB = (int)sizeof(OutE);
    // element i of a raw input group -> float
    static __device__ __forceinline__ float fi(const typename Vt<T>::g16 &g, int i)
    {
        if constexpr (FP8) {
            const u32x4 w = __builtin_bit_cast(u32x4, g);
            return fp8_value((w[i >> 2] >> (8 * (i & 3))) & 0xffu, E{});
        } else {
            // the element is copied out first: a bit cast of the vector
            // element expression itself reads element 0
            const T x = g[i];
            if constexpr (SAME) return (float)x;
            else return (float)__builtin_bit_cast(E, x);
        }
    }
    // float -> the stored output element (its bits in a T)
    static __device__ __forceinline__ T out(float x)
    {
        if constexpr (SAME || FP8) return (T)x;
        else return __builtin_bit_cast(T, (E)x);
    }
};

// A row pointer held as the operand type, seen as the memory element type
// (the same bytes; fp16 rows travel in bf16-typed storage).
template <typename IO, typename T> __device__ __host__ __forceinline__ const typename IO::elem *in_ptr(const T *p)
{
    return reinterpret_cast<const typename IO::elem *>(p);
}

// One raw input group at a byte offset of a buffer (offsets out of range read
// zeros, as for every buffer load here).
template <typename T, typename IO>
__device__ __forceinline__ typename Vt<T>::g16 load_in(Rsrc r, unsigned off)
{
    if constexpr (Io<T, IO>::FP8) {
        const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
        return __builtin_bit_cast(typename Vt<T>::g16, u32x4{x[0], x[1], 0u, 0u});
    } else {
        return buf_load16<typename Vt<T>::g16>(r, off);
    }
}

// The same with the non-temporal hint: for rows read once.
template <typename T, typename IO>
__device__ __forceinline__ typename Vt<T>::g16 load_in_nt(Rsrc r, unsigned off)
{
    if constexpr (Io<T, IO>::FP8) {
        const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2));
        return __builtin_bit_cast(typename Vt<T>::g16, u32x4{x[0], x[1], 0u, 0u});
    } else {
        return __builtin_bit_cast(typename Vt<T>::g16, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
    }
}

template <typename E> __device__ __forceinline__ typename Vt<E>::v8 cvt8(const float *x);
template <> __device__ __forceinline__ bf16x8 cvt8<bf16>(const float *x)
{
    f32x8 f{x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
    return __builtin_convertvector(f, bf16x8);
}
template <> __device__ __forceinline__ f32x8 cvt8<float>(const float *x)
{
    return f32x8{x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
}
template <typename E> __device__ __forceinline__ typename Vt<E>::v4 cvt4(f32x4 x);
template <> __device__ __forceinline__ bf16x4 cvt4<bf16>(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
template <> __device__ __forceinline__ f32x4 cvt4<float>(f32x4 x) { return x; }

// Four results -> four stored output elements of I/O type IO (in T-typed storage).
template <typename T, typename IO> __device__ __forceinline__ typename Vt<T>::v4 out4(f32x4 x)
{
    if constexpr (std::is_same_v<T, typename IO::elem> || Io<T, IO>::FP8) return cvt4<T>(x);
    else return __builtin_bit_cast(bf16x4, __builtin_convertvector(x, f16x4));
}
// A raw input group of IO elements -> the same values as operands of type T.
template <typename T, typename IO> __device__ __forceinline__ typename Vt<T>::g16 op16(const typename Vt<T>::g16 &g)
{
    if constexpr (std::is_same_v<T, typename IO::elem>) {
        return g;
    } else {
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = Io<T, IO>::fi(g, i);
        return cvt8<T>(x);
    }
}

// ---------------------------------------------------------- LDS tiles
//
// Row-major tiles whose 16-byte groups are XOR-permuted per row: element
// (r, c) lives at r * COLS + (c ^ (sig(r) * U)), sig(r) = r % (COLS / U).
// Runs of 4 or 8 elements starting on a 4-aligned column stay contiguous
// (an fp32 8-run spans two groups and is read as two), and both row walks
// and column walks spread over the LDS banks.

template <typename E, int COLS>
struct Tile {
    E *p;
    static constexpr int U = Vt<E>::U;
    static constexpr int NG = COLS / U;
    __device__ __forceinline__ static int sig(int r) { return r % NG; }
    __device__ __forceinline__ int at(int r, int c) const { return r * COLS + (c ^ (sig(r) * U)); }
    __device__ __forceinline__ typename Vt<E>::v8 read8(int r, int c) const
    {
        if constexpr (U == 8) {
            return *reinterpret_cast<const bf16x8 *>(p + at(r, c));
        } else {
            return cat(*reinterpret_cast<const f32x4 *>(p + at(r, c)), *reinterpret_cast<const f32x4 *>(p + at(r, c + 4)));
        }
    }
    __device__ __forceinline__ void write4(int r, int c, typename Vt<E>::v4 x) const
    {
        *reinterpret_cast<typename Vt<E>::v4 *>(p + at(r, c)) = x;
    }
    __device__ __forceinline__ typename Vt<E>::v4 read4(int r, int c) const
    {
        return *reinterpret_cast<const typename Vt<E>::v4 *>(p + at(r, c));
    }
    __device__ __forceinline__ void write16(int r, int c, typename Vt<E>::g16 x) const
    {
        *reinterpret_cast<typename Vt<E>::g16 *>(p + at(r, c)) = x;
    }
};

// Column fragment of an MFMA operand out of a row-major tile: lane
// (h = lane/32, x = lane%32) gets rows ra + e and rb + e (e = 0..3; ra, rb
// depend on h only) of column col + x, as slots 0..3 and 4..7.
//
// bf16 uses ds_read_b64_tr_b16: inside each 16-lane group, lane j receives
// element j%4 of the 8-byte reads issued by lanes j/4, j/4+4, j/4+8, j/4+12,
// so lane j supplies the address of row r0 + j/4, columns c0 + 4(j%4).
// fp32 reads one word per slot (32 lanes walk consecutive columns).
template <int COLS>
__device__ __forceinline__ bf16x8 colfrag(const Tile<bf16, COLS> &t, int ra, int rb, int col, int lane)
{
    const int j = lane & 15;
    const int c0 = col + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
    typedef __attribute__((address_space(3))) bf16x4 *lds4;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4)(t.p + t.at(ra + (j >> 2), c0)));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4)(t.p + t.at(rb + (j >> 2), c0)));
    return cat(lo, hi);
}
template <int COLS>
__device__ __forceinline__ f32x8 colfrag(const Tile<float, COLS> &t, int ra, int rb, int col, int lane)
{
    const int c = col + (lane & 31);
    f32x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = t.p[t.at(ra + e, c)];
        r[4 + e] = t.p[t.at(rb + e, c)];
    }
    return r;
}

// Shapes shared by the chunk kernels.
template <typename T, int D, int C>
struct Geo {
    static constexpr int U = Vt<T>::U;       // elements per 16 bytes (one global vector load)
    static constexpr int DT = D / 32;        // 32-wide feature tiles
    static constexpr int CT = C / 32;        // 32-row token tiles per chunk
    static constexpr int KBD = D / 16;       // K-blocks over features
    static constexpr int NST = DT * DT;      // 32x32 state tiles
    static constexpr int MAXST = (NST + 3) / 4;  // state tiles per wave
    static constexpr int GPR = D / U;        // 16-byte groups per token row
    static constexpr int NGRP = C * GPR;     // 16-byte groups per chunk per tensor
    static constexpr int LDV = (NGRP + kThreads - 1) / kThreads;  // groups per thread
    static constexpr int QV = 8 / U;         // 16-byte groups per 8-element fragment
    static constexpr size_t KV_BYTES = (size_t)C * D * sizeof(T);
    static constexpr size_t ST_BYTES = (size_t)CT * D * D * sizeof(T) + (size_t)CT * D * 4;
    // Double-buffer the K/V tiles when two workgroups still fit on a CU (or
    // when even one buffer would not leave room for two).
    static constexpr size_t LDS_CU = 160 * 1024;
    static constexpr bool FITS = 2 * KV_BYTES + ST_BYTES <= LDS_CU;
    static constexpr bool DB = 4 * KV_BYTES + ST_BYTES <= LDS_CU / 2 ||
                               (2 * KV_BYTES + ST_BYTES > LDS_CU / 2 && 4 * KV_BYTES + ST_BYTES <= LDS_CU);
    // State tile i of wave w is st = w * MAXST + i (d = 128: row block w);
    // only tile 0 of a wave can sit in column block 0 and own z.
    __device__ static int tile_of(int w, int i) { return w * MAXST + i; }
};

// Loads the 16-byte groups of one chunk of a [N][D] sequence (zeros past N).
template <typename T, int D, int C, int L>
__device__ __forceinline__ void load_chunk(typename Vt<T>::g16 (&r)[L], const T *base, int t0, int N, int tid)
{
    using G = Geo<T, D, C>;
    static_assert(L == G::LDV, "register array size");
    using g16 = typename Vt<T>::g16;
    if (t0 + C <= N && G::NGRP % kThreads == 0) {
#pragma unroll
        for (int l = 0; l < G::LDV; ++l) {
            const int e = tid + l * kThreads;
            r[l] = *reinterpret_cast<const g16 *>(base + (size_t)(t0 + e / G::GPR) * D + (e % G::GPR) * G::U);
        }
    } else {
#pragma unroll
        for (int l = 0; l < G::LDV; ++l) {
            const int e = tid + l * kThreads;
            const int t = e / G::GPR, q = e % G::GPR;
            g16 x = {};
            if (e < G::NGRP && t0 + t < N) x = *reinterpret_cast<const g16 *>(base + (size_t)(t0 + t) * D + q * G::U);
            r[l] = x;
        }
    }
}

// Writes a staged chunk to LDS: phi(K) and V, both row-major.  Only the
// first `rows` tokens are real; the others get phi(k) = 0 (their v is zero
// too) so that they add nothing to any sum.
template <typename T, int D, int C, int TH, typename IO, int L>
__device__ __forceinline__ void stage_rows(const typename Vt<T>::g16 (&kr)[L], const typename Vt<T>::g16 (&vr)[L],
                                           Tile<T, D> sK, Tile<T, D> sV, int rows, int tid)
{
    constexpr int U = Vt<T>::U, GPR = D / U, NGRP = C * GPR;
    static_assert(L == (NGRP + TH - 1) / TH, "register array size");
    const bool full = rows >= C;
#pragma unroll
    for (int l = 0; l < L; ++l) {
        const int e = tid + l * TH;
        if (NGRP % TH == 0 || e < NGRP) {
            const int t = e / GPR, q = e % GPR;
            typename Vt<T>::g16 fk;
#pragma unroll
            for (int i = 0; i < U; ++i) fk[i] = (T)IO::phi::f(Io<T, IO>::fi(kr[l], i));
            if (!full) {
                if (t >= rows) fk = typename Vt<T>::g16{};
            }
            sK.write16(t, q * U, fk);
            sV.write16(t, q * U, op16<T, IO>(vr[l]));
        }
    }
}

// A K-block operand whose every slot is 1 (for column sums on MFMA).
template <typename T> __device__ __forceinline__ typename Vt<T>::v8 ones8()
{
    typename Vt<T>::v8 o;
#pragma unroll
    for (int s = 0; s < 8; ++s) o[s] = (T)1.f;
    return o;
}

// ----------------------------------------------------------- decayed sums
//
// Decayed running sums (a reading of the Stream efficiency essay, section
// 4.2, whose scan is h_t = h_{t-1} a_t + b_t): with the log-decay g_t of
// every (sequence, kv head, token), S_t = exp(g_t) S_{t-1} + phi(k_t) v_t^T
// and z_t likewise.  Within a chunk every factor is taken from sums of g over
// one 32-token tile, so each exponent is a short sum and never positive for
// g <= 0:
//   L[t]  sum of g over the tile's tokens up to and including t;
//   TL[j] L at the last token of tile j (the tile's log-decay);
//   W[t]  exp(TL[tile(t)] - L[t]): the weight of key t in the sums at the
//         end of its tile.
// Then the state after tile j is exp(TL[j]) (state before it) + sum_t W[t]
// phi(k_t) v_t^T, key s reaches query t of the same tile with
// exp(L[t] - L[s]) (s <= t), and the state before a query's tile reaches it
// with exp(L[t]).
// A factor is exp of a difference of two such sums, so its relative error is
// about (|L[t]| + |L[s]|) 2^-24: log-decays below kMinLogDecay (a factor
// under 2.1e-9, which fp32 running sums cannot tell from zero) are taken as
// kMinLogDecay, keeping |L| <= 640 and every factor within ~4e-5.  NaN stays
// NaN.
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kMinLogDecay = -20.f;
__device__ __forceinline__ float clamp_log_decay(float g) { return g < kMinLogDecay ? kMinLogDecay : g; }

template <int C> struct DecayTab {
    float L[C];
    float W[C];
    float TL[C / 32];
};

// Fills the table from the log-decay gv of token tid (threads tid < C hold
// one token each; tokens past the sequence or segment carry g = 0).
template <int C>
__device__ __forceinline__ void decay_stage(DecayTab<C> &dt, float gv, int tid)
{
    if (tid < C) {
        float x = clamp_log_decay(gv);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) {
            const float y = __shfl_up(x, o, 32);
            if ((tid & 31) >= o) x += y;
        }
        const float tl = __shfl(x, 31, 32);
        dt.L[tid] = x;
        dt.W[tid] = __builtin_amdgcn_exp2f((tl - x) * kLog2e);
        if ((tid & 31) == 31) dt.TL[tid >> 5] = x;
    }
}

// Multiplies the 8 slots of a key fragment (tokens r0 .. r0 + 7) by their
// weights W[r0 .. r0 + 7].
template <typename T>
__device__ __forceinline__ typename Vt<T>::v8 weigh8(const typename Vt<T>::v8 &a, const float *w)
{
    const f32x4 w0 = *reinterpret_cast<const f32x4 *>(w);
    const f32x4 w1 = *reinterpret_cast<const f32x4 *>(w + 4);
    float x[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        x[s] = (float)a[s] * w0[s];
        x[4 + s] = (float)a[4 + s] * w1[s];
    }
    return cvt8<T>(x);
}

// State tile (it, jt) += phi(K)^T V over the 32 tokens of key tile kt.
// The K-block of 16 tokens kb2 puts token kt*32 + 16 kb2 + 8h + s in slot s.
// When want_z it also returns the tile's column sum of phi(K) for feature
// it*32 + lane%32: bf16 forms it on the matrix core (1 phi(K) into a scratch
// accumulator whose every register then holds the sum), fp32 adds on the
// vector ALUs and returns this half-wave's part (the caller adds the other).
// With a weight table W (decayed sums) every key is first multiplied by its
// weight W[token].
template <typename T, int D>
__device__ __forceinline__ float tile_state_update(f32x16 &acc, bool want_z, int it, int jt, int kt, Tile<T, D> sK,
                                                   Tile<T, D> sV, int lane, const float *W = nullptr)
{
    const int h = lane >> 5;
    float zs = 0.f;
    f32x16 Z = f32x16{};
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
        const int r0 = kt * 32 + 16 * kb2 + 8 * h;
        auto a = colfrag(sK, r0, r0 + 4, it * 32, lane);
        if (W) a = weigh8<T>(a, W + r0);
        const auto b = colfrag(sV, r0, r0 + 4, jt * 32, lane);
        mma(acc, a, b);
        if (want_z) {
            if constexpr (sizeof(T) == 2) {
                mma(Z, ones8<T>(), a);
            } else {
#pragma unroll
                for (int s = 0; s < 8; ++s) zs += a[s];
            }
        }
    }
    if constexpr (sizeof(T) == 2) zs = Z[0];
    return zs;
}

// -------------------------------------------------------------- seg_totals
//
// ---------------------------------------------------------- packed batches
//
// A packed batch holds nb sequences of different lengths with no padding
// (README "Features": variable sequence length): sequence b owns tokens
// [cu[b], cu[b+1]) of `total`, stored head-major per sequence (q and out:
// [H][n_b][d] from element H * cu[b] * d; k and v: [Hkv][n_b][d] from
// Hkv * cu[b] * d).  Sequences are cut into segments of seg_len tokens as in
// a dense batch; k_pack_plan writes the tables the kernels locate their
// segment with, into the workspace (ints):
//   segpre[nb + 1]  segments of the sequences before b
//   off[nb], len[nb]  token offset and length of sequence b
//   segb[nsmax]     the sequence of every segment
// The boundaries are clamped to [0, total] and made non-decreasing first, so
// malformed offsets give wrong rows but never an access out of range; every
// sequence has at least one segment (an empty one still writes its state).
struct Packed {
    const int *tab;  // the tables above; nullptr for a dense batch
    int nb, nsmax;   // sequences; segments the launches are sized for
};
struct SegLoc {
    int b, p, n, np, sb, off;  // sequence, segment in it, its tokens, its segments, segments before it, token offset
};
__device__ __forceinline__ bool packed_locate(const Packed &pk, int s, SegLoc &r)
{
    const int *segpre = pk.tab, *off = pk.tab + pk.nb + 1, *len = off + pk.nb, *segb = len + pk.nb;
    if (s >= min(segpre[pk.nb], pk.nsmax)) return false;
    const int b = segb[s];
    r.b = b;
    r.sb = segpre[b];
    r.np = segpre[b + 1] - r.sb;
    r.p = s - r.sb;
    r.off = off[b];
    r.n = len[b];
    return true;
}
// First workspace slot of (sequence b, kv head g): every sequence keeps
// np - 1 partial sums per kv head (causal) or np (non-causal), sequence-major
// as in a dense batch.
__device__ __forceinline__ size_t packed_slot0(const SegLoc &r, int g, int Hkv, int causal)
{
    return (size_t)(r.sb - causal * r.b) * Hkv + (size_t)g * (r.np - causal);
}

// One workgroup: builds the tables of a packed batch from cu[0..nb].
// Exclusive scan of x over the workgroup's threads in thread order, starting
// from init: thread t gets op(init, x_0, ..., x_{t-1}).  Shuffles within each
// wave, then the wave totals through LDS (sw: one int per wave).
template <class Op>
__device__ __forceinline__ int block_exclusive_scan(int x, int init, int *sw, Op op)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl = op(incl, y);
    }
    if (lane == 63) sw[w] = incl;
    __syncthreads();
    int pre = init;
    for (int i = 0; i < w; ++i) pre = op(pre, sw[i]);
    const int prev = __shfl_up(incl, 1);
    __syncthreads();  // sw may be reused by the caller
    return lane == 0 ? pre : op(pre, prev);
}

__global__ __launch_bounds__(kThreads) void k_pack_plan(const int *__restrict__ cu, int nb, int total, int seg_len,
                                                        int nsmax, int *__restrict__ tab)
{
    __shared__ int sw[kThreads / 64];
    int *segpre = tab, *off = tab + nb + 1, *len = off + nb, *segb = len + nb;
    const int tid = threadIdx.x;
    const int per = (nb + kThreads - 1) / kThreads;
    const int b0 = min(nb, tid * per), b1 = min(nb, b0 + per);
    auto clampt = [&](int x) { return x < 0 ? 0 : (x > total ? total : x); };
    // boundary j is the running maximum of cu[0..j], clamped to [0, total]
    int m = -2147483647 - 1;
    for (int j = b0 + 1; j <= b1; ++j) m = max(m, cu[j]);
    auto imax = [](int a, int b) { return a > b ? a : b; };
    auto iadd = [](int a, int b) { return a + b; };
    // maximum of cu[0 .. b0] for this thread's first sequence
    int run = block_exclusive_scan(m, cu[0], sw, imax), nseg = 0;
    for (int b = b0; b < b1; ++b) {
        const int lo = clampt(run);
        run = max(run, cu[b + 1]);
        const int hi = clampt(run);
        off[b] = lo;
        len[b] = hi - lo;
        nseg += hi > lo ? (hi - lo + seg_len - 1) / seg_len : 1;
    }
    int sbase = block_exclusive_scan(nseg, 0, sw, iadd);  // segments of the sequences before b0
    if (tid == kThreads - 1) segpre[nb] = sbase + nseg;
    for (int b = b0; b < b1; ++b) {
        segpre[b] = sbase;
        const int np = len[b] > 0 ? (len[b] + seg_len - 1) / seg_len : 1;
        for (int s = sbase; s < sbase + np && s < nsmax; ++s) segb[s] = b;
        sbase += np;
    }
}

// One workgroup per (sequence, segment): T_p = phi(K_p)^T V_p and
// sum phi(K_p), written as fp32 partials ws[seq][p] = [S (d x d) | z (d)].
// Chunks of C1 tokens, double-buffered in LDS (one barrier per chunk).
// Packed batches (pk.tab set): one workgroup per (kv head, segment of all
// sequences); the last segment of a causal sequence has nothing to do.
// DK (decayed sums, dense causal batches): gd [seq][N] is the log-decay; the
// total is the decayed sum at the segment's end, and the segment's summed g
// goes to gs[slot] for the scan.
template <typename T, int D, int C1, typename IO, bool DK = false>
__global__ __launch_bounds__(2 * kThreads) __attribute__((amdgpu_waves_per_eu(D <= 64 ? 4 : 2))) void k_seg_totals(const typename IO::elem *__restrict__ k,
                                                             const typename IO::elem *__restrict__ v,
                                                             float *__restrict__ ws, int N, int seg_len, int nslots,
                                                             Packed pk, int Hkv, int causal,
                                                             const float *__restrict__ gd = nullptr,
                                                             float *__restrict__ gs = nullptr)
{
    using G = Geo<T, D, C1>;
    __shared__ __attribute__((aligned(16))) T smK[2][C1 * D];
    __shared__ __attribute__((aligned(16))) T smV[2][C1 * D];
    __shared__ __attribute__((aligned(16))) DecayTab<C1> smD[DK ? 2 : 1];

    using In = typename IO::elem;
    int seq = blockIdx.x / nslots, p = blockIdx.x % nslots;
    const In *kb = k + (size_t)seq * N * D;
    const In *vb = v + (size_t)seq * N * D;
    size_t slot = (size_t)seq * nslots + p;
    if (pk.tab) {
        SegLoc r;
        const int gk = blockIdx.x / pk.nsmax;
        if (!packed_locate(pk, blockIdx.x % pk.nsmax, r) || (causal && r.p == r.np - 1)) return;
        p = r.p;
        N = r.n;
        kb = k + ((size_t)r.off * Hkv + (size_t)gk * r.n) * D;
        vb = v + ((size_t)r.off * Hkv + (size_t)gk * r.n) * D;
        slot = packed_slot0(r, gk, Hkv, causal) + r.p;
    }
    // Waves 0-3 absorb (they own the state tiles), waves 4-7 stage: while the
    // first four add chunk c from one LDS buffer, the other four write phi(K),
    // V of chunk c + 1 into the other buffer and request chunk c + 3, so the
    // vector work of staging runs beside the matrix work instead of before it.
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, h = lane >> 5, n = lane & 31;
    const bool stager = w >= 4;
    const int sid = tid - kThreads;  // staging thread 0..255
    const int s0 = p * seg_len, s1 = min(N, s0 + seg_len);
    const int nch = (s1 - s0 + C1 - 1) / C1;

    f32x16 acc[G::MAXST];
    float zacc = 0.f;
#pragma unroll
    for (int i = 0; i < G::MAXST; ++i) acc[i] = f32x16{};
    // The staging waves keep NS chunks in flight in register sets (two for
    // 16-bit rows at d = 128, where one workgroup fills a CU anyway; one
    // otherwise, so that two workgroups fit on a CU).  Buffer loads:
    // chunks past the segment read nothing, tokens past N read zeros.
    constexpr int NS = D >= 128 && sizeof(T) == 2 ? 2 : 1;
    using g16 = typename Vt<T>::g16;
    constexpr int E = Io<T, IO>::EB, GB = Io<T, IO>::GB;  // input element and raw group bytes
    g16 kR[NS][G::LDV], vR[NS][G::LDV];
    float gR[NS];
    auto rows_at = [&](int t0) { return t0 < s1 ? min(C1, s1 - t0) : 0; };
    // First token of the i-th chunk taken (i >= nch: past the segment, no
    // rows).  Plain sums take the segment's chunks last to first: the pass
    // that follows starts at the segment's first tokens, which are then the
    // ones most recently read, still in the memory-side cache when K and V
    // do not fit it whole.  Decayed sums need the forward order.
    auto tpos = [&](int i) {
        const int kx = DK ? i : nch - 1 - i;
        return i < nch && kx >= 0 ? s0 + kx * C1 : s1;
    };
    // log-decay of token t0 + sid (zero past the segment)
    const float *gb = DK ? gd + (size_t)seq * N : nullptr;
    float glog = 0.f;
    // chunk i into register set u
    auto load = [&](int u, int i) {
        const int t0 = tpos(i), rows = rows_at(t0);
        const Rsrc rk = make_rsrc(kb + (size_t)t0 * D, rows * D * E);
        const Rsrc rv = make_rsrc(vb + (size_t)t0 * D, rows * D * E);
#pragma unroll
        for (int l = 0; l < G::LDV; ++l) {
            const unsigned off = (unsigned)(sid + l * kThreads) * GB;
            kR[u][l] = load_in<T, IO>(rk, off);
            vR[u][l] = load_in<T, IO>(rv, off);
        }
        if constexpr (DK) gR[u] = sid < rows ? gb[t0 + sid] : 0.f;
    };
    // chunk i from register set u into LDS buffer buf
    auto stage = [&](int u, int buf, int i) {
        stage_rows<T, D, C1, kThreads, IO>(kR[u], vR[u], Tile<T, D>{smK[buf]}, Tile<T, D>{smV[buf]},
                                           rows_at(tpos(i)), sid);
        if constexpr (DK) decay_stage<C1>(smD[buf], gR[u], sid);
    };
    auto absorb = [&](int buf) {
        const Tile<T, D> sK{smK[buf]}, sV{smV[buf]};
#pragma unroll
        for (int i = 0; i < G::MAXST; ++i) {
            const int st = G::tile_of(w, i);
            if (st < G::NST) {
                const int it = st / G::DT, jt = st % G::DT;
#pragma unroll
                for (int kt = 0; kt < G::CT; ++kt) {
                    if constexpr (DK) {
                        // the sums so far fade over the tile, then its keys are added with their weights
                        const float a = __builtin_amdgcn_exp2f(smD[buf].TL[kt] * kLog2e);
                        acc[i] *= a;
                        if (i == 0 && jt == 0) zacc *= a;
                        zacc += tile_state_update<T, D>(acc[i], i == 0 && jt == 0, it, jt, kt, sK, sV, lane,
                                                        smD[buf].W);
                    } else {
                        zacc += tile_state_update<T, D>(acc[i], i == 0 && jt == 0, it, jt, kt, sK, sV, lane);
                    }
                }
            }
        }
        if constexpr (DK) {
#pragma unroll
            for (int kt = 0; kt < G::CT; ++kt) glog += smD[buf].TL[kt];
        }
    };
    if (stager) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            load(u, u);
            __builtin_amdgcn_sched_barrier(0);  // keep each chunk's loads ahead of the next one's
        }
        stage(0, 0, 0);
        load(0, NS);
    }
    lds_barrier();
    // Step ci: the absorbing waves add chunk ci (buffer ci & 1) while the
    // staging waves write chunk ci + 1 (register set (ci + 1) % NS) into the
    // other buffer and request chunk ci + 1 + NS into that set; one barrier
    // per step.  Steps in pairs, so that every step's register set is fixed.
    for (int ci = 0; ci < nch; ci += 2) {
        if (stager) {
            if (ci + 1 < nch) {
                stage(1 % NS, 1, ci + 1);
                load(1 % NS, ci + 1 + NS);
            }
        } else {
            absorb(0);
        }
        lds_barrier();
        if (ci + 1 < nch) {
            if (stager) {
                if (ci + 2 < nch) {
                    stage(0, 0, ci + 2);
                    load(0, ci + 2 + NS);
                }
            } else {
                absorb(1);
            }
            lds_barrier();
        }
    }
    if (stager) return;
    if constexpr (DK) {
        if (tid == 0) gs[slot] = glog;
    }
    float *out = ws + slot * (size_t)D * (D + 1);
#pragma unroll
    for (int i = 0; i < G::MAXST; ++i) {
        const int st = G::tile_of(w, i);
        if (st < G::NST) {
            const int it = st / G::DT, jt = st % G::DT;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = it * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                out[(size_t)row * D + jt * 32 + n] = acc[i][r];
            }
            if (i == 0 && jt == 0) {
                const float z = sizeof(T) == 2 ? zacc : zacc + __shfl_xor(zacc, 32);
                if (h == 0) out[(size_t)D * D + it * 32 + n] = z;
            }
        }
    }
}

// ------------------------------------------------------ fp32 totals pass
//
// For fp32 rows the 16x16x4 fp32 matrix instruction takes, per lane (j, kq)
// (j = lane % 16, kq = lane / 16), A[j][kq] and B[kq][j]: four tokens per
// instruction, one per quarter-wave.  Lane (j, kq) loads 16 bytes (4
// features; 8 bytes, 2 features, at d = 32) of token 4g + kq of K and of V
// straight from global memory, so one load instruction brings four whole
// rows (d = 64) with no LDS staging.  Instruction (e, e') takes feature
// VEC i + e of phi(K) as A and feature VEC j + e' of V as B: together the
// VEC^2 instructions add the four tokens' phi(k) v^T to a state whose row
// VEC i + e, column VEC j + e' sits in register r of lane (j, kq) of
// accumulator (e, e') with i = 4 kq + r.  d <= 64: each of the four waves
// keeps the whole state over every fourth group of tokens and the waves are
// summed through LDS at the end; d = 128: each wave keeps one quadrant (the
// 64-feature halves of K and V it reads) over every token.  Per-lane word
// loads in the 32x32x2 layout measured slower than LDS staging (a load
// instruction then carries 256 bytes, and the address unit, not memory,
// set the pace); these carry 1 KiB.  Same workgroups, slots and outputs as
// k_seg_totals (plain sums only); token groups last to first as there.
template <int D> struct X4 {
    static constexpr int NW = 4, TH = 64 * NW;
    static constexpr int VEC = D == 32 ? 2 : 4;  // features per lane and load
    static constexpr bool QUAD = D == 128;       // waves own quadrants of the state
    static constexpr int TS = QUAD ? 1 : NW;     // waves splitting the token groups
    static constexpr int PD = 4;                 // token groups in flight per wave
    static constexpr int NR = TS > 1 ? NW * VEC * VEC * 64 : 1;  // LDS f32x4 for the wave sums
};

template <int D, typename IO>
__global__ __launch_bounds__(X4<D>::TH) void k_seg_totals_f32(const float *__restrict__ k,
                                                              const float *__restrict__ v,
                                                              float *__restrict__ ws, int N, int seg_len,
                                                              int nslots, Packed pk, int Hkv, int causal)
{
    using X = X4<D>;
    constexpr int VEC = X::VEC, TS = X::TS, PD = X::PD, NW = X::NW;
    using fv = std::conditional_t<VEC == 4, f32x4, float __attribute__((ext_vector_type(2)))>;
    __shared__ f32x4 red[X::NR];
    __shared__ f32x4 redz[TS > 1 ? NW * 64 : 1];

    int seq = blockIdx.x / nslots, p = blockIdx.x % nslots;
    const float *kb = k + (size_t)seq * N * D;
    const float *vb = v + (size_t)seq * N * D;
    size_t slot = (size_t)seq * nslots + p;
    if (pk.tab) {
        SegLoc r;
        const int gk = blockIdx.x / pk.nsmax;
        if (!packed_locate(pk, blockIdx.x % pk.nsmax, r) || (causal && r.p == r.np - 1)) return;
        p = r.p;
        N = r.n;
        kb = k + ((size_t)r.off * Hkv + (size_t)gk * r.n) * D;
        vb = v + ((size_t)r.off * Hkv + (size_t)gk * r.n) * D;
        slot = packed_slot0(r, gk, Hkv, causal) + r.p;
    }
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, j = lane & 15, kq = lane >> 4;
    const int tsi = TS > 1 ? w : 0;                         // token share
    const int cK = X::QUAD ? w >> 1 : 0, cV = X::QUAD ? w & 1 : 0;  // quadrant (d = 128)
    const int s0 = p * seg_len, len = max(0, min(N, s0 + seg_len) - s0);
    const int ng = (len + 3) / 4, nj = (ng + TS - 1) / TS;
    const Rsrc rk = make_rsrc(kb + (size_t)s0 * D, len * D * 4);
    const Rsrc rv = make_rsrc(vb + (size_t)s0 * D, len * D * 4);

    // Step i of this wave: token group g = ng - 1 - (i TS + tsi).  Tokens past
    // the segment's end read zeros; groups before it (g < 0) have negative
    // offsets, which as unsigned lie beyond every range: no branch, no read.
    auto row_of = [&](int i) { return 4 * (ng - 1 - (i * TS + tsi)) + kq; };
    auto ld = [&](Rsrc r, int t, int c) {
        const unsigned off = (unsigned)((t * D + 64 * c + VEC * j) * 4);
        if constexpr (VEC == 4) return buf_load16<f32x4>(r, off);
        else return __builtin_bit_cast(fv, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    };
    fv kr[PD], vr[PD];
    auto load = [&](int u, int i) {
        const int t = row_of(i);
        kr[u] = ld(rk, t, cK);
        vr[u] = ld(rv, t, cV);
    };
    f32x4 acc[VEC][VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e)
#pragma unroll
        for (int f = 0; f < VEC; ++f) acc[e][f] = f32x4{};
    f32x4 zs = {};
    auto absorb = [&](int u, int i) {
        // Tokens outside the segment read k = v = 0: their products with v
        // vanish, and only z needs them masked (phi(0) need not be 0).
        const bool live = (unsigned)row_of(i) < (unsigned)len;
        float a[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            a[e] = IO::phi::f(kr[u][e]);
            zs[e] += live ? a[e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e)
#pragma unroll
            for (int f = 0; f < VEC; ++f)
                acc[e][f] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], vr[u][f], acc[e][f], 0, 0, 0);
    };
#pragma unroll
    for (int u = 0; u < PD; ++u) load(u, u);
    for (int i0 = 0; i0 < nj; i0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) {
            if (i0 + u < nj) absorb(u, i0 + u);
            load(u, i0 + u + PD);
        }
    }
    // z: the four quarter-waves hold four token subsets of the same features
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        zs[e] += __shfl_xor(zs[e], 16);
        zs[e] += __shfl_xor(zs[e], 32);
    }
    float *out = ws + slot * (size_t)D * (D + 1);
    // acc[e][f][r] is state row VEC (4 kq + r) + e of the wave's rows, column VEC j + f of its columns
    auto store_row = [&](const f32x4 (&s)[VEC], int e, int r) {
        float *o = out + (size_t)(64 * cK + VEC * (4 * kq + r) + e) * D + 64 * cV + VEC * j;
        if constexpr (VEC == 4) *reinterpret_cast<f32x4 *>(o) = f32x4{s[0][r], s[1][r], s[2][r], s[3][r]};
        else *reinterpret_cast<fv *>(o) = fv{s[0][r], s[1][r]};
    };
    if constexpr (TS > 1) {
        // the waves' sums through LDS; wave w then adds up and stores rows e = w
#pragma unroll
        for (int e = 0; e < VEC; ++e)
#pragma unroll
            for (int f = 0; f < VEC; ++f) red[(w * VEC * VEC + e * VEC + f) * 64 + lane] = acc[e][f];
        redz[w * 64 + lane] = zs;
        __syncthreads();
        if (w < VEC) {
            const int e = w;
            f32x4 s[VEC];
#pragma unroll
            for (int f = 0; f < VEC; ++f) {
                s[f] = red[(e * VEC + f) * 64 + lane];
#pragma unroll
                for (int o = 1; o < NW; ++o) s[f] += red[(o * VEC * VEC + e * VEC + f) * 64 + lane];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) store_row(s, e, r);
        }
        if (w == NW - 1 && kq == 0) {
            f32x4 z = redz[lane];
#pragma unroll
            for (int o = 1; o < NW; ++o) z += redz[o * 64 + lane];
            float *oz = out + (size_t)D * D + VEC * j;
            if constexpr (VEC == 4) *reinterpret_cast<f32x4 *>(oz) = z;
            else *reinterpret_cast<fv *>(oz) = fv{z[0], z[1]};
        }
    } else {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
#pragma unroll
            for (int r = 0; r < 4; ++r) store_row(acc[e], e, r);
        if (cV == 0 && kq == 0) *reinterpret_cast<f32x4 *>(out + (size_t)D * D + 64 * cK + VEC * j) = zs;
    }
}

// ---------------------------------------------------------------- seg_scan
//
// ws holds nslots partials of E = D*D + D floats per sequence.  mode 0:
// inclusive prefix along the slots, in place.  mode 1: the sum, written to
// slot 0 and, when given, to state_out / z_out.  mode 2: inclusive suffix
// (slot p gets the sum of slots p..nslots-1), in place.  Modes 0 and 1 start
// from s_in / z_in (the sums of earlier tokens) when given.
// Packed batches: blockIdx.y = b * Hkv + kv head, and sequence b's own slots.
// Decayed sums (gs set, mode 0 only): slot p also has its segment's summed
// log-decay gs[seq * nslots + p], and the prefix becomes the decayed one,
// acc = exp(gs[p]) acc + slot p.
__global__ __launch_bounds__(kThreads) void k_seg_scan(float *__restrict__ ws, int nslots, int D, int mode,
                                                       float *__restrict__ state_out, float *__restrict__ z_out,
                                                       const float *__restrict__ s_in, const float *__restrict__ z_in,
                                                       Packed pk = Packed{nullptr, 0, 0}, int Hkv = 1,
                                                       const float *__restrict__ gs = nullptr)
{
    // Four consecutive elements per thread (E is a multiple of 4), every
    // access a 16-byte buffer access: slots past the sequence's last read
    // zeros and take no stores, so no load or store sits behind a branch and
    // a whole batch of slots is in flight at once.
    const int E = D * D + D;
    const int seq = blockIdx.y;
    const int e = 4 * (int)(blockIdx.x * kThreads + threadIdx.x);
    if (e >= E) return;
    size_t base = (size_t)seq * nslots * E;
    if (pk.tab) {
        const int b = seq / Hkv, gk = seq % Hkv, causal = mode != 1;
        SegLoc r;
        r.b = b;
        r.sb = pk.tab[b];
        r.np = pk.tab[b + 1] - r.sb;
        nslots = r.np - causal;
        base = packed_slot0(r, gk, Hkv, causal) * E;
    }
    // the sums start from the given ones (continuation), else from zero
    f32x4 acc = f32x4{};
    if (e < D * D) {
        if (s_in) acc = *reinterpret_cast<const f32x4 *>(s_in + (size_t)seq * D * D + e);
    } else if (z_in) {
        acc = *reinterpret_cast<const f32x4 *>(z_in + (size_t)seq * D + (e - D * D));
    }
    const Rsrc rw = make_rsrc(ws + base, nslots > 0 ? nslots * E * 4 : 0);
    // byte offset of the slot visited at step i: forwards for modes 0 and 1,
    // backwards for mode 2 (steps past the last slot land out of range)
    auto off = [&](int i) {
        const int sl = mode == 2 ? nslots - 1 - i : i;
        return sl >= 0 && sl < nslots ? (unsigned)(sl * E + e) * 4u : kOutOfRange;
    };
    constexpr int BATCH = 32;
    for (int p0 = 0; p0 < nslots; p0 += BATCH) {
        f32x4 x[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) x[j] = buf_load16<f32x4>(rw, off(p0 + j));
        if (gs) {
            const float *gq = gs + (size_t)seq * nslots;
#pragma unroll
            for (int j = 0; j < BATCH; ++j) {
                if (p0 + j < nslots) {
                    acc = __builtin_amdgcn_exp2f(gq[p0 + j] * kLog2e) * acc + x[j];
                    buf_store16<f32x4>(rw, off(p0 + j), acc);
                }
            }
            continue;
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
            acc += x[j];
            if (mode != 1) buf_store16<f32x4>(rw, off(p0 + j), acc);
        }
    }
    if (mode == 1) {
        buf_store16<f32x4>(rw, off(0), acc);
        if (e < D * D) {
            if (state_out) *reinterpret_cast<f32x4 *>(state_out + (size_t)seq * D * D + e) = acc;
        } else if (z_out) {
            *reinterpret_cast<f32x4 *>(z_out + (size_t)seq * D + (e - D * D)) = acc;
        }
    }
}

// Grid of k_seg_scan for head dimension d over nseq sequences.
inline dim3 scan_grid(int d, int nseq)
{
    const int e4 = (d * d + d) / 4;
    return dim3((e4 + kThreads - 1) / kThreads, nseq);
}

// ------------------------------------------------------ format dispatch
//
// The `dtype` argument of the C ABI: element type in bits 0-7, feature map
// in bits 8-15.  with_format calls fn(Kind<T, Fmt<elem, phi>>{}) for the
// operand type T the element type computes in (float for fp32, bf16 for
// both 16-bit formats).
template <typename T_, typename IO_> struct Kind {
    using T = T_;
    using IO = IO_;
};
inline bool valid_dtype(int dtype)
{
    const int e = dtype & 0xff, m = dtype >> 8;
    return dtype >= 0 &&
           (e == LINATTN_F32 || e == LINATTN_BF16 || e == LINATTN_F16 || e == LINATTN_FP8_E4M3 ||
            e == LINATTN_FP8_E5M2) &&
           (m == LINATTN_PHI_ELU1 || m == LINATTN_PHI_RELU || m == LINATTN_PHI_SOFTPLUS);
}
template <class P, class Fn> int with_elem(int e, Fn &fn)
{
    switch (e) {
    case LINATTN_F32: return fn(Kind<float, Fmt<float, P>>{});
    case LINATTN_BF16: return fn(Kind<bf16, Fmt<bf16, P>>{});
    case LINATTN_F16: return fn(Kind<bf16, Fmt<f16, P>>{});
    }
    return LINATTN_ERR_DTYPE;
}
template <class Fn> int with_format(int dtype, Fn fn)
{
    if (!valid_dtype(dtype)) return LINATTN_ERR_DTYPE;
    switch (dtype >> 8) {
    case LINATTN_PHI_ELU1: return with_elem<PhiElu1>(dtype & 0xff, fn);
    case LINATTN_PHI_RELU: return with_elem<PhiRelu>(dtype & 0xff, fn);
    case LINATTN_PHI_SOFTPLUS: return with_elem<PhiSoftplus>(dtype & 0xff, fn);
    }
    return LINATTN_ERR_DTYPE;
}

// -------------------------------------------------------------- launchers

int launch_status()
{
    return hipGetLastError() == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest chunk of the staged totals pass: at most 16 KiB of K per chunk, so
// that two chunks of K and V double-buffer in 64 KiB of LDS, and for 16-bit
// rows at most 64 tokens, whose staging registers leave room for two
// workgroups per CU at d <= 64 (128-token chunks spill there).
template <typename T, int D> constexpr int totals_cap()
{
    constexpr int bytes = 65536 / (4 * D * (int)sizeof(T));
    constexpr int lim = sizeof(T) == 2 ? 64 : 128;
    return bytes < lim ? bytes : lim;
}

// Totals pass with chunks of c1 tokens (32, 64 or 128, at most totals_cap);
// plain fp32 sums take the pass without staging (k_seg_totals_f32), whatever c1.
template <typename T, int D, typename IO = Fmt<T, PhiElu1>, bool DK = false>
int launch_totals(int c1, unsigned nblocks, hipStream_t st, const typename IO::elem *k, const typename IO::elem *v,
                  float *ws, int N, int seg_len,
                  int nslots, Packed pk = Packed{nullptr, 0, 0}, int Hkv = 1, int causal = 1,
                  const float *gd = nullptr, float *gs = nullptr)
{
    if constexpr (std::is_same_v<T, float> && !DK) {
        hipLaunchKernelGGL((k_seg_totals_f32<D, IO>), dim3(nblocks), dim3(X4<D>::TH), 0, st, k, v, ws, N, seg_len,
                           nslots, pk, Hkv, causal);
        return LINATTN_OK;
    }
    constexpr int cap = totals_cap<T, D>();
    switch (c1) {
    case 32:
        hipLaunchKernelGGL((k_seg_totals<T, D, 32, IO, DK>), dim3(nblocks), dim3(2 * kThreads), 0, st, k, v, ws, N, seg_len,
                           nslots, pk, Hkv, causal, gd, gs);
        return LINATTN_OK;
    case 64:
        if constexpr (64 <= cap) {
            hipLaunchKernelGGL((k_seg_totals<T, D, 64, IO, DK>), dim3(nblocks), dim3(2 * kThreads), 0, st, k, v, ws, N,
                               seg_len, nslots, pk, Hkv, causal, gd, gs);
            return LINATTN_OK;
        }
        break;
    case 128:
        if constexpr (128 <= cap) {
            hipLaunchKernelGGL((k_seg_totals<T, D, 128, IO, DK>), dim3(nblocks), dim3(2 * kThreads), 0, st, k, v, ws, N,
                               seg_len, nslots, pk, Hkv, causal, gd, gs);
            return LINATTN_OK;
        }
        break;
    }
    return LINATTN_ERR_UNSUPPORTED;
}

template <typename T, int D>
int totals_chunk(int seg_len)
{
    int c1 = totals_cap<T, D>();
    while (c1 > 32 && seg_len % c1 != 0) c1 /= 2;  // segments are whole chunks of the pass
    return c1;
}

}  // namespace
