// linattn_plan.cpp - argument validation and launch planning (host only).
#include "linattn_plan.h"

#include <stdint.h>

#include "linattn.h"

namespace linattn {

namespace {
constexpr int kCUs = 256;
constexpr int kTargetWorkgroups = 2 * kCUs;  // non-causal partial sums: two workgroups per CU

bool valid_d(int d) { return d == 32 || d == 64 || d == 128; }
bool valid_chunk(int c) { return c == 32 || c == 64 || c == 128 || c == 256; }
}  // namespace

int heads_per_block(int dtype, int d, int chunk, int G)
{
    const int e = (dtype & 0xff) != LINATTN_F32 ? 2 : 4;
    for (int gt = 8; gt >= 1; gt /= 2)
        if (G % gt == 0 && main_shape(e, d, chunk, gt).fits) return gt;
    return 0;
}

int auto_chunk(int dtype, int d, int G, int causal)
{
    (void)causal;
    // Prefer the most query heads per workgroup (K and V are then read once
    // per head block), then about 128 query rows per chunk, which gives the
    // four waves one 32-row query tile each; fp32 prefers 64-token chunks,
    // whose tiles leave room for eight waves.
    const bool f32 = (dtype & 0xff) == LINATTN_F32;
    for (int gt = 8; gt >= 1; gt /= 2) {
        if (G % gt != 0) continue;
        const int rows = 128 / gt >= 32 ? 128 / gt : 32;  // about 128 query rows, at least one tile
        const int pref[4] = {f32 ? 64 : rows, f32 ? rows : 64, 32, 128};
        for (int i = 0; i < 4; ++i) {
            const int c = pref[i];
            if (heads_per_block(dtype, d, c, G) == gt) return c;
        }
    }
    return 0;
}

int decay_chunk(int dtype, int d, int H, int Hkv, int chunk)
{
    if (chunk != 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0) return chunk;
    // The decayed chunk kernel carries the tile decay sums and key weights
    // beside the plain kernel's registers: for 16-bit rows at d = 64 its
    // 128-token form spills, and the 64-token form measured faster.
    const int c = auto_chunk(dtype, d, H / Hkv, 1);
    return (dtype & 0xff) != LINATTN_F32 && d <= 64 && c > 64 ? 64 : c;
}

int make_plan(int B, int H, int Hkv, int N, int d, int causal, int dtype, int chunk, Plan *p)
{
    if (dtype < 0 || (dtype & 0xff) > LINATTN_FP8_E5M2 || (dtype >> 8) > LINATTN_PHI_SOFTPLUS) return LINATTN_ERR_DTYPE;
    if (B < 0 || H <= 0 || Hkv <= 0 || N < 0 || d <= 0 || H % Hkv != 0) return LINATTN_ERR_SHAPE;
    if ((int64_t)B * H > INT32_MAX / 2 || (int64_t)N * d > INT32_MAX / 2) return LINATTN_ERR_SHAPE;
    if (!valid_d(d)) return LINATTN_ERR_UNSUPPORTED;
    if (chunk != 0 && !valid_chunk(chunk)) return LINATTN_ERR_UNSUPPORTED;
    const int G = H / Hkv;
    const int C = chunk ? chunk : auto_chunk(dtype, d, G, causal);
    if (C == 0) return LINATTN_ERR_UNSUPPORTED;
    int gt = heads_per_block(dtype, d, C, G);
    if (gt == 0) return LINATTN_ERR_UNSUPPORTED;
    // The chunk kernel addresses a head block's q and out (gt * N * d
    // elements) with 32-bit byte offsets: fewer heads per block for very long
    // sequences, and an error when one head alone exceeds 2 GiB.
    const int64_t esz = (dtype & 0xff) != LINATTN_F32 ? 2 : 4;
    while (gt > 1 && (int64_t)gt * N * d * esz > INT32_MAX) gt /= 2;
    if ((int64_t)N * d * esz > INT32_MAX) return LINATTN_ERR_SHAPE;

    Plan q{};
    q.B = B; q.H = H; q.Hkv = Hkv; q.N = N; q.d = d; q.G = G;
    q.causal = causal ? 1 : 0;
    q.dtype = dtype;
    q.chunk = C;
    q.gt = gt;
    q.nseq = B * Hkv;
    q.segments = 0;
    q.seg_len = 0;
    q.ws_slots = 0;
    q.ws_bytes = 0;
    if (B > 0 && N > 0) {
        const int nchunks = (N + C - 1) / C;
        // Causal: one resident round of chunk-kernel workgroups (as many per
        // CU as its occupancy allows), so every workgroup walks several
        // chunks with the next one in flight instead of a second round
        // starting cold.
        const int e = (dtype & 0xff) != LINATTN_F32 ? 2 : 4;
        const int tgt = q.causal ? kCUs * main_shape(e, d, C, gt).occ : kTargetWorkgroups;
        int P = (tgt + q.nseq - 1) / q.nseq;
        if (P < 1) P = 1;
        if (P > nchunks) P = nchunks;
        const int seg_chunks = (nchunks + P - 1) / P;
        q.seg_len = seg_chunks * C;
        q.segments = (N + q.seg_len - 1) / q.seg_len;
        // Causal: the last segment's total is never needed by another segment.
        q.ws_slots = q.causal ? q.segments - 1 : q.segments;
        q.ws_bytes = (size_t)q.nseq * q.ws_slots * (size_t)d * (d + 1) * sizeof(float);
    }
    *p = q;
    return LINATTN_OK;
}

int make_plan_packed(int nb, int H, int Hkv, int total, int d, int causal, int dtype, int chunk, Plan *p)
{
    Plan q{};
    // Shapes, chunk and head block as for one sequence of `total` tokens.
    const int rc = make_plan(nb > 0 ? 1 : 0, H, Hkv, total, d, causal, dtype, chunk, &q);
    if (rc != LINATTN_OK) return rc;
    if (nb < 0) return LINATTN_ERR_SHAPE;
    q.B = nb;
    q.nb = nb;
    q.nseq = nb * Hkv;
    q.packed = 1;
    q.segments = q.seg_len = q.ws_slots = 0;
    q.ws_bytes = 0;
    q.tab_off = 0;
    if (nb > 0 && total > 0) {
        const int C = q.chunk;
        const int e = (dtype & 0xff) != LINATTN_F32 ? 2 : 4;
        const int hb = q.G / q.gt;
        // Workgroups as for a dense batch: one resident round of the chunk
        // kernel (causal) or 512 partial sums (non-causal), over all kv heads.
        const int tgt = q.causal ? kCUs * main_shape(e, d, C, q.gt).occ : kTargetWorkgroups;
        const int per = q.causal ? Hkv * hb : Hkv;
        const int nseg = (tgt + per - 1) / per;
        // The non-causal output pass takes 128-token blocks of a segment.
        const int unit = q.causal ? C : (C > 128 ? C : 128);
        int64_t len = ((int64_t)total + nseg - 1) / nseg;
        len = (len + unit - 1) / unit * unit;
        q.seg_len = (int)len;
        const int64_t nsmax = ((int64_t)total + len - 1) / len + nb;
        const int64_t slots = (int64_t)Hkv * nsmax;
        const int64_t tab_ints = 3 * (int64_t)nb + 1 + nsmax;
        if (nsmax > INT32_MAX / 2 || slots > INT32_MAX / 2) return LINATTN_ERR_SHAPE;
        q.segments = (int)nsmax;
        q.ws_slots = (int)nsmax;
        const size_t slot_bytes = (size_t)slots * (size_t)d * (d + 1) * sizeof(float);
        q.tab_off = (slot_bytes + 255) / 256 * 256;
        q.ws_bytes = q.tab_off + (size_t)tab_ints * sizeof(int);
    }
    *p = q;
    return LINATTN_OK;
}

bool decay_ok(const Plan &p)
{
    const int e = (p.dtype & 0xff) != LINATTN_F32 ? 2 : 4;
    const bool fp8 = (p.dtype & 0xff) == LINATTN_FP8_E4M3 || (p.dtype & 0xff) == LINATTN_FP8_E5M2;
    return p.causal && !p.packed && !fp8 && (p.dtype >> 8) == LINATTN_PHI_ELU1 &&
           !main_shape(e, p.d, p.chunk, p.gt).shift;
}

size_t decay_ws_bytes(const Plan &p)
{
    return p.ws_bytes + (size_t)p.nseq * p.ws_slots * sizeof(float);
}

}  // namespace linattn
