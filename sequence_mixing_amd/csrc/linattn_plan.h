// linattn_plan.h - argument validation and launch planning for liblinattn
// (host only, no HIP calls; unit-tested on machines without a GPU).
#pragma once
#include <stddef.h>

namespace linattn {

// Shape of one chunk-kernel instantiation: e = element bytes, D head
// dimension, C tokens per chunk, GT query heads per workgroup.  LDS holds
// phi(K), V and phi(Q) of a chunk ((2 + GT) C D elements) plus nsc copies of
// the transposed state (D x D) and of z (D); nsc is one copy per 32-token key
// tile, or one per two key tiles when that keeps two workgroups on a CU (or
// when one per tile does not fit; fp32 then drops only the first copy).
// Each thread stages lk + lk + lq 16-byte groups (raw K, V and q of the
// next chunk, 4 registers each).  A workgroup has 4 waves, or 8 when it is
// alone on its CU (two waves per SIMD then hide each other's waits) and the
// data are 16-bit or the fp32 tiles are small enough (d <= 64, d * C <= 4096)
// for two waves' registers.
struct MainShape {
    int nsc;      // state copies per chunk
    int occ;      // workgroups per CU the kernel is built for (1 or 2)
    int nw;       // waves per workgroup (4 or 8)
    int lk;       // 16-byte K (and V) groups each thread stages per chunk
    int lq;       // 16-byte q groups each thread stages per chunk
    bool shift;   // fp32 copies taken after key tiles 0 .. ct-2 instead of before 0 .. ct-1
    bool fits;    // buildable: LDS within 160 KiB, at most 8 q groups per thread of 4 waves
                  // (a register budget), at most 2 key tiles per copy
    unsigned long lds;
    bool pipe;    // fp32, 8 waves: state tiles and phase-2 items on waves 0-3, which only compute;
                  // waves 4-7 stage the next chunk meanwhile (K, V and q double-buffered)
};

constexpr unsigned long main_lds(int e, int D, int C, int GT, int nsc)
{
    return (unsigned long)e * ((unsigned long)(2 + GT) * C * D + (unsigned long)nsc * D * D + (unsigned long)nsc * D);
}

constexpr MainShape main_shape(int e, int D, int C, int GT)
{
    const unsigned long half = 80 * 1024, full = 160 * 1024;
    if (C < 32 || D < 32) return MainShape{1, 1, 4, 1, 1, false, false, 0, false};  // not a kernel shape
    const int ct = C / 32;
    const int u = 16 / e;
    const int lk4 = (C * (D / u) + 255) / 256;
    const int lq4 = (GT * C * (D / u) + 255) / 256;
    const int stage_regs = 4 * (2 * lk4 + lq4);
    // Two workgroups per CU leave 256 registers per lane: enough for the
    // 16-bit kernels up to d = 64 with at most 48 staging registers.
    const int occ_reg = (D * e <= 128 && stage_regs <= 48) ? 2 : 1;
    int nsc = ct;
    bool shift = false;
    if (occ_reg == 2 && main_lds(e, D, C, GT, ct) <= half) nsc = ct;
    else if (occ_reg == 2 && ct >= 2 && main_lds(e, D, C, GT, ct / 2) <= half) nsc = ct / 2;
    else if (main_lds(e, D, C, GT, ct) <= full) nsc = ct;
    else if (e == 4 && ct > 2 && main_lds(e, D, C, GT, ct - 1) <= full) {
        // fp32: the copy before key tile 0 is dropped; query tile 0 reads the
        // copy after tile 0 and subtracts its keys later than the query
        // (exact enough in fp32), so no tile needs an unmasked neighbour.
        nsc = ct - 1;
        shift = true;
    } else nsc = ct >= 2 ? ct / 2 : 1;
    const unsigned long lds = main_lds(e, D, C, GT, nsc);
    const int occ = (occ_reg == 2 && lds <= half) ? 2 : 1;
    const int nw = (occ == 1 && (e == 2 || (D <= 64 && D * C <= 4096))) ? 8 : 4;
    const int th = 64 * nw;
    const int lk = (C * (D / u) + th - 1) / th;
    const int lq = (GT * C * (D / u) + th - 1) / th;
    // Staging waves: every phase-2 item (query tile, output-column part) on
    // a wave of the first half of the workgroup, the second half staging
    // (state tiles stay spread over all waves); K, V and q double-buffered.
    // fp32 at d = 64 (its state tiles all sit on the first half anyway) and
    // 16-bit rows at d = 128, whose matrix work is small next to the bytes
    // each chunk moves, so deeper prefetch pays for fewer computing waves.
    const int dt = D / 32, nu = GT * ct, nwc = nw / 2;
    const int parts = nu >= nwc ? 1 : (nwc / nu < dt ? nwc / nu : dt);
    const unsigned long lds_pipe = (unsigned long)e * (4ul * C * D + 2ul * GT * C * D +
                                                       (unsigned long)nsc * ((unsigned long)D * D + D));
    const bool pipe = nw == 8 && occ == 1 && !shift && nu * parts <= nwc && lds_pipe <= full &&
                      ((e == 4 && D == 64 && dt * dt <= nwc) || (e == 2 && D == 128));
    const unsigned long lds_used = pipe ? lds_pipe : lds;
    MainShape m{nsc, occ, nw, lk, lq, shift, lds_used <= full && lq4 <= 8 && (shift || ct / nsc <= 2), lds_used, pipe};
    return m;
}

// How one linattn_fwd call is split into kernel launches.
//
// A sequence (one batch entry and kv head) of N tokens is cut into `segments`
// consecutive segments of `seg_len` tokens (a multiple of `chunk`; the last
// one may be shorter).  Causal: every segment but the last gets its key/value
// total phi(K)^T V and sum phi(K) from a first pass; a scan turns those into
// the state each segment starts from; the main pass then walks each segment
// chunk by chunk.  Non-causal: every segment writes a partial total, the
// partials are summed, and the sum is applied to every query.
struct Plan {
    int B, H, Hkv, N, d, G, causal, dtype;
    int chunk;       // tokens per intra-chunk block
    int gt;          // query heads per workgroup of the chunk kernel (divides G)
    int nseq;        // B * Hkv independent (batch, kv head) sequences
    int segments;    // segments per sequence
    int seg_len;     // tokens per segment (multiple of chunk)
    int ws_slots;    // fp32 partial states per sequence held in the workspace
    size_t ws_bytes; // workspace bytes: nseq * ws_slots * d * (d + 1) * 4 (dense)
    // packed batches (sequences of different lengths, no padding)
    int packed;      // 1: N is the total token count and segments an upper bound
    int nb;          // sequences
    size_t tab_off;  // byte offset of the segment tables in the workspace
    const int *cu = nullptr;  // device sequence offsets of a packed batch (set by the caller of the plan)
};

// Query heads per workgroup for (dtype, d, chunk, G): the largest of 8, 4,
// 2, 1 that divides G and whose kernel shape fits; 0 if none fits.
int heads_per_block(int dtype, int d, int chunk, int G);

// Chunk size used when the caller passes chunk = 0.
int auto_chunk(int dtype, int d, int G, int causal);

// Chunk size of a decayed pass of H query heads over Hkv kv heads: `chunk`
// itself when given, else the automatic one, capped at 64 tokens for 16-bit
// rows at d <= 64.
int decay_chunk(int dtype, int d, int H, int Hkv, int chunk);

// Fills `p` and returns LINATTN_OK or an error code (see linattn.h).
int make_plan(int B, int H, int Hkv, int N, int d, int causal, int dtype, int chunk, Plan *p);

// Plan of a packed batch of nb sequences with `total` tokens in all: one
// segment length for every sequence, launches sized for `segments` =
// ceil(total / seg_len) + nb segments (each sequence adds at most one partial
// segment), the workspace sized for that many partial states per kv head
// plus the segment tables.
int make_plan_packed(int nb, int H, int Hkv, int total, int d, int causal, int dtype, int chunk, Plan *p);

// Decayed sums (a log-decay per token) run on a dense causal plan with the
// default feature map and a chunk kernel that keeps one state copy per key
// tile or pair of tiles (never the shifted fp32 copies).
bool decay_ok(const Plan &p);
// Their workspace: the plan's slots plus one float per slot (the segment's
// summed log-decay), nseq * ws_slots * (d * (d + 1) + 1) * 4 bytes.
size_t decay_ws_bytes(const Plan &p);

}  // namespace linattn
