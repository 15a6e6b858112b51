// linattn_plan.cpp - argument validation and launch planning (host only).
#include "linattn_plan.h"

#include <stdint.h>

#include "linattn.h"

namespace linattn {

namespace {
constexpr size_t kLdsLimit = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kTargetWorkgroups = 512;    // two waves of workgroups over 256 CUs

bool valid_d(int d) { return d == 32 || d == 64 || d == 128; }
bool valid_chunk(int c) { return c == 32 || c == 64 || c == 128 || c == 256; }
}  // namespace

size_t chunk_kernel_lds_bytes(int dtype, int d, int chunk)
{
    const size_t e = dtype == LINATTN_BF16 ? 2 : 4;
    // phi(K) and V tiles (chunk x d each, single-buffered at least), one
    // transposed state copy (d x d) and one normaliser (d floats) per
    // 32-token key tile of the chunk.
    const size_t tiles = (size_t)chunk / 32;
    return e * 2 * (size_t)chunk * d + tiles * (e * (size_t)d * d + 4 * (size_t)d);
}

int auto_chunk(int dtype, int d, int G, int causal)
{
    (void)causal;
    (void)G;
    // The chunk only sets how many query tiles share one pass over the
    // state copies; 64 tokens keep the K/V tiles double-buffered in LDS.
    int c = 128;
    if (d >= 128) c = 32;
    if (dtype == LINATTN_F32) c = 32;
    while (c > 32 && chunk_kernel_lds_bytes(dtype, d, c) > kLdsLimit) c /= 2;
    return c;
}

int make_plan(int B, int H, int Hkv, int N, int d, int causal, int dtype, int chunk, Plan *p)
{
    if (dtype != LINATTN_F32 && dtype != LINATTN_BF16) return LINATTN_ERR_DTYPE;
    if (B < 0 || H <= 0 || Hkv <= 0 || N < 0 || d <= 0 || H % Hkv != 0) return LINATTN_ERR_SHAPE;
    if ((int64_t)B * H > INT32_MAX / 2 || (int64_t)N * d > INT32_MAX / 2) return LINATTN_ERR_SHAPE;
    if (!valid_d(d)) return LINATTN_ERR_UNSUPPORTED;
    if (chunk != 0 && !valid_chunk(chunk)) return LINATTN_ERR_UNSUPPORTED;
    const int G = H / Hkv;
    const int C = chunk ? chunk : auto_chunk(dtype, d, G, causal);
    if (chunk_kernel_lds_bytes(dtype, d, C) > kLdsLimit) return LINATTN_ERR_UNSUPPORTED;

    Plan q{};
    q.B = B; q.H = H; q.Hkv = Hkv; q.N = N; q.d = d; q.G = G;
    q.causal = causal ? 1 : 0;
    q.dtype = dtype;
    q.chunk = C;
    q.nseq = B * Hkv;
    q.segments = 0;
    q.seg_len = 0;
    q.ws_slots = 0;
    q.ws_bytes = 0;
    if (B > 0 && N > 0) {
        const int nchunks = (N + C - 1) / C;
        int P = (kTargetWorkgroups + q.nseq - 1) / q.nseq;
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

}  // namespace linattn
