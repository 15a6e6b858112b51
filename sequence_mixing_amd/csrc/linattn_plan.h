// linattn_plan.h - argument validation and launch planning for liblinattn
// (host only, no HIP calls; unit-tested on machines without a GPU).
#pragma once
#include <stddef.h>

namespace linattn {

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
    int nseq;        // B * Hkv independent (batch, kv head) sequences
    int segments;    // segments per sequence
    int seg_len;     // tokens per segment (multiple of chunk)
    int ws_slots;    // fp32 partial states per sequence held in the workspace
    size_t ws_bytes; // workspace bytes: nseq * ws_slots * d * (d + 1) * 4
};

// Bytes of LDS the chunk kernel needs for (dtype, d, chunk).
size_t chunk_kernel_lds_bytes(int dtype, int d, int chunk);

// Chunk size used when the caller passes chunk = 0.
int auto_chunk(int dtype, int d, int G, int causal);

// Fills `p` and returns LINATTN_OK or an error code (see linattn.h).
int make_plan(int B, int H, int Hkv, int N, int d, int causal, int dtype, int chunk, Plan *p);

}  // namespace linattn
