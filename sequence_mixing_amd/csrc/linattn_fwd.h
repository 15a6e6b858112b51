// linattn_fwd.h - the interface between the C ABI (linattn.hip) and the
// forward/decode launchers, which are built once per (feature map, element
// type) in separate translation units from linattn_fmt.hip.  Internal header;
// host types only.
#pragma once
#include <hip/hip_runtime_api.h>

#include "linattn.h"
#include "linattn_plan.h"

namespace linattn {

// Sums of earlier tokens a forward pass continues from (both nullable).
struct Start {
    const float *S;
    const float *z;
    const float *g = nullptr;  // decayed sums: log-decay [seq][N] (dense causal only)
};

// Stage timing (nullable): 4 events recorded before each of the three stages
// and after the last; the last stage is launched `reps` times in between.
struct Timing {
    hipEvent_t *ev;
    int reps;
};
inline int record(const Timing *t, int i, hipStream_t st)
{
    return (t && hipEventRecord(t->ev[i], st) != hipSuccess) ? LINATTN_ERR_HIP : LINATTN_OK;
}

// One forward pass as planned by `pl` (arguments checked by the caller).
struct FwdCall {
    const Plan *pl;
    const void *q, *k, *v;
    void *out;
    float *state_out, *z_out, *ws;
    int normalise;
    hipStream_t stream;
    const Timing *ev;
    Start s0;
};

// One decode step (arguments checked by the caller); g is the log-decay or NULL.
struct DecodeCall {
    float *state, *z;
    const void *q, *k, *v;
    const float *g;
    void *out;
    int B, H, Hkv, d, normalise;
    hipStream_t stream;
};

// One sliding-window forward pass (arguments checked by the caller).
struct WindowCall {
    const void *q, *k, *v;
    void *out;
    int B, H, Hkv, N, d, window, normalise;
    hipStream_t stream;
};

// PHI: LINATTN_PHI_*; ELEM: LINATTN_F32 / LINATTN_BF16 / LINATTN_F16.  Each
// pair is defined in the object built from linattn_fmt.hip with
// -DLINATTN_FMT_PHI=PHI -DLINATTN_FMT_ELEM=ELEM.
template <int PHI, int ELEM> int fwd_format(const FwdCall &c);
template <int PHI, int ELEM> int decode_format(const DecodeCall &c);
template <int PHI, int ELEM> int window_format(const WindowCall &c);

}  // namespace linattn
