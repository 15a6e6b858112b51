// linattn.hip - the C ABI of liblinattn.so (declared in include/linattn.h):
// argument checks, planning, and the call into the launchers of the requested
// format (linattn_fmt.hip, one object per feature map and element type).
//
// Linear attention with phi(x) = ELU(x) + 1 (LinearTile 1.0.0 README, "How It
// Works": O = phi(Q) (phi(K)^T V), key/value product first), causal rows from
// the running sums S_t = sum_{s<=t} phi(k_s) v_s^T and z_t = sum_{s<=t} phi(k_s)
// (Katharopoulos et al. 2020, cited in the README's "Reference" section).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "linattn.h"
#include "linattn_fwd.h"
#include "linattn_kern.h"
#include "linattn_plan.h"

namespace {

using linattn::record;
using linattn::Start;
using linattn::Timing;

// p[i] = src ? src[i] : 0 (a kernel rather than a memset node, so that the
// call can be captured in a graph).
__global__ void k_fill_copy(float *__restrict__ p, const float *__restrict__ src, size_t n)
{
    for (size_t i = blockIdx.x * (size_t)kThreads + threadIdx.x; i < n; i += (size_t)gridDim.x * kThreads)
        p[i] = src ? src[i] : 0.f;
}

#define LINATTN_FORMATS(X)                                                                                     \
    X(LINATTN_PHI_ELU1, LINATTN_F32)                                                                           \
    X(LINATTN_PHI_ELU1, LINATTN_BF16)                                                                          \
    X(LINATTN_PHI_ELU1, LINATTN_F16)                                                                           \
    X(LINATTN_PHI_ELU1, LINATTN_FP8_E4M3)                                                                      \
    X(LINATTN_PHI_ELU1, LINATTN_FP8_E5M2)                                                                      \
    X(LINATTN_PHI_RELU, LINATTN_F32)                                                                           \
    X(LINATTN_PHI_RELU, LINATTN_BF16)                                                                          \
    X(LINATTN_PHI_RELU, LINATTN_F16)                                                                           \
    X(LINATTN_PHI_RELU, LINATTN_FP8_E4M3)                                                                      \
    X(LINATTN_PHI_RELU, LINATTN_FP8_E5M2)                                                                      \
    X(LINATTN_PHI_SOFTPLUS, LINATTN_F32)                                                                       \
    X(LINATTN_PHI_SOFTPLUS, LINATTN_BF16)                                                                      \
    X(LINATTN_PHI_SOFTPLUS, LINATTN_F16)                                                                       \
    X(LINATTN_PHI_SOFTPLUS, LINATTN_FP8_E4M3)                                                                  \
    X(LINATTN_PHI_SOFTPLUS, LINATTN_FP8_E5M2)

// dtype: element type in bits 0-7, feature map in bits 8-15
int fwd_dispatch(int dtype, const linattn::FwdCall &c)
{
    if (!valid_dtype(dtype)) return LINATTN_ERR_DTYPE;
    switch (dtype) {
#define LINATTN_CASE(PHI, ELEM) \
    case (PHI << 8) | ELEM: return linattn::fwd_format<PHI, ELEM>(c);
        LINATTN_FORMATS(LINATTN_CASE)
#undef LINATTN_CASE
    }
    return LINATTN_ERR_DTYPE;
}

int decode_dispatch(int dtype, const linattn::DecodeCall &c)
{
    if (!valid_dtype(dtype)) return LINATTN_ERR_DTYPE;
    switch (dtype) {
#define LINATTN_CASE(PHI, ELEM) \
    case (PHI << 8) | ELEM: return linattn::decode_format<PHI, ELEM>(c);
        LINATTN_FORMATS(LINATTN_CASE)
#undef LINATTN_CASE
    }
    return LINATTN_ERR_DTYPE;
}

int window_dispatch(int dtype, const linattn::WindowCall &c)
{
    if (!valid_dtype(dtype)) return LINATTN_ERR_DTYPE;
    switch (dtype) {
#define LINATTN_CASE(PHI, ELEM) \
    case (PHI << 8) | ELEM: return linattn::window_format<PHI, ELEM>(c);
        LINATTN_FORMATS(LINATTN_CASE)
#undef LINATTN_CASE
    }
    return LINATTN_ERR_DTYPE;
}

}  // namespace

// =================================================================== C ABI

extern "C" {

int linattn_abi_version(void) { return LINATTN_ABI_VERSION; }

const char *linattn_status_string(int status)
{
    switch (status) {
    case LINATTN_OK: return "ok";
    case LINATTN_ERR_NULL: return "a required pointer is NULL";
    case LINATTN_ERR_SHAPE: return "invalid shape (B, H, Hkv, N, d) or H % Hkv != 0";
    case LINATTN_ERR_DTYPE: return "unsupported dtype";
    case LINATTN_ERR_UNSUPPORTED: return "unsupported head dimension or chunk size";
    case LINATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case LINATTN_ERR_HIP: return "HIP launch failed";
    case LINATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case LINATTN_ERR_SCRATCH: return "problem needs more than the library's static scratch (LINATTN_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

int linattn_fwd_plan(int B, int H, int Hkv, int N, int d, int causal, int dtype, int chunk, int *chunk_out,
                     int *segments_out)
{
    linattn::Plan pl;
    const int rc = linattn::make_plan(B, H, Hkv, N, d, causal, dtype, chunk, &pl);
    if (rc != LINATTN_OK) return rc;
    if (chunk_out) *chunk_out = pl.chunk;
    if (segments_out) *segments_out = pl.segments;
    return LINATTN_OK;
}

size_t linattn_fwd_workspace_bytes(int B, int H, int Hkv, int N, int d, int causal, int dtype, int chunk)
{
    linattn::Plan pl;
    if (linattn::make_plan(B, H, Hkv, N, d, causal, dtype, chunk, &pl) != LINATTN_OK) return (size_t)-1;
    return pl.ws_bytes;
}

}  // extern "C"

namespace {
int fwd_impl(const void *q, const void *k, const void *v, void *out, int B, int H, int Hkv, int N, int d, int causal,
             int normalise, int dtype, float *state_out, float *z_out, int chunk, void *workspace,
             size_t workspace_bytes, hipStream_t stream, const Timing *ev, const Start &s0 = Start{nullptr, nullptr},
             bool packed = false, const int *cu = nullptr)
{
    // packed: B sequences of N tokens in all, delimited by cu[0..B] (device)
    linattn::Plan pl;
    const int rc = packed ? linattn::make_plan_packed(B, H, Hkv, N, d, causal, dtype, chunk, &pl)
                          : linattn::make_plan(B, H, Hkv, N, d, causal, dtype, chunk, &pl);
    if (rc != LINATTN_OK) return rc;
    const bool decay = s0.g != nullptr;
    if (decay && (packed || !causal || !linattn::decay_ok(pl))) return LINATTN_ERR_UNSUPPORTED;
    const size_t need = decay ? linattn::decay_ws_bytes(pl) : pl.ws_bytes;
    if (B == 0) return LINATTN_OK;
    if (packed && !cu) return LINATTN_ERR_NULL;
    pl.cu = cu;
    if (N > 0 && (!q || !k || !v || !out)) return LINATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(state_out) ||
        !aligned16(z_out) || !aligned16(workspace) || !aligned16(s0.S) || !aligned16(s0.z) || ((uintptr_t)s0.g & 3u))
        return LINATTN_ERR_ALIGN;
    if (need > 0 && (!workspace || workspace_bytes < need)) return LINATTN_ERR_WORKSPACE;
    if (N == 0) {
        // No keys: the state and normaliser are the start sums (zero unless
        // continuing); there is no output row.
        if (state_out)
            hipLaunchKernelGGL(k_fill_copy, dim3(256), dim3(kThreads), 0, stream, state_out, s0.S, (size_t)pl.nseq * d * d);
        if (z_out) hipLaunchKernelGGL(k_fill_copy, dim3(16), dim3(kThreads), 0, stream, z_out, s0.z, (size_t)pl.nseq * d);
        return launch_status();
    }
    const linattn::FwdCall c{&pl, q, k, v, out, state_out, z_out, static_cast<float *>(workspace),
                             normalise ? 1 : 0, stream, ev, s0};
    return fwd_dispatch(dtype, c);
}
}  // namespace

extern "C" {

int linattn_fwd(const void *q, const void *k, const void *v, void *out, int B, int H, int Hkv, int N, int d,
                int causal, int normalise, int dtype, float *state_out, float *z_out, int chunk, void *workspace,
                size_t workspace_bytes, hipStream_t stream)
{
    return fwd_impl(q, k, v, out, B, H, Hkv, N, d, causal, normalise, dtype, state_out, z_out, chunk, workspace,
                    workspace_bytes, stream, nullptr);
}

int linattn_fwd_from_state(const void *q, const void *k, const void *v, void *out, int B, int H, int Hkv, int N,
                           int d, int causal, int normalise, int dtype, const float *state_in, const float *z_in,
                           float *state_out, float *z_out, int chunk, void *workspace, size_t workspace_bytes,
                           hipStream_t stream)
{
    if (B > 0 && (!state_in || (normalise && !z_in))) return LINATTN_ERR_NULL;
    if ((state_out && (const float *)state_out == state_in) || (z_out && z_in && (const float *)z_out == z_in))
        return LINATTN_ERR_SHAPE;  // the start sums are read while the final ones are written
    return fwd_impl(q, k, v, out, B, H, Hkv, N, d, causal, normalise, dtype, state_out, z_out, chunk, workspace,
                    workspace_bytes, stream, nullptr, Start{state_in, z_in});
}

size_t linattn_fwd_decay_workspace_bytes(int B, int H, int Hkv, int N, int d, int dtype, int chunk)
{
    linattn::Plan pl;
    if (linattn::make_plan(B, H, Hkv, N, d, 1, dtype, linattn::decay_chunk(dtype, d, H, Hkv, chunk), &pl) !=
            LINATTN_OK ||
        !linattn::decay_ok(pl))
        return (size_t)-1;
    return linattn::decay_ws_bytes(pl);
}

int linattn_fwd_decay(const void *q, const void *k, const void *v, const float *g, void *out, int B, int H, int Hkv,
                      int N, int d, int normalise, int dtype, const float *state_in, const float *z_in,
                      float *state_out, float *z_out, int chunk, void *workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    if (B > 0 && N > 0 && !g) return LINATTN_ERR_NULL;
    if ((state_out && state_in && (const float *)state_out == state_in) ||
        (z_out && z_in && (const float *)z_out == z_in))
        return LINATTN_ERR_SHAPE;  // the start sums are read while the final ones are written
    // a g pointer is what selects the decayed kernels: with N == 0 none is read
    static const float no_tokens = 0.f;
    return fwd_impl(q, k, v, out, B, H, Hkv, N, d, 1, normalise, dtype, state_out, z_out,
                    linattn::decay_chunk(dtype, d, H, Hkv, chunk), workspace, workspace_bytes, stream, nullptr,
                    Start{state_in, z_in, g ? g : &no_tokens});
}

size_t linattn_fwd_packed_workspace_bytes(int nseqs, int H, int Hkv, int total, int d, int causal, int dtype,
                                          int chunk)
{
    linattn::Plan pl;
    if (linattn::make_plan_packed(nseqs, H, Hkv, total, d, causal, dtype, chunk, &pl) != LINATTN_OK) return (size_t)-1;
    return pl.ws_bytes;
}

int linattn_fwd_packed(const void *q, const void *k, const void *v, void *out, const int *cu_seqlens, int nseqs,
                       int total, int H, int Hkv, int d, int causal, int normalise, int dtype, float *state_out,
                       float *z_out, int chunk, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return fwd_impl(q, k, v, out, nseqs, H, Hkv, total, d, causal, normalise, dtype, state_out, z_out, chunk,
                    workspace, workspace_bytes, stream, nullptr, Start{nullptr, nullptr}, true, cu_seqlens);
}

int linattn_fwd_timed(const void *q, const void *k, const void *v, void *out, int B, int H, int Hkv, int N, int d,
                      int causal, int normalise, int dtype, float *state_out, float *z_out, int chunk,
                      void *workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t *events, int n_events,
                      int reps)
{
    if (!events || n_events != 4) return LINATTN_ERR_NULL;
    for (int i = 0; i < 4; ++i)
        if (!events[i]) return LINATTN_ERR_NULL;
    if (reps < 0) return LINATTN_ERR_SHAPE;
    const Timing t{events, reps};
    if (B > 0 && N > 0)
        return fwd_impl(q, k, v, out, B, H, Hkv, N, d, causal, normalise, dtype, state_out, z_out, chunk,
                        workspace, workspace_bytes, stream, &t);
    // Nothing to stage: every event marks the same point.
    const int rc = fwd_impl(q, k, v, out, B, H, Hkv, N, d, causal, normalise, dtype, state_out, z_out, chunk,
                            workspace, workspace_bytes, stream, nullptr);
    if (rc != LINATTN_OK) return rc;
    for (int i = 0; i < 4; ++i)
        if (record(&t, i, stream)) return LINATTN_ERR_HIP;
    return LINATTN_OK;
}

}  // extern "C"

// ------------------------------------------------ forward without allocation
//
// linattn_fwd_noalloc runs linattn_fwd with the library's own device scratch
// instead of a caller's workspace: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol); each device's address is taken once with hipGetSymbolAddress,
// with that device current, and kept in scratch_ptr[device].  Nothing in the
// scratch has to start at zero: every pass writes the slots it later reads.
namespace {
static __device__ __align__(256) float scratch[LINATTN_NOALLOC_SCRATCH_BYTES / sizeof(float)];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];

// Address of this library's scratch on the device that runs `stream`.
int scratch_for(hipStream_t stream, void **out)
{
    int dev = -1, cur = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || hipGetDevice(&cur) != hipSuccess) return LINATTN_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return LINATTN_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return LINATTN_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return LINATTN_ERR_HIP;
        if (e != hipSuccess || !p) return LINATTN_ERR_HIP;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return LINATTN_OK;
}
}  // namespace

extern "C" {

int linattn_fwd_noalloc(const void *q, const void *k, const void *v, void *out, int B, int H, int Hkv, int N, int d,
                        int causal, int normalise, int dtype, float *state_out, float *z_out, int chunk,
                        hipStream_t stream)
{
    const size_t need = linattn_fwd_workspace_bytes(B, H, Hkv, N, d, causal, dtype, chunk);
    if (need == (size_t)-1) {
        linattn::Plan pl;
        return linattn::make_plan(B, H, Hkv, N, d, causal, dtype, chunk, &pl);
    }
    if (need > LINATTN_NOALLOC_SCRATCH_BYTES) return LINATTN_ERR_SCRATCH;
    void *ws = nullptr;
    if (need > 0) {
        const int rc = scratch_for(stream, &ws);
        if (rc != LINATTN_OK) return rc;
    }
    return fwd_impl(q, k, v, out, B, H, Hkv, N, d, causal, normalise, dtype, state_out, z_out, chunk, ws,
                    LINATTN_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

}  // extern "C"

namespace {
int decode_impl(float *state, float *z, const void *q, const void *k, const void *v, const float *g, void *out, int B,
                int H, int Hkv, int d, int normalise, int dtype, hipStream_t stream)
{
    if (!valid_dtype(dtype)) return LINATTN_ERR_DTYPE;
    if (B < 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || (int64_t)B * Hkv > INT32_MAX) return LINATTN_ERR_SHAPE;
    if (d != 32 && d != 64 && d != 128) return LINATTN_ERR_UNSUPPORTED;
    if (B == 0) return LINATTN_OK;
    if (!state || !q || !k || !v || !out || (normalise && !z)) return LINATTN_ERR_NULL;
    if (!aligned16(state) || !aligned16(z) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        ((uintptr_t)g & 3u))
        return LINATTN_ERR_ALIGN;
    const linattn::DecodeCall c{state, z, q, k, v, g, out, B, H, Hkv, d, normalise ? 1 : 0, stream};
    return decode_dispatch(dtype, c);
}
}  // namespace

extern "C" {

int linattn_decode_step(float *state, float *z, const void *q, const void *k, const void *v, void *out, int B, int H,
                        int Hkv, int d, int normalise, int dtype, hipStream_t stream)
{
    return decode_impl(state, z, q, k, v, nullptr, out, B, H, Hkv, d, normalise, dtype, stream);
}

int linattn_fwd_window(const void *q, const void *k, const void *v, void *out, int B, int H, int Hkv, int N, int d,
                       int window, int normalise, int dtype, hipStream_t stream)
{
    if (!valid_dtype(dtype)) return LINATTN_ERR_DTYPE;
    if (B < 0 || H <= 0 || Hkv <= 0 || N < 0 || H % Hkv != 0 || window < 1) return LINATTN_ERR_SHAPE;
    if (d != 32 && d != 64 && d != 128) return LINATTN_ERR_UNSUPPORTED;
    if ((int64_t)N * d > INT32_MAX / 4) return LINATTN_ERR_SHAPE;  // byte offsets of one head stay 32-bit
    const int64_t blocks = (int64_t)B * H * ((N + 127) / 128);
    if (blocks > INT32_MAX) return LINATTN_ERR_SHAPE;
    if (B == 0 || N == 0) return LINATTN_OK;
    if (!q || !k || !v || !out) return LINATTN_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return LINATTN_ERR_ALIGN;
    const linattn::WindowCall c{q, k, v, out, B, H, Hkv, N, d, window, normalise ? 1 : 0, stream};
    return window_dispatch(dtype, c);
}

int linattn_decode_step_decay(float *state, float *z, const void *q, const void *k, const void *v, const float *g,
                              void *out, int B, int H, int Hkv, int d, int normalise, int dtype, hipStream_t stream)
{
    if (B > 0 && !g) return LINATTN_ERR_NULL;
    return decode_impl(state, z, q, k, v, g, out, B, H, Hkv, d, normalise, dtype, stream);
}

}  // extern "C"
