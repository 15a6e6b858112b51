"""Python binding of liblinattn.so (ELU+1 linear attention on MI355X / gfx950).

The functions below carry the C ABI's names and arguments (see
``include/linattn.h``) and do argument marshalling only: torch tensors are
passed as their device pointers, ``stream=None`` means torch's current stream.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  If the library is not built this module raises on first use.

``ops`` holds convenience wrappers that allocate outputs and the workspace
with torch and then call these functions.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LINATTN_F32", "LINATTN_BF16", "LINATTN_F16", "LINATTN_OK", "LinattnError", "library_path", "load",
    "linattn_fwd", "linattn_fwd_from_state", "linattn_fwd_timed", "linattn_fwd_workspace_bytes", "linattn_fwd_plan", "linattn_decode_step",
    "linattn_status_string", "linattn_abi_version", "linattn_bwd", "linattn_bwd_workspace_bytes",
    "linattn_fwd_packed", "linattn_fwd_packed_workspace_bytes", "linattn_fwd_noalloc", "linattn_fwd_window",
    "LINATTN_NOALLOC_SCRATCH_BYTES",
]

LINATTN_F32 = 0
LINATTN_BF16 = 1
LINATTN_F16 = 2
LINATTN_OK = 0
ERRORS = {
    -1: "LINATTN_ERR_NULL", -2: "LINATTN_ERR_SHAPE", -3: "LINATTN_ERR_DTYPE",
    -4: "LINATTN_ERR_UNSUPPORTED", -5: "LINATTN_ERR_WORKSPACE", -6: "LINATTN_ERR_HIP",
    -7: "LINATTN_ERR_ALIGN", -8: "LINATTN_ERR_SCRATCH",
}
# size of the library's static device scratch used by linattn_fwd_noalloc
LINATTN_NOALLOC_SCRATCH_BYTES = 64 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblinattn.so")
_lib = None


class LinattnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where} failed: {ERRORS.get(code, code)} ({linattn_status_string(code)})")


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load liblinattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m sequence_mixing_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        lib.linattn_fwd.restype = i
        lib.linattn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, i, vp, sz, vp]
        lib.linattn_fwd_from_state.restype = i
        lib.linattn_fwd_from_state.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, vp, vp, i, vp, sz, vp]
        lib.linattn_fwd_timed.restype = i
        lib.linattn_fwd_timed.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, i, vp, sz, vp,
                                          ctypes.POINTER(vp), i, i]
        lib.linattn_fwd_noalloc.restype = i
        lib.linattn_fwd_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, i, vp]
        lib.linattn_fwd_workspace_bytes.restype = sz
        lib.linattn_fwd_workspace_bytes.argtypes = [i] * 8
        lib.linattn_fwd_plan.restype = i
        lib.linattn_fwd_plan.argtypes = [i] * 8 + [ctypes.POINTER(i), ctypes.POINTER(i)]
        lib.linattn_fwd_window.restype = i
        lib.linattn_fwd_window.argtypes = [vp] * 4 + [i] * 8 + [vp]
        lib.linattn_decode_step.restype = i
        lib.linattn_decode_step.argtypes = [vp] * 6 + [i] * 6 + [vp]
        lib.linattn_fwd_packed.restype = i
        lib.linattn_fwd_packed.argtypes = [vp] * 5 + [i] * 8 + [vp, vp, i, vp, sz, vp]
        lib.linattn_fwd_packed_workspace_bytes.restype = sz
        lib.linattn_fwd_packed_workspace_bytes.argtypes = [i] * 8
        lib.linattn_bwd.restype = i
        lib.linattn_bwd.argtypes = [vp] * 8 + [i] * 8 + [vp, sz, vp]
        lib.linattn_bwd_workspace_bytes.restype = sz
        lib.linattn_bwd_workspace_bytes.argtypes = [i] * 7
        lib.linattn_fwd_decay.restype = i
        lib.linattn_fwd_decay.argtypes = [vp] * 5 + [i] * 7 + [vp] * 4 + [i, vp, sz, vp]
        lib.linattn_fwd_decay_workspace_bytes.restype = sz
        lib.linattn_fwd_decay_workspace_bytes.argtypes = [i] * 7
        lib.linattn_decode_step_decay.restype = i
        lib.linattn_decode_step_decay.argtypes = [vp] * 7 + [i] * 6 + [vp]
        lib.linattn_status_string.restype = ctypes.c_char_p
        lib.linattn_status_string.argtypes = [i]
        lib.linattn_abi_version.restype = i
        lib.linattn_abi_version.argtypes = []
        _lib = lib
    return _lib


def _ptr(x):
    """Device pointer of a tensor (or an int address, or None for NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def linattn_fwd(q, k, v, out, B, H, Hkv, N, d, causal, normalise, dtype, state_out=None, z_out=None,
                chunk=0, workspace=None, workspace_bytes=0, stream=None) -> int:
    """C ``linattn_fwd``; returns the status code (0 = ok)."""
    return load().linattn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, N, d, int(causal),
                              int(normalise), dtype, _ptr(state_out), _ptr(z_out), chunk, _ptr(workspace),
                              workspace_bytes, _stream(stream))


def linattn_fwd_noalloc(q, k, v, out, B, H, Hkv, N, d, causal, normalise, dtype, state_out=None, z_out=None,
                        chunk=0, stream=None) -> int:
    """C ``linattn_fwd_noalloc`` (the library's static scratch, no workspace); returns the status code."""
    return load().linattn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, N, d, int(causal),
                                      int(normalise), dtype, _ptr(state_out), _ptr(z_out), chunk, _stream(stream))


def linattn_fwd_from_state(q, k, v, out, B, H, Hkv, N, d, causal, normalise, dtype, state_in, z_in,
                           state_out=None, z_out=None, chunk=0, workspace=None, workspace_bytes=0,
                           stream=None) -> int:
    """C ``linattn_fwd_from_state``; returns the status code (0 = ok)."""
    return load().linattn_fwd_from_state(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, N, d, int(causal),
                                         int(normalise), dtype, _ptr(state_in), _ptr(z_in), _ptr(state_out),
                                         _ptr(z_out), chunk, _ptr(workspace), workspace_bytes, _stream(stream))


def linattn_fwd_timed(q, k, v, out, B, H, Hkv, N, d, causal, normalise, dtype, state_out=None, z_out=None,
                      chunk=0, workspace=None, workspace_bytes=0, stream=None, events=(), reps=1) -> int:
    """C ``linattn_fwd_timed``; ``events`` are 4 raw hipEvent_t handles (ints)."""
    arr = (ctypes.c_void_p * len(events))(*events) if events else None
    return load().linattn_fwd_timed(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, N, d, int(causal),
                                    int(normalise), dtype, _ptr(state_out), _ptr(z_out), chunk, _ptr(workspace),
                                    workspace_bytes, _stream(stream), arr, len(events), reps)


def linattn_fwd_workspace_bytes(B, H, Hkv, N, d, causal, dtype, chunk=0) -> int:
    """C ``linattn_fwd_workspace_bytes``; returns -1 for invalid arguments."""
    r = load().linattn_fwd_workspace_bytes(B, H, Hkv, N, d, int(causal), dtype, chunk)
    return -1 if r == ctypes.c_size_t(-1).value else r


def linattn_fwd_plan(B, H, Hkv, N, d, causal, dtype, chunk=0):
    """C ``linattn_fwd_plan``; returns (status, chunk, segments)."""
    c, p = ctypes.c_int(0), ctypes.c_int(0)
    rc = load().linattn_fwd_plan(B, H, Hkv, N, d, int(causal), dtype, chunk, ctypes.byref(c), ctypes.byref(p))
    return rc, c.value, p.value


def linattn_fwd_window(q, k, v, out, B, H, Hkv, N, d, window, normalise, dtype, stream=None) -> int:
    """C ``linattn_fwd_window``; returns the status code (0 = ok)."""
    return load().linattn_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, N, d, int(window),
                                     int(normalise), dtype, _stream(stream))


def linattn_decode_step(state, z, q, k, v, out, B, H, Hkv, d, normalise, dtype, stream=None) -> int:
    """C ``linattn_decode_step``; returns the status code (0 = ok)."""
    return load().linattn_decode_step(_ptr(state), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, d,
                                      int(normalise), dtype, _stream(stream))


def linattn_fwd_packed(q, k, v, out, cu_seqlens, nseqs, total, H, Hkv, d, causal, normalise, dtype, state_out=None,
                       z_out=None, chunk=0, workspace=None, workspace_bytes=0, stream=None) -> int:
    """C ``linattn_fwd_packed``; returns the status code (0 = ok)."""
    return load().linattn_fwd_packed(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(cu_seqlens), nseqs, total, H, Hkv, d,
                                     int(causal), int(normalise), dtype, _ptr(state_out), _ptr(z_out), chunk,
                                     _ptr(workspace), workspace_bytes, _stream(stream))


def linattn_fwd_packed_workspace_bytes(nseqs, H, Hkv, total, d, causal, dtype, chunk=0) -> int:
    """C ``linattn_fwd_packed_workspace_bytes``; returns -1 for invalid arguments."""
    r = load().linattn_fwd_packed_workspace_bytes(nseqs, H, Hkv, total, d, int(causal), dtype, chunk)
    return -1 if r == ctypes.c_size_t(-1).value else r


def linattn_bwd(q, k, v, out, dout, dq, dk, dv, B, H, Hkv, N, d, causal, normalise, dtype, workspace=None,
                workspace_bytes=0, stream=None) -> int:
    """C ``linattn_bwd``; returns the status code (0 = ok)."""
    return load().linattn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H,
                              Hkv, N, d, int(causal), int(normalise), dtype, _ptr(workspace), workspace_bytes,
                              _stream(stream))


def linattn_bwd_workspace_bytes(B, H, Hkv, N, d, causal, dtype) -> int:
    """C ``linattn_bwd_workspace_bytes``; returns -1 for invalid arguments."""
    r = load().linattn_bwd_workspace_bytes(B, H, Hkv, N, d, int(causal), dtype)
    return -1 if r == ctypes.c_size_t(-1).value else r


def linattn_fwd_decay(q, k, v, g, out, B, H, Hkv, N, d, normalise, dtype, state_in=None, z_in=None,
                      state_out=None, z_out=None, chunk=0, workspace=None, workspace_bytes=0, stream=None) -> int:
    """C ``linattn_fwd_decay``; returns the status code (0 = ok)."""
    return load().linattn_fwd_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), B, H, Hkv, N, d, int(normalise),
                                    dtype, _ptr(state_in), _ptr(z_in), _ptr(state_out), _ptr(z_out), chunk,
                                    _ptr(workspace), workspace_bytes, _stream(stream))


def linattn_fwd_decay_workspace_bytes(B, H, Hkv, N, d, dtype, chunk=0) -> int:
    """C ``linattn_fwd_decay_workspace_bytes``; returns -1 for arguments it rejects."""
    r = load().linattn_fwd_decay_workspace_bytes(B, H, Hkv, N, d, dtype, chunk)
    return -1 if r == ctypes.c_size_t(-1).value else r


def linattn_decode_step_decay(state, z, q, k, v, g, out, B, H, Hkv, d, normalise, dtype, stream=None) -> int:
    """C ``linattn_decode_step_decay``; returns the status code (0 = ok)."""
    return load().linattn_decode_step_decay(_ptr(state), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), B,
                                            H, Hkv, d, int(normalise), dtype, _stream(stream))


def linattn_status_string(code: int) -> str:
    return load().linattn_status_string(code).decode()


def linattn_abi_version() -> int:
    return load().linattn_abi_version()
