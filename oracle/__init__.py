"""fp64 CPU oracle for ELU+1 linear attention (test infrastructure only).

The oracle is the slow, plainly written checker the GPU library is compared
against.  Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg may import it; the product path never does.  It shares no
code with the HIP library: the arithmetic lives in ``linattn_ref.c`` (plain C,
double precision), this module only converts arrays and calls it.

Definition followed (LinearTile 1.0.0 README, "How It Works"; causal form
from its "Features" list and Katharopoulos et al. 2020 cited under its
"Reference" section): O = phi(Q) (phi(K)^T V), phi = ELU + 1, causal rows
see keys s <= t, optional normaliser phi(q_t) . z_t.  The sliding window
(a reading of the "Features" list's sliding-window item) restricts query t
to the keys t - W < s <= t.  The backward pass is the
chain rule on that definition, with the reverse-time walk of a running sum
(Stream efficiency essay, section 4.2).  The decayed variant multiplies the
running sums by exp(g_t) before token t is added, the essay's scan form
h_t = h_{t-1} a_t + b_t carried over to S and z (a reading: the pages give no
decayed linear attention).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "linattn_ref.c")
_LIB_PATH = os.path.join(_HERE, "liblinattn_ref.so")
# A test may point the wrapper at a deliberately broken build of the oracle
# (mutation tests); normal use never sets this.
_LIB_OVERRIDE = os.environ.get("LINATTN_REF_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE double, no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
             "-shared", _SRC, "-o", tmp, "-lm", "-lpthread"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB_PATH
        if not _LIB_OVERRIDE and not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.linattn_ref_set_feature_map.restype = ctypes.c_int
        lib.linattn_ref_set_feature_map.argtypes = [ctypes.c_int]
        lib.linattn_ref_phi.restype = ctypes.c_double
        lib.linattn_ref_phi.argtypes = [ctypes.c_double]
        lib.linattn_ref_fwd.restype = ctypes.c_int
        lib.linattn_ref_fwd.argtypes = [dp, dp, dp, dp] + [ctypes.c_int] * 7 + [dp, dp, ctypes.c_int]
        lib.linattn_ref_fwd_from.restype = ctypes.c_int
        lib.linattn_ref_fwd_from.argtypes = [dp, dp, dp, dp] + [ctypes.c_int] * 7 + [dp, dp, dp, dp, ctypes.c_int]
        lib.linattn_ref_dphi.restype = ctypes.c_double
        lib.linattn_ref_dphi.argtypes = [ctypes.c_double]
        lib.linattn_ref_bwd.restype = ctypes.c_int
        lib.linattn_ref_bwd.argtypes = [dp] * 8 + [ctypes.c_int] * 8
        lib.linattn_ref_decode_step.restype = ctypes.c_int
        lib.linattn_ref_decode_step.argtypes = [dp] * 6 + [ctypes.c_int] * 5
        lib.linattn_ref_fwd_decay.restype = ctypes.c_int
        lib.linattn_ref_fwd_decay.argtypes = [dp] * 5 + [ctypes.c_int] * 6 + [dp] * 4 + [ctypes.c_int]
        lib.linattn_ref_fwd_window.restype = ctypes.c_int
        lib.linattn_ref_fwd_window.argtypes = [dp, dp, dp, dp] + [ctypes.c_int] * 8
        lib.linattn_ref_decode_step_decay.restype = ctypes.c_int
        lib.linattn_ref_decode_step_decay.argtypes = [dp] * 7 + [ctypes.c_int] * 5
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Exact fp64 copy of a numpy array or a CPU torch tensor (fp32/bf16/fp64)."""
    if hasattr(x, "detach"):  # torch tensor: widen exactly through float64
        import torch

        x = x.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# Feature maps the oracle knows: the README's ELU + 1 (the default), ReLU, softplus.
FEATURE_MAPS = {"elu1": 0, "relu": 1, "softplus": 2}


def _use(phi_map: str):
    if _load().linattn_ref_set_feature_map(FEATURE_MAPS[phi_map]) != 0:
        raise ValueError(phi_map)


def dphi(x: float, phi_map: str = "elu1") -> float:
    """d phi / dx of the selected feature map, evaluated by the C oracle."""
    _use(phi_map)
    try:
        return _load().linattn_ref_dphi(float(x))
    finally:
        _use("elu1")


def phi(x: float, phi_map: str = "elu1") -> float:
    """The selected feature map (default ELU + 1), evaluated by the C oracle."""
    _use(phi_map)
    try:
        return _load().linattn_ref_phi(float(x))
    finally:
        _use("elu1")


def ref_fwd(q, k, v, causal: bool = True, normalise: bool = True,
            want_state: bool = False, nthreads: int | None = None, state_in=None, z_in=None, phi_map: str = "elu1"):
    """Forward pass.  q [B,H,N,d], k/v [B,Hkv,N,d] -> out [B,H,N,d] (fp64).

    With ``want_state`` also returns S_N [B,Hkv,d,d] and z_N [B,Hkv,d].
    ``state_in`` [B,Hkv,d,d] / ``z_in`` [B,Hkv,d] (optional): the sums of
    earlier tokens that S and z start from (zero when omitted).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == (B, Hkv, N, d)
    Si = None if state_in is None else _f64(state_in)
    zi = None if z_in is None else _f64(z_in)
    assert Si is None or Si.shape == (B, Hkv, d, d)
    assert zi is None or zi.shape == (B, Hkv, d)
    out = np.zeros((B, H, N, d), dtype=np.float64)
    S = np.zeros((B, Hkv, d, d), dtype=np.float64) if want_state else None
    z = np.zeros((B, Hkv, d), dtype=np.float64) if want_state else None
    _use(phi_map)
    try:
        rc = _load().linattn_ref_fwd_from(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, N, d,
                                          int(bool(causal)), int(bool(normalise)), _ptr(Si), _ptr(zi),
                                          _ptr(S), _ptr(z), nthreads or default_threads())
    finally:
        _use("elu1")
    if rc != 0:
        raise ValueError(f"linattn_ref_fwd_from rejected its arguments (rc={rc})")
    return (out, S, z) if want_state else out


def ref_fwd_window(q, k, v, window: int, normalise: bool = True, nthreads: int | None = None,
                   phi_map: str = "elu1"):
    """Sliding-window forward pass: query t sees keys t - window < s <= t.
    q [B,H,N,d], k/v [B,Hkv,N,d] -> out [B,H,N,d] (fp64)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == (B, Hkv, N, d)
    out = np.zeros((B, H, N, d), dtype=np.float64)
    _use(phi_map)
    try:
        rc = _load().linattn_ref_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, Hkv, N, d, int(window),
                                            int(bool(normalise)), nthreads or default_threads())
    finally:
        _use("elu1")
    if rc != 0:
        raise ValueError(f"linattn_ref_fwd_window rejected its arguments (rc={rc})")
    return out


def ref_bwd(q, k, v, out, dout, causal: bool = True, normalise: bool = True, nthreads: int | None = None,
            phi_map: str = "elu1"):
    """Backward pass.  q/out/dout [B,H,N,d], k/v [B,Hkv,N,d] -> (dq, dk, dv) in fp64.

    ``out`` is the forward output the gradient of the normaliser uses (may be
    None when ``normalise`` is false)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    o = None if out is None else _f64(out)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == (B, Hkv, N, d) and dout.shape == q.shape
    assert o is None or o.shape == q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    _use(phi_map)
    try:
        rc = _load().linattn_ref_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                     B, H, Hkv, N, d, int(bool(causal)), int(bool(normalise)),
                                     nthreads or default_threads())
    finally:
        _use("elu1")
    if rc != 0:
        raise ValueError(f"linattn_ref_bwd rejected its arguments (rc={rc})")
    return dq, dk, dv


def ref_decode_step(S: np.ndarray, z: np.ndarray | None, q, k, v, normalise: bool = True, phi_map: str = "elu1"):
    """One decode step; S [B,Hkv,d,d] and z [B,Hkv,d] (fp64) are updated in place.

    q [B,H,d], k/v [B,Hkv,d]; returns out [B,H,d] (fp64).
    """
    assert S.dtype == np.float64 and S.flags.c_contiguous
    if z is not None:
        assert z.dtype == np.float64 and z.flags.c_contiguous
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, d = q.shape
    Hkv = k.shape[1]
    out = np.zeros((B, H, d), dtype=np.float64)
    _use(phi_map)
    try:
        rc = _load().linattn_ref_decode_step(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                             B, H, Hkv, d, int(bool(normalise)))
    finally:
        _use("elu1")
    if rc != 0:
        raise ValueError(f"linattn_ref_decode_step rejected its arguments (rc={rc})")
    return out


def ref_fwd_decay(q, k, v, g, normalise: bool = True, want_state: bool = False, nthreads: int | None = None,
                  state_in=None, z_in=None):
    """Causal forward pass with decayed sums.  g [B,Hkv,N] is the log-decay of
    every token: S_t = exp(g_t) S_{t-1} + phi(k_t) v_t^T (z likewise).  Other
    arguments and results as ref_fwd."""
    q, k, v, gg = _f64(q), _f64(k), _f64(v), _f64(g)
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    assert k.shape == (B, Hkv, N, d) and v.shape == (B, Hkv, N, d) and gg.shape == (B, Hkv, N)
    Si = None if state_in is None else _f64(state_in)
    zi = None if z_in is None else _f64(z_in)
    assert Si is None or Si.shape == (B, Hkv, d, d)
    assert zi is None or zi.shape == (B, Hkv, d)
    out = np.zeros((B, H, N, d), dtype=np.float64)
    S = np.zeros((B, Hkv, d, d), dtype=np.float64) if want_state else None
    z = np.zeros((B, Hkv, d), dtype=np.float64) if want_state else None
    rc = _load().linattn_ref_fwd_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(gg), _ptr(out), B, H, Hkv, N, d,
                                       int(bool(normalise)), _ptr(Si), _ptr(zi), _ptr(S), _ptr(z),
                                       nthreads or default_threads())
    if rc != 0:
        raise ValueError(f"linattn_ref_fwd_decay rejected its arguments (rc={rc})")
    return (out, S, z) if want_state else out


def ref_decode_step_decay(S: np.ndarray, z: np.ndarray | None, q, k, v, g, normalise: bool = True):
    """One decode step with decayed sums; g [B,Hkv] is the token's log-decay.
    S, z (fp64) are updated in place; returns out [B,H,d]."""
    assert S.dtype == np.float64 and S.flags.c_contiguous
    if z is not None:
        assert z.dtype == np.float64 and z.flags.c_contiguous
    q, k, v, gg = _f64(q), _f64(k), _f64(v), _f64(g)
    B, H, d = q.shape
    Hkv = k.shape[1]
    assert gg.shape == (B, Hkv)
    out = np.zeros((B, H, d), dtype=np.float64)
    rc = _load().linattn_ref_decode_step_decay(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(gg), _ptr(out),
                                               B, H, Hkv, d, int(bool(normalise)))
    if rc != 0:
        raise ValueError(f"linattn_ref_decode_step_decay rejected its arguments (rc={rc})")
    return out
