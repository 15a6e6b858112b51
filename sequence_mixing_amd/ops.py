"""Torch-facing wrappers over the C ABI: allocate outputs / workspace, check status.

Allocation and stream plumbing only; the computation is the library's.
"""
from __future__ import annotations

import torch

from . import (LINATTN_BF16, LINATTN_F16, LINATTN_F32, LinattnError, linattn_bwd, linattn_bwd_workspace_bytes,
               linattn_fwd_plan, linattn_fwd_window,
               linattn_decode_step, linattn_decode_step_decay, linattn_fwd, linattn_fwd_decay,
               linattn_fwd_decay_workspace_bytes, linattn_fwd_from_state, linattn_fwd_packed,
               linattn_fwd_packed_workspace_bytes, linattn_fwd_workspace_bytes)

_DT = {torch.float32: LINATTN_F32, torch.bfloat16: LINATTN_BF16, torch.float16: LINATTN_F16,
       torch.float8_e4m3fn: 3, torch.float8_e5m2: 4}
_FP8 = (torch.float8_e4m3fn, torch.float8_e5m2)


def out_dtype(t: torch.dtype) -> torch.dtype:
    """Element type of the outputs for inputs of type t: the same, except bf16 for fp8 rows."""
    return torch.bfloat16 if t in _FP8 else t


def _empty_out(q):
    return torch.empty(q.shape, dtype=out_dtype(q.dtype), device=q.device)


# feature maps (the `dtype` code's bits 8-15)
PHI = {"elu1": 0, "relu": 1, "softplus": 2}


def dtype_code(t: torch.dtype, phi: str = "elu1") -> int:
    """The C ABI's dtype argument: element type, and the feature map in bits 8-15."""
    if t not in _DT:
        raise TypeError(f"unsupported dtype {t}")
    if phi not in PHI:
        raise ValueError(f"unknown feature map {phi}")
    return _DT[t] | (PHI[phi] << 8)


def workspace(B, H, Hkv, N, d, causal, dtype: torch.dtype, chunk=0, device="cuda") -> torch.Tensor | None:
    n = linattn_fwd_workspace_bytes(B, H, Hkv, N, d, causal, dtype_code(dtype), chunk)
    if n < 0:
        # the plan call reports why the arguments were rejected
        rc, _, _ = linattn_fwd_plan(B, H, Hkv, N, d, causal, dtype_code(dtype), chunk)
        raise LinattnError(rc if rc != 0 else -2, "linattn_fwd_workspace_bytes")
    return torch.empty((n + 3) // 4, dtype=torch.float32, device=device) if n > 0 else None


def _nbytes(ws) -> int:
    """Bytes of a caller's workspace tensor (any dtype), 0 for None."""
    return ws.numel() * ws.element_size() if ws is not None else 0


def _check_decode(state, z, q, k, v, normalise):
    """Shapes, dtypes, contiguity and device of a decode step's tensors: the kernel writes
    B*Hkv*d*d fp32 state values in place, so a wrong buffer must be refused here."""
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [B, H, d] and k, v [B, Hkv, d]")
    B, H, d = q.shape
    Hkv = k.shape[1]
    for t in (q, k, v):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == q.dtype and t.device == q.device):
            raise ValueError("q, k, v must be contiguous device tensors of one dtype on one device")
    if k.shape != (B, Hkv, d) or v.shape != (B, Hkv, d):
        raise ValueError("k and v must be [B, Hkv, d]")
    if not (state.is_cuda and state.is_contiguous() and state.dtype == torch.float32 and
            state.shape == (B, Hkv, d, d) and state.device == q.device):
        raise ValueError("state must be a contiguous fp32 device tensor [B, Hkv, d, d] on q's device")
    if z is None:
        if normalise:
            raise ValueError("z is required when normalise is set")
    elif not (z.is_cuda and z.is_contiguous() and z.dtype == torch.float32 and z.shape == (B, Hkv, d) and
              z.device == q.device):
        raise ValueError("z must be a contiguous fp32 device tensor [B, Hkv, d] on q's device")
    return B, H, Hkv, d


def _check_out(out, q):
    if out is None:
        return _empty_out(q)
    if not (out.is_cuda and out.is_contiguous() and out.dtype == out_dtype(q.dtype) and out.shape == q.shape and
            out.device == q.device):
        raise ValueError("out must be a contiguous device tensor of q's shape and device, of q's dtype "
                         "(bf16 for fp8 q)")
    return out


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal=True, normalise=True, chunk=0,
        want_state=False, out=None, ws=None, stream=None, state_in=None, z_in=None, phi="elu1"):
    """O = phi(Q)(phi(K)^T V) through ``linattn_fwd`` (``linattn_fwd_from_state`` when
    ``state_in`` is given); q [B,H,N,d], k/v [B,Hkv,N,d] on the GPU."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    for t in (q, k, v):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == q.dtype):
            raise ValueError("q, k, v must be contiguous device tensors of one dtype")
    if k.shape != (B, Hkv, N, d) or v.shape != (B, Hkv, N, d):
        raise ValueError("k and v must be [B, Hkv, N, d]")
    code = dtype_code(q.dtype, phi)
    out = _check_out(out, q)
    S = z = None
    if want_state:
        S = torch.empty(B, Hkv, d, d, dtype=torch.float32, device=q.device)
        z = torch.empty(B, Hkv, d, dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(B, H, Hkv, N, d, causal, q.dtype, chunk, q.device)
    nbytes = _nbytes(ws)
    if state_in is not None:
        starts = ((state_in, (B, Hkv, d, d)),) + (((z_in, (B, Hkv, d)),) if z_in is not None else ())
        for t, shape in starts:
            if not (t.is_cuda and t.is_contiguous() and t.dtype == torch.float32 and t.shape == shape):
                raise ValueError("state_in / z_in must be contiguous fp32 device tensors [B,Hkv,d,d] / [B,Hkv,d]")
        rc = linattn_fwd_from_state(q, k, v, out, B, H, Hkv, N, d, causal, normalise, code, state_in, z_in, S, z,
                                    chunk, ws, nbytes, stream)
        if rc != 0:
            raise LinattnError(rc, "linattn_fwd_from_state")
        return (out, S, z) if want_state else out
    rc = linattn_fwd(q, k, v, out, B, H, Hkv, N, d, causal, normalise, code, S, z, chunk, ws, nbytes, stream)
    if rc != 0:
        raise LinattnError(rc, "linattn_fwd")
    return (out, S, z) if want_state else out


def fwd_window(q, k, v, window, normalise=True, out=None, stream=None, phi="elu1"):
    """Sliding-window causal pass through ``linattn_fwd_window``: query t sees keys
    t - window < s <= t; q [B,H,N,d], k/v [B,Hkv,N,d] on the GPU."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    for t in (q, k, v):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == q.dtype and t.device == q.device):
            raise ValueError("q, k, v must be contiguous device tensors of one dtype on one device")
    if k.shape != (B, Hkv, N, d) or v.shape != (B, Hkv, N, d):
        raise ValueError("k and v must be [B, Hkv, N, d]")
    out = _check_out(out, q)
    rc = linattn_fwd_window(q, k, v, out, B, H, Hkv, N, d, window, normalise, dtype_code(q.dtype, phi), stream)
    if rc != 0:
        raise LinattnError(rc, "linattn_fwd_window")
    return out


def fwd_decay(q, k, v, g, normalise=True, chunk=0, want_state=False, out=None, ws=None, stream=None, state_in=None,
              z_in=None):
    """Causal forward pass with decayed sums through ``linattn_fwd_decay``: g [B,Hkv,N] fp32
    is every token's log-decay (S_t = exp(g_t) S_{t-1} + phi(k_t) v_t^T, z likewise)."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    for t in (q, k, v):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == q.dtype):
            raise ValueError("q, k, v must be contiguous device tensors of one dtype")
    if k.shape != (B, Hkv, N, d) or v.shape != (B, Hkv, N, d):
        raise ValueError("k and v must be [B, Hkv, N, d]")
    if not (g.is_cuda and g.is_contiguous() and g.dtype == torch.float32 and g.shape == (B, Hkv, N)):
        raise ValueError("g must be a contiguous fp32 device tensor [B, Hkv, N]")
    for t, shape in ((state_in, (B, Hkv, d, d)), (z_in, (B, Hkv, d))):
        if t is not None and not (t.is_cuda and t.is_contiguous() and t.dtype == torch.float32 and t.shape == shape):
            raise ValueError("state_in / z_in must be contiguous fp32 device tensors [B,Hkv,d,d] / [B,Hkv,d]")
    code = dtype_code(q.dtype)
    out = _check_out(out, q)
    S = z = None
    if want_state:
        S = torch.empty(B, Hkv, d, d, dtype=torch.float32, device=q.device)
        z = torch.empty(B, Hkv, d, dtype=torch.float32, device=q.device)
    if ws is None:
        n = linattn_fwd_decay_workspace_bytes(B, H, Hkv, N, d, code, chunk)
        if n < 0:
            raise LinattnError(-4, "linattn_fwd_decay_workspace_bytes")
        ws = torch.empty((n + 3) // 4, dtype=torch.float32, device=q.device) if n > 0 else None
    nbytes = _nbytes(ws)
    rc = linattn_fwd_decay(q, k, v, g, out, B, H, Hkv, N, d, normalise, code, state_in, z_in, S, z, chunk, ws, nbytes,
                           stream)
    if rc != 0:
        raise LinattnError(rc, "linattn_fwd_decay")
    return (out, S, z) if want_state else out


def pack(seqs):
    """Concatenates per-sequence tensors [heads, n_b, d] (one dtype and device) into the
    packed layout: a flat tensor holding each sequence's head-major block in turn, and
    cu_seqlens (int32, nseqs + 1 token offsets) on the same device."""
    cu = [0]
    for x in seqs:
        cu.append(cu[-1] + x.shape[1])
    flat = torch.cat([x.contiguous().reshape(-1) for x in seqs]) if seqs else torch.empty(0)
    return flat, torch.tensor(cu, dtype=torch.int32, device=flat.device)


def unpack(flat, cu, heads, d):
    """Inverse of pack: the list of [heads, n_b, d] views of a packed tensor."""
    cu = [int(x) for x in cu]
    return [flat[heads * a * d: heads * b * d].view(heads, b - a, d) for a, b in zip(cu[:-1], cu[1:])]


def fwd_packed(q, k, v, cu_seqlens, H, Hkv, d, causal=True, normalise=True, chunk=0, want_state=False, out=None,
               ws=None, stream=None, phi="elu1"):
    """linattn_fwd_packed on packed tensors (see pack): q of H * total * d elements, k and v
    of Hkv * total * d; cu_seqlens an int32 device tensor of nseqs + 1 offsets."""
    nseqs = cu_seqlens.numel() - 1
    total = q.numel() // (H * d)
    for t in (q, k, v):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == q.dtype):
            raise ValueError("q, k, v must be contiguous device tensors of one dtype")
    if q.numel() != H * total * d or k.numel() != Hkv * total * d or v.numel() != k.numel():
        raise ValueError("q must hold H * total * d elements and k, v Hkv * total * d")
    if not (cu_seqlens.is_cuda and cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous()):
        raise ValueError("cu_seqlens must be a contiguous int32 device tensor")
    code = dtype_code(q.dtype, phi)
    out = _check_out(out, q)
    S = z = None
    if want_state:
        S = torch.empty(nseqs, Hkv, d, d, dtype=torch.float32, device=q.device)
        z = torch.empty(nseqs, Hkv, d, dtype=torch.float32, device=q.device)
    nbytes = linattn_fwd_packed_workspace_bytes(nseqs, H, Hkv, total, d, causal, code, chunk)
    if nbytes < 0:
        raise LinattnError(-2, "linattn_fwd_packed_workspace_bytes")
    if ws is None:
        ws = torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.float32, device=q.device)
    rc = linattn_fwd_packed(q, k, v, out, cu_seqlens, nseqs, total, H, Hkv, d, causal, normalise, code, S, z, chunk,
                            ws, _nbytes(ws), stream)
    if rc != 0:
        raise LinattnError(rc, "linattn_fwd_packed")
    return (out, S, z) if want_state else out


def bwd(q, k, v, out, dout, causal=True, normalise=True, ws=None, stream=None, grads=None, phi="elu1"):
    """dQ, dK, dV through ``linattn_bwd``; q/out/dout [B,H,N,d], k/v [B,Hkv,N,d] on the GPU."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    for t in (q, k, v, dout) + ((out,) if normalise else ()):
        if not (t.is_cuda and t.is_contiguous() and t.dtype == q.dtype):
            raise ValueError("q, k, v, out, dout must be contiguous device tensors of one dtype")
    if k.shape != (B, Hkv, N, d) or v.shape != (B, Hkv, N, d) or dout.shape != q.shape:
        raise ValueError("k, v must be [B, Hkv, N, d] and dout [B, H, N, d]")
    code = dtype_code(q.dtype, phi)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    nbytes = linattn_bwd_workspace_bytes(B, H, Hkv, N, d, causal, code)
    if nbytes < 0:
        raise LinattnError(-2, "linattn_bwd_workspace_bytes")
    if ws is None:
        ws = torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.float32, device=q.device)
    rc = linattn_bwd(q, k, v, out if normalise else None, dout, dq, dk, dv, B, H, Hkv, N, d, causal, normalise, code,
                     ws, _nbytes(ws), stream)
    if rc != 0:
        raise LinattnError(rc, "linattn_bwd")
    return dq, dk, dv


def decode_step(state: torch.Tensor, z: torch.Tensor | None, q, k, v, normalise=True, out=None, stream=None,
                phi="elu1"):
    """One recurrent step through ``linattn_decode_step``; state [B,Hkv,d,d] and z [B,Hkv,d] fp32, in place."""
    B, H, Hkv, d = _check_decode(state, z, q, k, v, normalise)
    out = _check_out(out, q)
    rc = linattn_decode_step(state, z, q, k, v, out, B, H, Hkv, d, normalise, dtype_code(q.dtype, phi), stream)
    if rc != 0:
        raise LinattnError(rc, "linattn_decode_step")
    return out


def decode_step_decay(state: torch.Tensor, z: torch.Tensor | None, q, k, v, g, normalise=True, out=None,
                      stream=None):
    """One step through ``linattn_decode_step_decay``: S and z fade by exp(g) [B,Hkv] (fp32,
    device), then absorb (k, v) and are read by q; state and z are updated in place."""
    B, H, Hkv, d = _check_decode(state, z, q, k, v, normalise)
    if not (g.is_cuda and g.is_contiguous() and g.dtype == torch.float32 and g.shape == (B, Hkv)):
        raise ValueError("g must be a contiguous fp32 device tensor [B, Hkv]")
    out = _check_out(out, q)
    rc = linattn_decode_step_decay(state, z, q, k, v, g, out, B, H, Hkv, d, normalise, dtype_code(q.dtype), stream)
    if rc != 0:
        raise LinattnError(rc, "linattn_decode_step_decay")
    return out
