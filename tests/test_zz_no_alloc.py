"""linattn_fwd_noalloc (the library's static device scratch, no workspace
argument) against linattn_fwd with a caller workspace, through the C ABI.

Two calls in a row on one stream, the second with a smaller input, so the
second reuses a scratch that still holds the first call's contents; both must
equal linattn_fwd's results (bitwise: the same kernels and plan) and the fp64
oracle within the forward's bar.  A call that needs more scratch than the
library holds is refused before any launch.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_mixing_amd as la
from linattn_inputs import make_qkv
from sequence_mixing_amd import ops

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rows_rel_err(got, ref):
    g = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(g - r).max(axis=1) / den).max())


def run_both(B, H, Hkv, N, d, dtype, causal, normalise, seed):
    print(f"noalloc B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype} causal={causal} norm={normalise}", flush=True)
    q, k, v = make_qkv(B, H, Hkv, N, d, dtype, seed)
    qg, kg, vg = (t.contiguous().cuda() for t in (q, k, v))
    code = ops.dtype_code(qg.dtype)
    out_a, out_b = torch.empty_like(qg), torch.empty_like(qg)
    S_a = torch.empty(B, Hkv, d, d, device="cuda")
    z_a = torch.empty(B, Hkv, d, device="cuda")
    S_b, z_b = torch.empty_like(S_a), torch.empty_like(z_a)
    ws = ops.workspace(B, H, Hkv, N, d, causal, qg.dtype)
    nbytes = ws.numel() * 4 if ws is not None else 0
    assert la.linattn_fwd(qg, kg, vg, out_a, B, H, Hkv, N, d, causal, normalise, code, S_a, z_a, 0, ws, nbytes) == 0
    assert la.linattn_fwd_noalloc(qg, kg, vg, out_b, B, H, Hkv, N, d, causal, normalise, code, S_b, z_b) == 0
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(S_a, S_b) and torch.equal(z_a, z_b)
    ref = oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise)
    e = rows_rel_err(out_b.double().cpu().numpy(), ref)
    assert e <= TOL[dtype], f"rel err {e:.3e}"
    return e


def test_noalloc_two_calls_second_smaller():
    # fp32 B2 H8 N4096 d64 (the headline shape), then a smaller GQA bf16 call
    run_both(2, 8, 8, 4096, 64, "f32", 1, 1, 1002)
    run_both(1, 4, 2, 777, 128, "bf16", 1, 1, 77)


def test_noalloc_noncausal_then_causal():
    run_both(2, 8, 8, 2048, 64, "bf16", 0, 0, 5)
    run_both(1, 2, 2, 300, 32, "f32", 1, 0, 6)


def test_noalloc_refuses_beyond_scratch():
    # non-causal d = 128 with 1024 sequences: one partial state per sequence,
    # 1024 * 128 * 129 * 4 bytes > 64 MiB; refused before any launch
    B, H, Hkv, N, d = 1024, 1, 1, 4, 128
    need = la.linattn_fwd_workspace_bytes(B, H, Hkv, N, d, 0, la.LINATTN_F32)
    assert need > la.LINATTN_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, H, N, d, device="cuda")
    out = torch.full_like(q, 7.0)
    rc = la.linattn_fwd_noalloc(q, q, q, out, B, H, Hkv, N, d, 0, 1, la.LINATTN_F32)
    assert rc == -8
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
