"""GPU parity for the staging-wave forms of the causal chunk kernel, against the fp64 oracle.

Those forms (fp32 rows at d = 64 with chunk 32 or 64 and at most two heads per
block; 16-bit rows at d = 128 with at most four query units per chunk) give the
phase-2 work to half of the waves and let the other half stage the next chunks:
fp32 one chunk ahead, 16-bit rows two chunks ahead in two register sets walked
in pairs.  The shapes below are chosen so that the plan cuts each sequence into
segments of one, two, three and five chunks (an odd count ends the paired walk
on a single step), with ragged tails, query-head groups of one, two and four,
fp16 rows, continuation from given sums and the final sums checked.  Same bar
as the other parity tests: per-row relative error <= 1e-4 (fp32), <= 2e-2
(16-bit rows).
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_mixing_amd as la
from linattn_inputs import make_qkv
from sequence_mixing_amd import ops

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}


def rel_err(got, ref):
    g = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(got)[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(g - r).max(axis=1) / den).max())


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


CASES = [
    # B, H, Hkv, N, d, dtype, chunk
    (1, 1, 1, 200, 64, "f32", 64),      # one sequence: a segment per chunk, ragged last chunk
    (8, 8, 8, 512, 64, "f32", 64),      # 64 sequences: segments of two chunks
    (8, 8, 8, 760, 64, "f32", 64),      # segments of three chunks, ragged tail
    (8, 8, 8, 700, 64, "f32", 32),      # chunk 32 (one key tile per chunk)
    (4, 8, 4, 650, 64, "f32", 32),      # two query heads per block
    (1, 4, 1, 70, 128, "bf16", 0),      # one chunk per segment
    (8, 16, 4, 1270, 128, "bf16", 0),   # 32 sequences: segments of five chunks, ragged tail
    (8, 16, 4, 1270, 128, "f16", 0),
    (4, 8, 4, 1500, 128, "bf16", 32),   # two query heads per kv head: segments of three chunks
    (4, 4, 4, 2000, 128, "bf16", 32),   # one query head: its output columns in four parts, four chunks per segment
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dH%dK%dN%dd%d%s_c%d" % c)
@pytest.mark.parametrize("normalise", [1, 0])
@pytest.mark.parametrize("cont", [0, 1])
def test_staging_forms(case, normalise, cont):
    B, H, Hkv, N, d, dtype, chunk = case
    q, k, v = make_qkv(B, H, Hkv, N, d, dtype, 31 + N + d)
    rc, c, P = la.linattn_fwd_plan(B, H, Hkv, N, d, 1, ops.dtype_code(q.dtype), chunk)
    assert rc == 0
    nchunks = (N + c - 1) // c
    print(f"staging B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype} chunk={c} segments={P} "
          f"chunks/segment={-(-nchunks // P)} normalise={normalise} continuation={cont}", flush=True)
    S0 = z0 = None
    if cont:
        # start sums of a seeded 200-token prefix, rounded to fp32 for both sides
        _, kp, vp = make_qkv(B, Hkv, Hkv, 200, d, dtype, 7 + d)
        _, Sp, zp = oracle.ref_fwd(kp, kp, vp, causal=True, want_state=True)
        S0, z0 = torch.from_numpy(Sp).float(), torch.from_numpy(zp).float()
    out, S, z = ops.fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, normalise=normalise, chunk=chunk,
                        want_state=True, state_in=S0.cuda() if cont else None,
                        z_in=z0.cuda() if cont and normalise else None)
    torch.cuda.synchronize()
    ref, Sr, zr = oracle.ref_fwd(q, k, v, causal=True, normalise=normalise, want_state=True,
                                 state_in=S0 if cont else None, z_in=z0 if cont and normalise else None)
    tol = TOL[dtype]
    e = rel_err(host(out), ref)
    assert e <= tol, f"output rel err {e:.3e} > {tol}"
    es = rel_err(host(S).reshape(B * Hkv, -1), Sr.reshape(B * Hkv, -1))
    assert es <= tol, f"state rel err {es:.3e} > {tol}"
    ez = rel_err(host(z), zr)
    assert ez <= tol, f"z rel err {ez:.3e} > {tol}"


def test_staging_forms_bitwise_repeatable():
    # the same call twice gives the same bits (no atomics, fixed plan)
    q, k, v = (t.cuda() for t in make_qkv(8, 16, 4, 1270, 128, "bf16", 5))
    a = ops.fwd(q, k, v)
    b = ops.fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
