"""fp8 rows (LinearTile 1.0.0 README, "Features": mixed precision; the OCP 8-bit
formats E4M3 and E5M2): q, k and v stored as fp8, widened exactly to the bf16
matrix-core operands at staging, outputs bf16.  The oracle reads the fp8 values
themselves (exactly, through fp64), so the bar is bf16's, 2e-2.

Checked through the C ABI: every one of the 256 codes of both formats decoded
exactly (a decode step from zero sums with zero q and k returns v itself);
forward (causal and not, both normalisers, GQA, d 32/64/128, ragged), the
bf16 B2 H8 N16384 d64 workload shape, continuation from given sums, packed
batches, the sliding window and decode steps; the entry points that do not
take fp8 refuse it."""
import numpy as np
import pytest
import torch

import oracle
import sequence_mixing_amd as la
from linattn_inputs import WORKLOADS, DecodeStream, make_qkv
from sequence_mixing_amd import ops

pytestmark = pytest.mark.gpu

FP8 = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}
TOL = 2e-2


def rows_rel_err(got, ref):
    g = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    if g.size == 0:
        return 0.0
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(g - r).max(axis=1) / den).max())


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def gpu(t):
    return t.contiguous().cuda()


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_every_code_decodes_exactly(fmt):
    dt = FP8[fmt]
    B, H, Hkv, d = 1, 2, 2, 128
    codes = torch.arange(256, dtype=torch.uint8).view(dt).reshape(B, Hkv, d)
    zq = torch.zeros(B, H, d).to(dt)
    zk = torch.zeros(B, Hkv, d).to(dt)
    S = torch.zeros(B, Hkv, d, d, device="cuda")
    z = torch.zeros(B, Hkv, d, device="cuda")
    o = ops.decode_step(S, z, gpu(zq), gpu(zk), gpu(codes))
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    want = codes.to(torch.float32)
    got = o.float().cpu()
    nan = torch.isnan(want)
    assert torch.equal(torch.isnan(got), nan)
    assert torch.equal(got[~nan], want[~nan]), "an fp8 code decoded wrongly"
    # the state holds phi(0) v = v exactly, z = phi(0) = 1
    assert torch.equal(torch.isnan(S[0, :, 0].cpu()), nan[0])


SMALL = [
    # B, H, Hkv, N, d
    (1, 2, 2, 300, 32),
    (2, 4, 2, 257, 64),
    (1, 4, 1, 333, 128),
    (2, 8, 8, 1000, 64),
    (1, 8, 2, 2049, 128),
    (2, 2, 2, 7, 64),
]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dK%dN%dd%d" % s)
@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_fp8_forward(fmt, shape, causal, normalise):
    B, H, Hkv, N, d = shape
    q, k, v = make_qkv(B, H, Hkv, N, d, fmt, N + d)
    print(f"fp8 {fmt} {shape} causal {causal} norm {normalise}", flush=True)
    out, S, z = ops.fwd(gpu(q), gpu(k), gpu(v), causal=causal, normalise=normalise, want_state=True)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    ref, Sr, zr = oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise, want_state=True)
    assert rows_rel_err(host(out), ref) <= TOL
    assert rows_rel_err(host(S).reshape(B * Hkv, -1), Sr.reshape(B * Hkv, -1)) <= TOL
    assert rows_rel_err(host(z), zr) <= TOL


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_workload_shape(fmt):
    w = WORKLOADS["cfg3"]
    q, k, v = make_qkv(w.B, w.H, w.Hkv, w.N, w.d, fmt, w.seed)
    print(f"fp8 {fmt} B2 H8 N16384 d64", flush=True)
    out = ops.fwd(gpu(q), gpu(k), gpu(v))
    torch.cuda.synchronize()
    ref = oracle.ref_fwd(q, k, v, causal=True, normalise=True)
    assert rows_rel_err(host(out), ref) <= TOL


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_continuation_and_window(fmt):
    B, H, Hkv, N, d = 2, 4, 2, 900, 64
    q, k, v = make_qkv(B, H, Hkv, N, d, fmt, 41)
    g = torch.Generator().manual_seed(42)
    S0 = (torch.randn(B, Hkv, d, d, generator=g) * 5).float()
    z0 = (torch.rand(B, Hkv, d, generator=g) * 20 + 1).float()
    out = ops.fwd(gpu(q), gpu(k), gpu(v), state_in=gpu(S0), z_in=gpu(z0))
    wout = ops.fwd_window(gpu(q), gpu(k), gpu(v), 100)
    torch.cuda.synchronize()
    ref = oracle.ref_fwd(q, k, v, causal=True, normalise=True, state_in=S0, z_in=z0)
    assert rows_rel_err(host(out), ref) <= TOL
    assert rows_rel_err(host(wout), oracle.ref_fwd_window(q, k, v, 100, True)) <= TOL


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_packed(fmt):
    H, Hkv, d = 4, 2, 64
    lens = [1, 300, 0, 1000, 77]
    seqs = [make_qkv(1, H, Hkv, n, d, fmt, 100 + i) for i, n in enumerate(lens)]
    qf, cu = ops.pack([gpu(s[0][0]) for s in seqs])
    kf, _ = ops.pack([gpu(s[1][0]) for s in seqs])
    vf, _ = ops.pack([gpu(s[2][0]) for s in seqs])
    out = ops.fwd_packed(qf, kf, vf, cu, H, Hkv, d)
    torch.cuda.synchronize()
    for (q, k, v), o in zip(seqs, ops.unpack(out, cu, H, d)):
        if q.shape[2] == 0:
            continue
        ref = oracle.ref_fwd(q, k, v, causal=True, normalise=True)[0]
        assert rows_rel_err(host(o), ref) <= TOL


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_decode_steps(fmt):
    B, H, Hkv, d = 3, 8, 2, 128
    q0, k0, v0 = make_qkv(B, Hkv, Hkv, 50, d, fmt, 7)
    _, S, z = ops.fwd(gpu(q0), gpu(k0), gpu(v0), want_state=True)
    Sr, zr = host(S).copy(), host(z).copy()
    stream = DecodeStream(B, H, Hkv, d, fmt, 8)
    for _ in range(4):
        q, k, v = stream.next()
        o = ops.decode_step(S, z, gpu(q), gpu(k), gpu(v))
        ref = oracle.ref_decode_step(Sr, zr, q, k, v, normalise=True)
        torch.cuda.synchronize()
        assert rows_rel_err(host(o), ref) <= TOL
        assert rows_rel_err(host(S).reshape(B * Hkv, -1), Sr.reshape(B * Hkv, -1)) <= 1e-5


def test_fp8_refused_where_not_taken():
    q = torch.zeros(1, 2, 64, 64, device="cuda").to(torch.float8_e4m3fn)
    o = torch.zeros(1, 2, 64, 64, device="cuda", dtype=torch.bfloat16)
    nb = la.linattn_bwd_workspace_bytes(1, 2, 2, 64, 64, 1, 3)
    assert nb == -1 or la.linattn_bwd(q, q, q, o, o, o, o, o, 1, 2, 2, 64, 64, 1, 1, 3, None, 0) == -4
    assert la.linattn_fwd_decay_workspace_bytes(1, 2, 2, 64, 64, 3, 0) == -1
