"""GPU parity with the other feature maps (ReLU, softplus in place of ELU + 1;
README "Features": custom kernel plugins): every entry point through the C ABI
against the oracle with the same map, at the ELU + 1 bars.  ReLU can zero a
normalised row's denominator, so its normalised cases use inputs shifted to be
positive (the same inputs on both sides)."""
import numpy as np
import pytest
import torch

import oracle
from linattn_inputs import DecodeStream, make_qkv, randn
from sequence_mixing_amd import ops

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}
TOL_BWD = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def rows_rel_err(got, ref, scale=0.0):
    """Worst row of max|got - ref| / max|ref|; a row whose exact value vanishes (its
    terms cancel, e.g. dq of a normalised sequence's first token) is measured
    against `scale`, the size of those terms."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    den = np.abs(r).max(axis=1)
    den = np.where(den <= 1e-9 * scale, scale, den)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(g - r).max(axis=1) / den).max())


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def qkv(B, H, Hkv, N, d, dtype, seed, m, normalise):
    q, k, v = make_qkv(B, H, Hkv, N, d, dtype, seed)
    if m == "relu" and normalise:
        q, k = (q.float().abs() + 0.05).to(TORCH[dtype]), (k.float().abs() + 0.05).to(TORCH[dtype])
    return q, k, v


@pytest.mark.parametrize("m", ["relu", "softplus"])
@pytest.mark.parametrize("B,H,Hkv,N,d,dtype", [(1, 2, 2, 300, 64, "f32"), (2, 4, 2, 1000, 64, "bf16"),
                                               (1, 8, 2, 700, 128, "bf16"), (1, 4, 4, 257, 32, "f16")])
@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_forward_feature_maps(m, B, H, Hkv, N, d, dtype, causal, normalise):
    print(f"phi={m} B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype} causal={causal} norm={normalise}", flush=True)
    q, k, v = qkv(B, H, Hkv, N, d, dtype, N + d, m, normalise)
    out, S, z = ops.fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, normalise=normalise, want_state=True, phi=m)
    torch.cuda.synchronize()
    ref, Sr, zr = oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise, want_state=True, phi_map=m)
    assert rows_rel_err(host(out), ref) <= TOL[dtype]
    assert rows_rel_err(host(S).reshape(-1, d * d), Sr.reshape(-1, d * d)) <= TOL[dtype]


@pytest.mark.parametrize("m", ["relu", "softplus"])
def test_decode_and_packed_feature_maps(m):
    B, H, Hkv, d = 3, 8, 2, 64
    st = DecodeStream(B, H, Hkv, d, "bf16", 9)
    q, k, v = st.next()
    if m == "relu":
        q, k = (q.float().abs() + 0.05).bfloat16(), (k.float().abs() + 0.05).bfloat16()
    S0 = torch.rand(B, Hkv, d, d, generator=torch.Generator().manual_seed(1))
    z0 = torch.rand(B, Hkv, d, generator=torch.Generator().manual_seed(2)) * 10 + 1
    S, z = S0.clone().cuda(), z0.clone().cuda()
    out = ops.decode_step(S, z, q.cuda(), k.cuda(), v.cuda(), phi=m)
    torch.cuda.synchronize()
    Sr, zr = S0.double().numpy(), z0.double().numpy()
    ref = oracle.ref_decode_step(Sr, zr, q, k, v, phi_map=m)
    assert rows_rel_err(host(out), ref) <= TOL["bf16"]
    assert rows_rel_err(host(S).reshape(-1, d), Sr.reshape(-1, d)) <= 1e-5
    # packed: two sequences
    lens = [100, 357]
    seqs = [qkv(1, 4, 2, n, 64, "bf16", 70 + i, m, True) for i, n in enumerate(lens)]
    qf, cu = ops.pack([s_[0][0] for s_ in seqs])
    kf, _ = ops.pack([s_[1][0] for s_ in seqs])
    vf, _ = ops.pack([s_[2][0] for s_ in seqs])
    o = ops.fwd_packed(qf.cuda(), kf.cuda(), vf.cuda(), cu.cuda(), 4, 2, 64, phi=m)
    torch.cuda.synchronize()
    for i, (qq, kk, vv) in enumerate(seqs):
        r = oracle.ref_fwd(qq, kk, vv, phi_map=m)
        got = ops.unpack(o.cpu(), cu, 4, 64)[i]
        assert rows_rel_err(got.double().numpy(), r[0]) <= TOL["bf16"]


@pytest.mark.parametrize("m", ["relu", "softplus"])
@pytest.mark.parametrize("B,H,Hkv,N,d,dtype", [(1, 2, 2, 300, 64, "f32"), (2, 4, 2, 257, 64, "bf16"),
                                               (1, 8, 2, 600, 128, "bf16")])
@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_backward_feature_maps(m, B, H, Hkv, N, d, dtype, causal, normalise):
    print(f"bwd phi={m} B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype} causal={causal} norm={normalise}", flush=True)
    q, k, v = qkv(B, H, Hkv, N, d, dtype, N + 2 * d, m, normalise)
    dout = randn((B, H, N, d), N + 1).to(TORCH[dtype])
    out = torch.from_numpy(oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise, phi_map=m)).to(TORCH[dtype])
    dq, dk, dv = ops.bwd(*(t.contiguous().cuda() for t in (q, k, v, out, dout)), causal=causal, normalise=normalise,
                         phi=m)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.ref_bwd(q, k, v, out, dout, causal=causal, normalise=normalise, phi_map=m)
    # rows whose exact gradient vanishes are measured against the size of their terms
    scale = float(dout.float().abs().max() * v.float().abs().max())
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = rows_rel_err(host(got), ref, scale)
        print(f"  {name} {e:.2e}", flush=True)
        assert e <= TOL_BWD[dtype], f"{name} {e:.3e}"
