"""GPU parity of the backward pass: linattn_bwd (through the C ABI) against the
fp64 oracle's backward, on the same inputs.

Both sides take the same q, k, v, dO and the same forward output `out`
(the oracle's forward, rounded to the input dtype), so the comparison is of
the gradient computation alone.  Metric: per output row (token, head) the
largest error over the largest reference value of that row, as for the
forward; dq, dk and dv are checked separately.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_mixing_amd as la
from linattn_inputs import WORKLOADS, make_qkv, randn
from sequence_mixing_amd import ops

pytestmark = pytest.mark.gpu

# fp32: fp32 products and sums, the forward's bar.  bf16: the MFMA operands
# (a, b, v, g, the masked scores, the carried S and R copies) are each rounded
# to bf16 (2^-9 relative), and dq, dk subtract the normaliser term from the
# value term, which amplifies those roundings by a small factor; measured
# worst rows stay under 2e-2, which is the bar (the forward's bf16 bar).
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}
TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def rows_rel_err(got, ref, scale):
    """Worst row of max|got - ref| / max|ref|.

    Rows whose exact gradient vanishes are measured against `scale`
    (max|dO| * max|v|, the size of the terms they are made of) instead: dq of
    the first token of a normalised causal sequence (o = v there, so the value
    and normaliser terms cancel exactly) and dq, dk of a lone token.  Their
    computed value is the rounding left from that cancellation."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    if g.size == 0:
        return 0.0
    den = np.abs(r).max(axis=1)
    den = np.where(den <= 1e-9 * scale, scale, den)
    return float((np.abs(g - r).max(axis=1) / den).max())


def term_scale(dout, v):
    return float(np.abs(np.asarray(dout, dtype=np.float64)).max() * np.abs(np.asarray(v, dtype=np.float64)).max())


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def case_inputs(B, H, Hkv, N, d, dtype, causal, normalise, seed):
    q, k, v = make_qkv(B, H, Hkv, N, d, dtype, seed)
    dout = randn((B, H, N, d), seed + 1).to(TORCH[dtype])
    out = torch.from_numpy(oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise)).to(TORCH[dtype])
    return q, k, v, out, dout


def run_case(B, H, Hkv, N, d, dtype, causal, normalise, seed=0):
    print(f"bwd B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype} causal={causal} norm={normalise} seed={seed}", flush=True)
    q, k, v, out, dout = case_inputs(B, H, Hkv, N, d, dtype, causal, normalise, seed)
    dq, dk, dv = ops.bwd(*(t.contiguous().cuda() for t in (q, k, v, out, dout)), causal=causal, normalise=normalise)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.ref_bwd(q, k, v, out, dout, causal=causal, normalise=normalise)
    tol = TOL[dtype]
    sc = term_scale(dout.float(), v.float())
    e = {"dq": rows_rel_err(host(dq), rq, sc), "dk": rows_rel_err(host(dk), rk, sc),
         "dv": rows_rel_err(host(dv), rv, sc)}
    print("  errors", {a: f"{b:.2e}" for a, b in e.items()}, flush=True)
    for name, err in e.items():
        assert err <= tol, f"{name} rel err {err:.3e} > {tol}"
    return e


SMALL = [
    # B, H, Hkv, N, d, dtype
    (1, 1, 1, 1, 32, "f32"),
    (1, 2, 2, 64, 32, "f32"),
    (1, 2, 2, 100, 64, "f32"),
    (2, 4, 2, 257, 64, "bf16"),
    (1, 4, 4, 1000, 32, "bf16"),
    (1, 4, 1, 333, 128, "bf16"),
    (1, 2, 2, 300, 128, "f32"),
    (3, 6, 3, 515, 64, "f32"),
    (1, 8, 2, 2049, 128, "bf16"),
    (2, 6, 2, 300, 64, "bf16"),
    (1, 8, 1, 500, 64, "f32"),
    (2, 2, 2, 7, 64, "bf16"),
    (2, 4, 2, 257, 64, "f16"),
    (1, 8, 2, 600, 128, "f16"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dK%dN%dd%d%s" % s)
@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_bwd_small_shapes(shape, causal, normalise):
    B, H, Hkv, N, d, dtype = shape
    run_case(B, H, Hkv, N, d, dtype, causal, normalise, seed=N + d)


@pytest.mark.parametrize("causal", [1, 0])
def test_bwd_config2_full(causal):
    w = WORKLOADS["cfg2"]
    run_case(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, causal, 1, seed=w.seed)


def test_bwd_config5_sampled():
    """GQA d = 128 bf16 at full length; the oracle runs on one (batch, kv head) group."""
    w = WORKLOADS["cfg5"]
    G = w.H // w.Hkv
    q, k, v = make_qkv(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, w.seed)
    dout = randn((w.B, w.H, w.N, w.d), w.seed + 1).to(torch.bfloat16)
    out = ops.fwd(q.cuda(), k.cuda(), v.cuda())          # the forward output the gradient is taken at
    print("bwd cfg5 full size", flush=True)
    dq, dk, dv = ops.bwd(q.cuda(), k.cuda(), v.cuda(), out, dout.cuda())
    torch.cuda.synchronize()
    for g in (0, w.Hkv - 1):
        hs = slice(g * G, (g + 1) * G)
        rq, rk, rv = oracle.ref_bwd(q[:, hs], k[:, g:g + 1], v[:, g:g + 1], out[:, hs].cpu(), dout[:, hs])
        sc = term_scale(dout[:, hs].float(), v[:, g:g + 1].float())
        for name, got, ref in (("dq", dq[:, hs], rq), ("dk", dk[:, g:g + 1], rk), ("dv", dv[:, g:g + 1], rv)):
            err = rows_rel_err(host(got), ref, sc)
            print(f"  group {g} {name} {err:.2e}", flush=True)
            assert err <= TOL["bf16"], f"group {g} {name} rel err {err:.3e}"


def test_bwd_directional_derivative_matches_forward_differences():
    """<dL/dq, dq_dir> equals the directional derivative of L = sum(dO * fwd) taken by
    central differences of the GPU forward itself (fp32, small step)."""
    B, H, Hkv, N, d = 1, 4, 2, 300, 64
    q, k, v = (t.cuda() for t in make_qkv(B, H, Hkv, N, d, "f32", 41))
    dout = randn((B, H, N, d), 42).cuda()
    out = ops.fwd(q, k, v)
    dq, dk, dv = ops.bwd(q, k, v, out, dout)
    gen = torch.Generator(device="cpu").manual_seed(43)
    dirs = [torch.randn(t.shape, generator=gen).cuda() for t in (q, k, v)]
    # fp32 outputs carry ~1e-6 relative rounding noise, so L does too: with a step of
    # 1e-2 that noise and the O(eps^2) truncation stay near 1e-3 of the derivative,
    # while a dropped term or a wrong sign would be off by O(1).
    eps = 1e-2
    fd = 0.0
    for i in range(3):
        args = [q, k, v]
        up = [a + eps * dirs[i] if j == i else a for j, a in enumerate(args)]
        dn = [a - eps * dirs[i] if j == i else a for j, a in enumerate(args)]
        lu = (ops.fwd(*(x.contiguous() for x in up)).double() * dout.double()).sum()
        ld = (ops.fwd(*(x.contiguous() for x in dn)).double() * dout.double()).sum()
        fd = float((lu - ld) / (2 * eps))
        an = float((dirs[i].double() * (dq, dk, dv)[i].double()).sum())
        assert abs(an - fd) <= 2e-2 * max(1.0, abs(fd)), (i, an, fd)


def test_bwd_deterministic_and_gqa_sum():
    B, H, Hkv, N, d = 1, 6, 2, 700, 64
    q, k, v, out, dout = (t.contiguous().cuda() for t in case_inputs(B, H, Hkv, N, d, "bf16", 1, 1, 5))
    a = ops.bwd(q, k, v, out, dout)
    b = ops.bwd(q, k, v, out, dout)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    G = H // Hkv
    kr, vr = k.repeat_interleave(G, 1).contiguous(), v.repeat_interleave(G, 1).contiguous()
    m = ops.bwd(q, kr, vr, out, dout)
    torch.cuda.synchronize()
    sc = term_scale(host(dout), host(v))
    assert rows_rel_err(host(a[0]), host(m[0]), sc) <= 2e-2
    assert rows_rel_err(host(a[1]), host(m[1].view(B, Hkv, G, N, d).float().sum(2)), sc) <= 2e-2
    assert rows_rel_err(host(a[2]), host(m[2].view(B, Hkv, G, N, d).float().sum(2)), sc) <= 2e-2


def test_bwd_argument_errors():
    q = torch.zeros(1, 2, 64, 64, device="cuda")
    k = torch.zeros(1, 2, 64, 64, device="cuda")
    f32 = la.LINATTN_F32
    ws_bytes = la.linattn_bwd_workspace_bytes(1, 2, 2, 64, 64, 1, f32)
    ws = torch.empty(ws_bytes // 4 + 1, device="cuda")
    g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)]
    call = lambda **kw: la.linattn_bwd(kw.get("q", q), k, k, kw.get("out", q), q, *g, 1, 2, 2, 64, 64, 1,
                                       kw.get("norm", 1), f32, kw.get("ws", ws), kw.get("wsb", ws_bytes))
    assert call() == 0
    assert call(out=None) == -1              # out is needed for the normalised gradient
    assert call(out=None, norm=0) == 0
    assert call(wsb=ws_bytes - 4) == -5
    assert call(ws=None) == -5
    torch.cuda.synchronize()
