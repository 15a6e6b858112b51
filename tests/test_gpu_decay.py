"""GPU parity of the decayed sums (linattn_fwd_decay, linattn_decode_step_decay)
against the fp64 oracle's recurrence S_t = exp(g_t) S_{t-1} + phi(k_t) v_t^T.

Same bar as the plain forward pass (per-row max error over the row's max:
1e-4 for fp32, 2e-2 for bf16 and fp16).  Shapes cover several tiles, chunks
and segments with a ragged tail, both copy spacings of the chunk kernel (one
state copy per key tile, and per pair of tiles with the tile before the
diagonal read directly), GQA head blocks, continuation from given sums,
a strong decay, g = 0 (the plain method), decode, and the cfg3-shaped
decayed workload at full size.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_mixing_amd as la
from linattn_inputs import DECAY, make_decay, make_qkv
from sequence_mixing_amd import ops

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}


def gpu(t):
    return t.contiguous().cuda()


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rows_rel_err(got, ref):
    g = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(got)[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    if g.size == 0:
        return 0.0
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(g - r).max(axis=1) / den).max())


def mat_rel_err(got, ref):
    lead = np.shape(got)[:2]
    return rows_rel_err(np.reshape(got, (int(np.prod(lead)), -1)), np.reshape(ref, (int(np.prod(lead)), -1)))


def run_case(B, H, Hkv, N, d, dtype, normalise=True, chunk=0, seed=0, scale=1.0, start=False):
    print(f"decay case B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype} norm={normalise} chunk={chunk} seed={seed} "
          f"scale={scale} start={start}", flush=True)
    q, k, v = make_qkv(B, H, Hkv, N, d, dtype, seed)
    g = make_decay(B, Hkv, N, seed + 1) * scale
    Si = zi = None
    if start:
        Si = torch.rand(B, Hkv, d, d, generator=torch.Generator().manual_seed(seed + 2)) * 8.0
        zi = torch.rand(B, Hkv, d, generator=torch.Generator().manual_seed(seed + 3)) * 8.0
    out, S, z = ops.fwd_decay(gpu(q), gpu(k), gpu(v), gpu(g), normalise=normalise, chunk=chunk, want_state=True,
                              state_in=None if Si is None else gpu(Si), z_in=None if zi is None else gpu(zi))
    torch.cuda.synchronize()
    ref, Sr, zr = oracle.ref_fwd_decay(q, k, v, g, normalise=normalise, want_state=True, state_in=Si, z_in=zi)
    tol = TOL[dtype]
    e = rows_rel_err(host(out), ref)
    assert e <= tol, f"output rel err {e:.3e} > {tol}"
    if N > 0:
        es, ez = mat_rel_err(host(S), Sr), mat_rel_err(host(z), zr)
        assert es <= tol and ez <= tol, f"state rel err {es:.3e}, z rel err {ez:.3e}"
    return e


SMALL = [
    # B, H, Hkv, N, d, dtype
    (1, 2, 2, 300, 32, "f32"),
    (1, 2, 2, 300, 64, "f32"),
    (2, 4, 2, 257, 64, "bf16"),
    (1, 4, 4, 1000, 64, "bf16"),
    (1, 2, 2, 777, 64, "f16"),
    (1, 8, 2, 700, 128, "bf16"),   # GQA, head blocks of 4
    (2, 6, 2, 300, 64, "bf16"),    # G = 3
    (1, 2, 2, 450, 128, "f32"),
    (1, 1, 1, 1, 64, "f32"),
    (3, 2, 1, 33, 32, "bf16"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dK%dN%dd%d%s" % s)
@pytest.mark.parametrize("normalise", [1, 0])
def test_small_shapes(shape, normalise):
    B, H, Hkv, N, d, dtype = shape
    run_case(B, H, Hkv, N, d, dtype, normalise, seed=N + d)


@pytest.mark.parametrize("chunk", [32, 64, 128, 256])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_chunk_size(chunk, dtype):
    """Chunk 128 (bf16 d = 64) and 256 keep one state copy per pair of key tiles: the
    tile before the diagonal is read directly and faded per key."""
    code = ops.dtype_code({"f32": torch.float32, "bf16": torch.bfloat16}[dtype])
    if la.linattn_fwd_decay_workspace_bytes(2, 4, 2, 1100, 64, code, chunk) < 0:
        pytest.skip("chunk not available with decayed sums for this dtype")
    run_case(2, 4, 2, 1100, 64, dtype, 1, chunk=chunk, seed=chunk)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strong_decay(dtype):
    """g = logsigmoid(u): factors down to about exp(-3) per token."""
    run_case(1, 4, 2, 900, 64, dtype, 1, seed=5, scale=16.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_continuation_from_given_sums(dtype):
    run_case(2, 4, 2, 600, 64, dtype, 1, seed=9, start=True)


def test_zero_decay_matches_the_plain_forward():
    q, k, v = make_qkv(2, 4, 2, 999, 64, "f32", 13)
    g = torch.zeros(2, 2, 999)
    a, Sa, za = ops.fwd(gpu(q), gpu(k), gpu(v), want_state=True)
    b, Sb, zb = ops.fwd_decay(gpu(q), gpu(k), gpu(v), gpu(g), want_state=True)
    torch.cuda.synchronize()
    assert rows_rel_err(host(b), host(a)) <= 1e-5
    assert mat_rel_err(host(Sb), host(Sa)) <= 1e-6 and mat_rel_err(host(zb), host(za)) <= 1e-6


@pytest.mark.parametrize("reset", [-1e4, -float("inf")])
def test_reset_token_forgets_the_past(reset):
    """A reset at token r (the GPU takes log-decays below -20 as -20, a factor of 2e-9):
    rows from r on equal a fresh pass over tokens r.., and all rows match the oracle,
    which takes g as given."""
    q, k, v = make_qkv(1, 2, 2, 500, 64, "f32", 17)
    g = make_decay(1, 2, 500, 18)
    r = 211
    g[:, :, r] = reset
    out = ops.fwd_decay(gpu(q), gpu(k), gpu(v), gpu(g))
    tail = ops.fwd_decay(gpu(q[:, :, r:]), gpu(k[:, :, r:]), gpu(v[:, :, r:]), gpu(g[:, :, r:]))
    torch.cuda.synchronize()
    assert rows_rel_err(host(out)[:, :, r:], host(tail)) <= 1e-5
    assert rows_rel_err(host(out), oracle.ref_fwd_decay(q, k, v, g)) <= TOL["f32"]


def test_decayed_workload_full_size():
    w = DECAY
    q, k, v = make_qkv(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, w.seed)
    g = make_decay(w.B, w.Hkv, w.N, w.seed + 1)
    print(f"decay workload {w.name}", flush=True)
    out, S, z = ops.fwd_decay(gpu(q), gpu(k), gpu(v), gpu(g), want_state=True)
    torch.cuda.synchronize()
    ref, Sr, zr = oracle.ref_fwd_decay(q, k, v, g, want_state=True)
    assert rows_rel_err(host(out), ref) <= TOL[w.dtype]
    assert mat_rel_err(host(S), Sr) <= TOL[w.dtype] and mat_rel_err(host(z), zr) <= TOL[w.dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_steps_against_the_oracle(dtype):
    """Decode with decay from a decayed prefill's sums, 64 steps, GQA d = 128."""
    B, H, Hkv, N, d = 2, 8, 2, 300, 128
    q, k, v = make_qkv(B, H, Hkv, N, d, dtype, 21)
    g = make_decay(B, Hkv, N, 22)
    _, S, z = ops.fwd_decay(gpu(q), gpu(k), gpu(v), gpu(g), want_state=True)
    torch.cuda.synchronize()
    _, Sr, zr = oracle.ref_fwd_decay(q, k, v, g, want_state=True)
    gen = torch.Generator().manual_seed(23)
    worst = 0.0
    for step in range(64):
        qs, ks, vs = (torch.randn(B, h, d, generator=gen).to(q.dtype) for h in (H, Hkv, Hkv))
        gs = torch.nn.functional.logsigmoid(torch.randn(B, Hkv, generator=gen)) / 16.0
        o = ops.decode_step_decay(S, z, gpu(qs), gpu(ks), gpu(vs), gpu(gs))
        ref = oracle.ref_decode_step_decay(Sr, zr, qs, ks, vs, gs)
        torch.cuda.synchronize()
        e = rows_rel_err(host(o), ref)
        worst = max(worst, e)
        assert e <= TOL[dtype], f"step {step}: {e:.3e}"
    assert mat_rel_err(host(S), Sr) <= TOL[dtype]
    print(f"decay decode worst rel err {worst:.3e}", flush=True)


def test_decode_zero_decay_equals_plain_decode():
    B, H, Hkv, d = 3, 4, 2, 64
    gen = torch.Generator().manual_seed(31)
    S0 = torch.rand(B, Hkv, d, d, generator=gen).cuda()
    z0 = torch.rand(B, Hkv, d, generator=gen).cuda() + 1.0
    q, k, v = (torch.randn(B, h, d, generator=gen).cuda() for h in (H, Hkv, Hkv))
    S1, z1, S2, z2 = S0.clone(), z0.clone(), S0.clone(), z0.clone()
    a = ops.decode_step(S1, z1, q, k, v)
    b = ops.decode_step_decay(S2, z2, q, k, v, torch.zeros(B, Hkv, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(S1, S2) and torch.equal(z1, z2)


def test_rejections():
    q = torch.zeros(1, 2, 64, 64, device="cuda")
    g = torch.zeros(1, 2, 64, device="cuda")
    with pytest.raises(la.LinattnError):
        ops.fwd_decay(q, q.clone(), q.clone(), g, chunk=128)  # fp32 d = 64 chunk 128: shifted copies
    code = ops.dtype_code(torch.float32, "relu")
    assert la.linattn_fwd_decay(q, q, q, g, q.clone(), 1, 2, 2, 64, 64, 1, code) == -4
    assert la.linattn_fwd_decay(q, q, q, None, q.clone(), 1, 2, 2, 64, 64, 1, 0) == -1
