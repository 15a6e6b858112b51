"""GPU parity of packed batches (sequences of different lengths, no padding):
linattn_fwd_packed through the C ABI against the fp64 oracle run on every
sequence on its own, at the forward's bar (worst row 1e-4 fp32, 2e-2 bf16).

Length mixes are seeded: empty sequences, single tokens, lengths that are
not multiples of the chunk or the segment, and many short sequences."""
import numpy as np
import pytest
import torch

import oracle
import sequence_mixing_amd as la
from linattn_inputs import make_qkv
from sequence_mixing_amd import ops

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}


def rows_rel_err(got, ref):
    g = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    if g.size == 0:
        return 0.0
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(g - r).max(axis=1) / den).max())


def lengths_mix(nseqs, lo, hi, seed, extra=()):
    rng = np.random.default_rng(seed)
    return list(extra) + [int(x) for x in rng.integers(lo, hi + 1, nseqs - len(extra))]


def run_packed(lens, H, Hkv, d, dtype, causal, normalise, chunk=0, seed=0):
    print(f"packed n={len(lens)} total={sum(lens)} lens[:8]={lens[:8]} H{H} Hkv{Hkv} d{d} {dtype} "
          f"causal={causal} norm={normalise} chunk={chunk}", flush=True)
    seqs = [make_qkv(1, H, Hkv, n, d, dtype, seed + 17 * i) for i, n in enumerate(lens)]
    qf, cu = ops.pack([s[0][0] for s in seqs])
    kf, _ = ops.pack([s[1][0] for s in seqs])
    vf, _ = ops.pack([s[2][0] for s in seqs])
    out, S, z = ops.fwd_packed(qf.cuda(), kf.cuda(), vf.cuda(), cu.cuda(), H, Hkv, d, causal=causal,
                               normalise=normalise, chunk=chunk, want_state=True)
    torch.cuda.synchronize()
    outs = ops.unpack(out.cpu(), cu, H, d)
    tol = TOL[dtype]
    worst = 0.0
    for i, (q, k, v) in enumerate(seqs):
        ref, Sr, zr = oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise, want_state=True)
        e = rows_rel_err(outs[i].double().numpy(), ref[0])
        worst = max(worst, e)
        assert e <= tol, f"sequence {i} (n={lens[i]}): output rel err {e:.3e}"
        Sg, zg = S[i].double().cpu().numpy(), z[i].double().cpu().numpy()
        if lens[i] == 0:
            assert not Sg.any() and not zg.any()
        else:
            es = rows_rel_err(Sg.reshape(Hkv, -1), Sr[0].reshape(Hkv, -1))
            ez = rows_rel_err(zg, zr[0])
            assert es <= tol and ez <= tol, f"sequence {i}: state {es:.3e} z {ez:.3e}"
    print(f"  worst row {worst:.2e}", flush=True)


@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
@pytest.mark.parametrize("H,Hkv,d,dtype", [(4, 4, 64, "f32"), (8, 2, 128, "bf16"), (2, 1, 32, "bf16"),
                                           (6, 3, 64, "bf16"), (4, 2, 64, "f16"), (2, 2, 32, "f32"),
                                           (4, 2, 128, "f32")])
def test_packed_mixed_lengths(H, Hkv, d, dtype, causal, normalise):
    lens = lengths_mix(9, 1, 1500, seed=d + H, extra=(0, 1, 33, 700))
    run_packed(lens, H, Hkv, d, dtype, causal, normalise, seed=H * d)


def test_packed_many_short_sequences():
    lens = lengths_mix(300, 0, 90, seed=5)
    run_packed(lens, 4, 2, 64, "bf16", 1, 1, seed=11)


@pytest.mark.parametrize("chunk", [32, 64, 128, 256])
def test_packed_every_chunk(chunk):
    lens = lengths_mix(6, 100, 2500, seed=chunk)
    run_packed(lens, 2, 2, 64, "bf16", 1, 1, chunk=chunk, seed=chunk)


def test_packed_one_long_sequence_equals_dense():
    """A packed batch of one sequence is the dense pass of that sequence (same plan
    inputs up to the segment length: rows agree to the bar, states likewise)."""
    H, Hkv, N, d = 8, 8, 4096, 64
    q, k, v = (t.cuda() for t in make_qkv(1, H, Hkv, N, d, "f32", 3))
    cu = torch.tensor([0, N], dtype=torch.int32, device="cuda")
    o_p, S_p, z_p = ops.fwd_packed(q.reshape(-1), k.reshape(-1), v.reshape(-1), cu, H, Hkv, d, want_state=True)
    o_d, S_d, z_d = ops.fwd(q, k, v, want_state=True)
    torch.cuda.synchronize()
    assert rows_rel_err(o_p.view(1, H, N, d).cpu().numpy(), o_d.cpu().numpy()) <= 1e-5
    assert rows_rel_err(S_p.cpu().numpy().reshape(H, -1), S_d.cpu().numpy().reshape(H, -1)) <= 1e-5


def test_packed_malformed_offsets_stay_in_bounds():
    """Decreasing and out-of-range offsets: the call succeeds and touches nothing outside
    the buffers (the output guard bands stay untouched); the rows of the well-formed
    sequences (those whose clamped boundaries are their own) are still right."""
    H, Hkv, d, total = 2, 2, 64, 300
    q, k, v = (t.cuda() for t in make_qkv(1, H, Hkv, total, d, "bf16", 8))
    guard = 4096
    out_buf = torch.full((H * total * d + 2 * guard,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = out_buf[guard:guard + H * total * d]
    cu = torch.tensor([0, 100, 50, 400, -5, 300], dtype=torch.int32, device="cuda")
    o = ops.fwd_packed(q.reshape(-1), k.reshape(-1), v.reshape(-1), cu, H, Hkv, d, out=out)
    torch.cuda.synchronize()
    assert torch.all(out_buf[:guard] == 7.0) and torch.all(out_buf[-guard:] == 7.0)
    # sequence 0 owns tokens [0, 100) (boundaries 0 and 100 clamp to themselves): its
    # blocks are the first H * 100 * d elements of q, k, v read as [H][100][d]
    blocks = [t.reshape(-1)[: H * 100 * d].view(1, H, 100, d).cpu() for t in (q, k, v)]
    ref = oracle.ref_fwd(*blocks)
    got = o[: H * 100 * d].view(1, H, 100, d).double().cpu().numpy()
    assert rows_rel_err(got, ref) <= TOL["bf16"]


def test_packed_argument_errors():
    H, Hkv, d = 2, 2, 64
    x = torch.zeros(H * 10 * d, device="cuda")
    cu = torch.tensor([0, 10], dtype=torch.int32, device="cuda")
    nb = la.linattn_fwd_packed_workspace_bytes(1, H, Hkv, 10, d, 1, la.LINATTN_F32)
    ws = torch.empty(nb // 4 + 1, device="cuda")
    assert la.linattn_fwd_packed(x, x, x, torch.empty_like(x), None, 1, 10, H, Hkv, d, 1, 1, la.LINATTN_F32,
                                 workspace=ws, workspace_bytes=nb) == -1
    assert la.linattn_fwd_packed(x, x, x, torch.empty_like(x), cu, 1, 10, H, Hkv, d, 1, 1, la.LINATTN_F32,
                                 workspace=ws, workspace_bytes=nb - 4) == -5
    assert la.linattn_fwd_packed(x, x, x, torch.empty_like(x), cu, 1, 10, H, Hkv, d, 1, 1, la.LINATTN_F32,
                                 workspace=ws, workspace_bytes=nb) == 0
    torch.cuda.synchronize()
