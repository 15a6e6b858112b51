"""The library's launches captured in a HIP graph and replayed.

A serving loop captures linattn_fwd / linattn_decode_step once and replays
the graph.  Every replay here runs after eager work of the program's own
(other launches, host synchronisation) and must reproduce the eager result
bitwise: the kernels are deterministic and none of them is a memset node.
"""
import numpy as np
import pytest
import torch

import oracle
from linattn_inputs import DecodeStream, make_qkv
from sequence_mixing_amd import ops

pytestmark = pytest.mark.gpu


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("B,H,Hkv,N,d,dtype,causal", [
    (2, 8, 8, 1000, 64, "f32", 1),
    (1, 8, 2, 700, 128, "bf16", 1),
    (2, 4, 4, 513, 32, "bf16", 0),
])
def test_fwd_graph_replays_match_eager(B, H, Hkv, N, d, dtype, causal):
    print(f"graph fwd B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype} causal={causal}", flush=True)
    q, k, v = (t.contiguous().cuda() for t in make_qkv(B, H, Hkv, N, d, dtype, 404 + N))
    out = torch.empty_like(q)
    ws = ops.workspace(B, H, Hkv, N, d, causal, q.dtype)
    ref = ops.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()

    def step():
        ops.fwd(q, k, v, causal=causal, out=out, ws=ws)

    g = _capture(step)
    noise = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        out.fill_(float("nan"))
        noise.mul_(1.0001).sum()            # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep} differs from the eager result"


def test_decode_graph_replays_match_eager():
    B, H, Hkv, d = 4, 8, 2, 128
    q0, k0, v0 = (t.contiguous().cuda() for t in make_qkv(B, Hkv, Hkv, 60, d, "bf16", 9))
    _, S0, z0 = ops.fwd(q0, k0, v0, want_state=True)
    stream = DecodeStream(B, H, Hkv, d, "bf16", 77)
    steps = [tuple(t.cuda() for t in stream.next()) for _ in range(3)]
    outs = [torch.empty_like(s[0]) for s in steps]

    # eager reference: three steps from (S0, z0)
    S, z = S0.clone(), z0.clone()
    ref = [ops.decode_step(S, z, *st).clone() for st in steps]
    S_ref, z_ref = S.clone(), z.clone()

    S.copy_(S0)
    z.copy_(z0)

    def run():
        for st, o in zip(steps, outs):
            ops.decode_step(S, z, *st, out=o)

    g = _capture(run)
    for rep in range(3):
        S.copy_(S0)
        z.copy_(z0)
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t in range(3):
            assert torch.equal(outs[t], ref[t]), f"replay {rep} step {t}"
        assert torch.equal(S, S_ref) and torch.equal(z, z_ref)
    # and the eager chain itself against the oracle
    Sr, zr = S0.double().cpu().numpy(), z0.double().cpu().numpy()
    for st, r in zip(steps, ref):
        o = oracle.ref_decode_step(Sr, zr, *(x.cpu() for x in st), normalise=True)
        g_ = r.double().cpu().numpy()
        assert np.max(np.abs(g_ - o) / np.abs(o).max(axis=-1, keepdims=True)) <= 2e-2
