"""Non-finite inputs on the GPU, through the C ABI, against the oracle.

NaN and Inf are not checked and propagate (include/linattn.h).  What the
kernels guarantee, and what this file checks:
  * a NaN query spoils its own row only;
  * a NaN or Inf key at token s spoils the causal rows t >= s of its kv group
    and no row before s (the causal mask is a select, not a product, so a
    masked non-finite score does not leak);
  * a NaN or Inf value at token s spoils the rows t >= s; rows before the
    32-token key tile that holds s (before the pair of tiles, for kernels
    that keep one state copy per pair) stay finite and equal the oracle's;
    rows of that tile before s may be spoiled too: the product of the tile's
    values with the masked scores multiplies the non-finite value by a zero
    score (NaN), which the oracle's token-by-token sum never forms;
  * non-causal: every row of the group is spoiled.
Clean rows are compared with the oracle at the forward's bars.
"""
import numpy as np
import pytest
import torch

import oracle
from linattn_inputs import make_qkv
from sequence_mixing_amd import ops

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err_rows(got, ref):
    den = np.abs(ref).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(got - ref).max(axis=-1) / den).max()) if got.size else 0.0


def run(q, k, v, causal):
    out = ops.fwd(q.contiguous().cuda(), k.contiguous().cuda(), v.contiguous().cuda(), causal=causal)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy()
    ref = oracle.ref_fwd(q, k, v, causal=causal, normalise=True)
    return got, ref


SHAPES = [(2, 4, 2, 700, 64, "f32"), (1, 8, 8, 1500, 64, "bf16"), (1, 4, 1, 600, 128, "bf16")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dK%dN%dd%d%s" % s)
def test_nan_query_row(shape):
    B, H, Hkv, N, d, dtype = shape
    q, k, v = make_qkv(B, H, Hkv, N, d, dtype, 5)
    q[B - 1, H - 1, N // 2, 3] = float("nan")
    print(f"nan query {shape}", flush=True)
    got, ref = run(q, k, v, True)
    fin = np.isfinite(got).all(axis=-1)
    assert not fin[B - 1, H - 1, N // 2] and fin.sum() == fin.size - 1
    assert rel_err_rows(got[fin], ref[fin]) <= TOL[dtype]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dK%dN%dd%d%s" % s)
@pytest.mark.parametrize("what,val", [("k", float("nan")), ("k", float("inf")), ("v", float("nan")),
                                      ("v", float("inf"))])
def test_bad_key_or_value(shape, what, val):
    B, H, Hkv, N, d, dtype = shape
    G = H // Hkv
    q, k, v = make_qkv(B, H, Hkv, N, d, dtype, 6)
    s = (N * 2) // 3 + 5  # inside a tile, not at its start
    g = Hkv - 1
    (k if what == "k" else v)[0, g, s, 1] = val
    print(f"bad {what}={val} at token {s}, {shape}", flush=True)
    got, ref = run(q, k, v, True)
    heads = slice(g * G, (g + 1) * G)
    fin = np.isfinite(got).all(axis=-1)
    assert (~fin[0, heads, s:]).all(), "rows from the bad token on must be spoiled"
    # rows before s: finite and at the bar for keys; before the tile pair for values
    clean_to = s if what == "k" else (s // 64) * 64
    assert fin[0, heads, :clean_to].all()
    assert rel_err_rows(got[0, heads, :clean_to], ref[0, heads, :clean_to]) <= TOL[dtype]
    # every other (batch, kv group) untouched
    other = np.ones(got.shape[:2], dtype=bool)
    other[0, heads] = False
    assert fin[other].all() and rel_err_rows(got[other], ref[other]) <= TOL[dtype]


@pytest.mark.parametrize("shape", SHAPES[:2], ids=lambda s: "B%dH%dK%dN%dd%d%s" % s)
def test_noncausal_bad_key_spoils_group(shape):
    B, H, Hkv, N, d, dtype = shape
    G = H // Hkv
    q, k, v = make_qkv(B, H, Hkv, N, d, dtype, 7)
    k[0, 0, N // 3, 0] = float("nan")
    got, ref = run(q, k, v, False)
    fin = np.isfinite(got).all(axis=-1)
    assert (~fin[0, :G]).all()
    other = np.ones(got.shape[:2], dtype=bool)
    other[0, :G] = False
    assert fin[other].all() and rel_err_rows(got[other], ref[other]) <= TOL[dtype]
