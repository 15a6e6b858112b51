"""Pins for the oracle's backward pass (CPU only).

The oracle differentiates the forward pass by hand (the chain rule written as
a forward walk for dQ and a reverse-time walk for dK, dV).  Each test checks
it against something other than itself: torch autograd of the quadratic
masked attention form in fp64 (a different route to the same gradient),
central finite differences of the oracle's own forward pass, closed forms for
one token, and invariants the normalised form implies.  The planted slips in
``test_oracle_mutants.py`` must fail at least one of these.

Method: the forward of the LinearTile 1.0.0 README, "How It Works"
(O = phi(Q)(phi(K)^T V), phi = ELU + 1, optional normaliser); the backward is
its gradient.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from linattn_inputs import make_qkv, randn


def autograd_quadratic(q, k, v, dout, causal, normalise):
    """dQ, dK, dV by torch autograd (fp64) of (M * phi(Q) phi(K)^T) V [/ row sums]."""
    q, k, v, dout = (torch.as_tensor(np.asarray(t, dtype=np.float64)) for t in (q, k, v, dout))
    q.requires_grad_(True)
    k.requires_grad_(True)
    v.requires_grad_(True)
    B, H, N, d = q.shape
    G = H // k.shape[1]
    kk = k.repeat_interleave(G, dim=1)
    vv = v.repeat_interleave(G, dim=1)
    A = (F.elu(q) + 1) @ (F.elu(kk) + 1).transpose(-1, -2)
    if causal:
        A = A * torch.tril(torch.ones(N, N, dtype=torch.float64))
    o = A @ vv
    if normalise:
        o = o / A.sum(-1, keepdim=True)
    (o * dout).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy(), o.detach().numpy()


def rel(got, ref):
    """Largest difference over the larger of the largest reference value and 1 (an
    exactly-zero gradient, such as dQ for one normalised token, is compared absolutely)."""
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1.0))


SHAPES = [(1, 1, 1, 1, 4), (1, 2, 2, 7, 8), (2, 4, 2, 13, 4), (1, 6, 2, 32, 16), (1, 3, 1, 20, 5), (2, 2, 1, 40, 32)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dH%dK%dN%dd%d" % s)
@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_bwd_matches_autograd_of_quadratic_form(shape, causal, normalise):
    B, H, Hkv, N, d = shape
    q, k, v = make_qkv(B, H, Hkv, N, d, "f32", 31 + N + d)
    dout = randn((B, H, N, d), 77 + N)
    dq_r, dk_r, dv_r, o = autograd_quadratic(q, k, v, dout, causal, normalise)
    dq, dk, dv = oracle.ref_bwd(q, k, v, o, dout, causal=causal, normalise=normalise)
    assert rel(dq, dq_r) <= 1e-10 and rel(dk, dk_r) <= 1e-10 and rel(dv, dv_r) <= 1e-10


@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_bwd_matches_finite_differences(causal, normalise):
    """Central differences of L = sum(dO * O) through the oracle's own forward."""
    B, H, Hkv, N, d = 1, 4, 2, 9, 6
    q, k, v = (t.double().numpy() for t in make_qkv(B, H, Hkv, N, d, "f32", 5))
    dout = randn((B, H, N, d), 6).double().numpy()

    def loss(q_, k_, v_):
        return float((oracle.ref_fwd(q_, k_, v_, causal=causal, normalise=normalise) * dout).sum())

    o = oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise)
    grads = oracle.ref_bwd(q, k, v, o, dout, causal=causal, normalise=normalise)
    rng = np.random.default_rng(9)
    eps = 1e-6
    for which, x in enumerate((q, k, v)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in x.shape)
            args = [q.copy(), k.copy(), v.copy()]
            args[which][idx] += eps
            up = loss(*args)
            args[which][idx] -= 2 * eps
            dn = loss(*args)
            fd = (up - dn) / (2 * eps)
            g = grads[which][idx]
            assert abs(g - fd) <= 1e-6 * max(1.0, abs(fd)), (which, idx, g, fd)


@pytest.mark.parametrize("normalise", [1, 0])
def test_bwd_single_token_closed_form(normalise):
    """N = 1: normalised o = v, so dQ = dK = 0 and dV = sum of dO over the group;
    unnormalised o_h = (a_h . b) v."""
    B, H, Hkv, d = 2, 6, 2, 8
    q, k, v = (t.double().numpy() for t in make_qkv(B, H, Hkv, 1, d, "f32", 12))
    dout = randn((B, H, 1, d), 13).double().numpy()
    o = oracle.ref_fwd(q, k, v, normalise=normalise)
    dq, dk, dv = oracle.ref_bwd(q, k, v, o, dout, normalise=normalise)
    G = H // Hkv
    phi = lambda x: np.where(x > 0, x + 1, np.exp(x))
    dphi = lambda x: np.where(x > 0, 1.0, np.exp(x))
    for b in range(B):
        for g in range(Hkv):
            bk, vk = phi(k[b, g, 0]), v[b, g, 0]
            heads = range(g * G, (g + 1) * G)
            if normalise:
                assert np.abs(dq[b, g * G:(g + 1) * G]).max() <= 1e-12
                assert np.abs(dk[b, g]).max() <= 1e-12
                np.testing.assert_allclose(dv[b, g, 0], sum(dout[b, h, 0] for h in heads), rtol=1e-13)
            else:
                a = {h: phi(q[b, h, 0]) for h in heads}
                np.testing.assert_allclose(dv[b, g, 0], sum((a[h] @ bk) * dout[b, h, 0] for h in heads),
                                           rtol=1e-12)
                for h in heads:
                    np.testing.assert_allclose(dq[b, h, 0], (vk @ dout[b, h, 0]) * bk * dphi(q[b, h, 0]),
                                               rtol=1e-12)
                np.testing.assert_allclose(dk[b, g, 0],
                                           sum((vk @ dout[b, h, 0]) * a[h] for h in heads) * dphi(k[b, g, 0]),
                                           rtol=1e-12)


@pytest.mark.parametrize("causal", [1, 0])
def test_bwd_normalised_invariants(causal):
    """Normalised rows are convex combinations of values: the dV rows sum to the dO rows' sum,
    and shifting every value by one vector leaves dQ and dK unchanged."""
    B, H, Hkv, N, d = 1, 4, 2, 30, 8
    q, k, v = (t.double().numpy() for t in make_qkv(B, H, Hkv, N, d, "f32", 21))
    dout = randn((B, H, N, d), 22).double().numpy()
    o = oracle.ref_fwd(q, k, v, causal=causal)
    dq, dk, dv = oracle.ref_bwd(q, k, v, o, dout, causal=causal)
    np.testing.assert_allclose(dv.sum(axis=(1, 2)), dout.sum(axis=(1, 2)), rtol=1e-11, atol=1e-11)
    shift = np.linspace(-2, 3, d)
    v2 = v + shift
    o2 = oracle.ref_fwd(q, k, v2, causal=causal)
    dq2, dk2, dv2 = oracle.ref_bwd(q, k, v2, o2, dout, causal=causal)
    assert rel(dq2, dq) <= 1e-10 and rel(dk2, dk) <= 1e-10 and rel(dv2, dv) <= 1e-12


def test_bwd_gqa_equals_mha_with_repeated_kv():
    B, H, Hkv, N, d = 1, 6, 2, 17, 8
    q, k, v = (t.double().numpy() for t in make_qkv(B, H, Hkv, N, d, "f32", 3))
    dout = randn((B, H, N, d), 4).double().numpy()
    G = H // Hkv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    for causal in (1, 0):
        o = oracle.ref_fwd(q, k, v, causal=causal)
        dq, dk, dv = oracle.ref_bwd(q, k, v, o, dout, causal=causal)
        dq_m, dk_m, dv_m = oracle.ref_bwd(q, kr, vr, o, dout, causal=causal)
        assert rel(dq, dq_m) <= 1e-13
        assert rel(dk, dk_m.reshape(B, Hkv, G, N, d).sum(2)) <= 1e-13
        assert rel(dv, dv_m.reshape(B, Hkv, G, N, d).sum(2)) <= 1e-13


def test_bwd_causal_last_key_only_seen_by_last_query():
    """The last key is seen by the last query only: its dV equals (a_N . b_N) g_N."""
    B, H, Hkv, N, d = 1, 1, 1, 12, 4
    q, k, v = (t.double().numpy() for t in make_qkv(B, H, Hkv, N, d, "f32", 8))
    dout = randn((B, H, N, d), 9).double().numpy()
    o = oracle.ref_fwd(q, k, v, normalise=False)
    _, _, dv = oracle.ref_bwd(q, k, v, o, dout, normalise=False)
    phi = lambda x: np.where(x > 0, x + 1, np.exp(x))
    a, b = phi(q[0, 0, -1]), phi(k[0, 0, -1])
    np.testing.assert_allclose(dv[0, 0, -1], (a @ b) * dout[0, 0, -1], rtol=1e-13)
