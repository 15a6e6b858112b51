"""Pins for the oracle's other feature maps (CPU only): ReLU and softplus in
place of ELU + 1 (README "Features": custom kernel plugins, phi replaceable).

Each map is checked against torch's own routine and its autograd derivative,
and the forward and backward with that map against the quadratic masked
attention form built from torch's routine (a different route: brute force and
autograd).  ReLU can zero a denominator, so its normalised cases use inputs
shifted to be positive."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from linattn_inputs import make_qkv, randn

# torch returns x itself for softplus above x = 20 by default; the cutoff is raised so the
# library routine computes log(1 + e^x) everywhere, the definition.
LIB = {"elu1": lambda x: F.elu(x) + 1, "relu": F.relu, "softplus": lambda x: F.softplus(x, threshold=100.0)}


@pytest.mark.parametrize("m", ["elu1", "relu", "softplus"])
def test_feature_map_and_derivative_match_torch(m):
    xs = torch.tensor([-30.0, -5.0, -1.0, -1e-3, 0.0, 1e-3, 0.5, 1.0, 3.0, 25.0], dtype=torch.float64,
                      requires_grad=True)
    y = LIB[m](xs)
    y.sum().backward()
    for x, yy, gg in zip(xs.detach().tolist(), y.detach().tolist(), xs.grad.tolist()):
        assert abs(oracle.phi(x, m) - yy) <= 1e-15 * max(1.0, abs(yy))
        if x != 0.0:  # ReLU's derivative at 0 is a convention (both sides are reported here as 0)
            assert abs(oracle.dphi(x, m) - gg) <= 1e-15 * max(1.0, abs(gg))
    assert oracle.phi(-0.7) == pytest.approx(np.exp(-0.7), rel=1e-15)  # the default is ELU + 1 again


def quadratic(q, k, v, causal, normalise, m):
    q, k, v = (torch.as_tensor(np.asarray(t, dtype=np.float64)) for t in (q, k, v))
    G = q.shape[1] // k.shape[1]
    A = LIB[m](q) @ LIB[m](k.repeat_interleave(G, 1)).transpose(-1, -2)
    if causal:
        A = A * torch.tril(torch.ones(q.shape[2], q.shape[2], dtype=torch.float64))
    o = A @ v.repeat_interleave(G, 1)
    return (o / A.sum(-1, keepdim=True) if normalise else o).numpy()


def inputs(m, normalise, seed, shape=(1, 4, 2, 24, 8)):
    q, k, v = (t.double() for t in make_qkv(*shape, "f32", seed))
    if m == "relu" and normalise:
        q, k = q.abs() + 0.1, k.abs() + 0.1
    return q, k, v


@pytest.mark.parametrize("m", ["relu", "softplus"])
@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_forward_with_feature_map(m, causal, normalise):
    q, k, v = inputs(m, normalise, 40 + causal)
    got = oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise, phi_map=m)
    ref = quadratic(q, k, v, causal, normalise, m)
    assert np.abs(got - ref).max() <= 1e-12 * max(1.0, np.abs(ref).max())
    # and the default map is untouched
    assert np.array_equal(oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise),
                          oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise, phi_map="elu1"))


@pytest.mark.parametrize("m", ["relu", "softplus"])
@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_backward_with_feature_map(m, causal, normalise):
    q, k, v = inputs(m, normalise, 50 + causal)
    dout = randn(tuple(q.shape), 51).double()
    qt, kt, vt = (t.clone().requires_grad_(True) for t in (q, k, v))
    G = q.shape[1] // k.shape[1]
    A = LIB[m](qt) @ LIB[m](kt.repeat_interleave(G, 1)).transpose(-1, -2)
    if causal:
        A = A * torch.tril(torch.ones(q.shape[2], q.shape[2], dtype=torch.float64))
    o = A @ vt.repeat_interleave(G, 1)
    if normalise:
        o = o / A.sum(-1, keepdim=True)
    (o * dout).sum().backward()
    got = oracle.ref_bwd(q, k, v, o.detach().numpy(), dout, causal=causal, normalise=normalise, phi_map=m)
    for g, r in zip(got, (qt.grad, kt.grad, vt.grad)):
        r = r.numpy()
        assert np.abs(g - r).max() <= 1e-10 * max(1.0, np.abs(r).max())


def test_decode_with_softplus_continues_prefill():
    B, H, Hkv, N, d = 2, 4, 2, 9, 8
    q, k, v = (t.double() for t in make_qkv(B, H, Hkv, N + 1, d, "f32", 61))
    full = oracle.ref_fwd(q, k, v, phi_map="softplus")
    _, S, z = oracle.ref_fwd(q[:, :, :N], k[:, :, :N], v[:, :, :N], want_state=True, phi_map="softplus")
    o = oracle.ref_decode_step(S, z, q[:, :, N], k[:, :, N], v[:, :, N], phi_map="softplus")
    assert np.abs(o - full[:, :, N]).max() <= 1e-12 * np.abs(full).max()
