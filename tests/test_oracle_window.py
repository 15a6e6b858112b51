"""Pins of the oracle's sliding-window pass (a reading of the LinearTile 1.0.0
README's "Features" list, sliding-window item: the causal band of W keys,
query t sees t - W < s <= t).  Each pin reaches the result by a route other
than the oracle's own per-query band sum:
  * W >= N is the plain causal pass (the oracle's running-state code);
  * row t is the last row of a plain causal pass over the tokens of its band
    alone (brute force over every t on small inputs);
  * the running sums' difference S_t - S_{t-W}, z_t - z_{t-W} built with numpy
    cumulative sums of outer products;
  * W = 1 gives o_t = v_t (normalised) and (phi(q_t) . phi(k_t)) v_t
    (unnormalised);
  * normalised rows are convex combinations of the band's values, a common
    shift of every value shifts every row, and a token s changes only the rows
    s .. s + W - 1 (bitwise).
"""
import numpy as np
import pytest
import torch

import oracle


def phi(x):
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def inputs(B, H, Hkv, N, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, N, d)), rng.standard_normal((B, Hkv, N, d)),
            rng.standard_normal((B, Hkv, N, d)))


def rel(a, b):
    den = np.maximum(np.abs(b).max(axis=-1, keepdims=True), 1e-300)
    return float((np.abs(a - b) / den).max()) if a.size else 0.0


SHAPES = [(1, 1, 1, 17, 4), (2, 4, 2, 40, 8), (1, 3, 1, 33, 16), (1, 2, 2, 64, 32)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("normalise", [1, 0])
def test_window_at_least_n_is_causal(shape, normalise):
    q, k, v = inputs(*shape, seed=1)
    N = shape[3]
    for W in (N, N + 5, 10 * N):
        assert rel(oracle.ref_fwd_window(q, k, v, W, normalise), oracle.ref_fwd(q, k, v, True, normalise)) < 1e-12


@pytest.mark.parametrize("shape", SHAPES[:3])
@pytest.mark.parametrize("W", [1, 2, 5, 16])
@pytest.mark.parametrize("normalise", [1, 0])
def test_row_is_last_row_of_causal_pass_over_its_band(shape, W, normalise):
    q, k, v = inputs(*shape, seed=2 + W)
    B, H, Hkv, N, d = shape
    o = oracle.ref_fwd_window(q, k, v, W, normalise)
    for t in range(N):
        s0 = max(0, t - W + 1)
        sub = oracle.ref_fwd(q[:, :, s0:t + 1], k[:, :, s0:t + 1], v[:, :, s0:t + 1], True, normalise)
        assert rel(o[:, :, t], sub[:, :, -1]) < 1e-12


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("W", [1, 3, 8, 31])
@pytest.mark.parametrize("normalise", [1, 0])
def test_difference_of_running_sums(shape, W, normalise):
    """num_t = phi(q_t)^T (S_t - S_{t-W}), den_t = phi(q_t) . (z_t - z_{t-W}), with S the
    cumulative sum of phi(k_s) v_s^T (torch, fp64), GQA by repeating the kv heads."""
    B, H, Hkv, N, d = shape
    q, k, v = inputs(*shape, seed=3 + W)
    G = H // Hkv
    pk = torch.from_numpy(phi(np.repeat(k, G, axis=1)))
    vv = torch.from_numpy(np.repeat(v, G, axis=1))
    pq = torch.from_numpy(phi(q))
    S = torch.cumsum(pk[..., :, None] * vv[..., None, :], dim=2)   # [B,H,N,d,d]
    z = torch.cumsum(pk, dim=2)
    Sw, zw = S.clone(), z.clone()
    Sw[:, :, W:] -= S[:, :, :-W] if W < N else 0
    zw[:, :, W:] -= z[:, :, :-W] if W < N else 0
    num = torch.einsum("bhti,bhtij->bhtj", pq, Sw)
    den = (pq * zw).sum(-1, keepdim=True)
    ref = (num / den if normalise else num).numpy()
    # S_t - S_{t-W} cancels: bound the error by the same form taken with |v|
    Sa = torch.cumsum(pk[..., :, None] * vv.abs()[..., None, :], dim=2)
    scale = torch.einsum("bhti,bhtij->bhtj", pq, Sa).numpy()
    if normalise:
        scale = scale / den.numpy()
    o = oracle.ref_fwd_window(q, k, v, W, normalise)
    err = np.abs(o - ref).max()
    assert err <= 1e-12 * max(1.0, float(np.abs(scale).max()))


@pytest.mark.parametrize("normalise", [1, 0])
def test_window_one_closed_form(normalise):
    q, k, v = inputs(2, 4, 2, 25, 8, seed=5)
    o = oracle.ref_fwd_window(q, k, v, 1, normalise)
    vv = np.repeat(v, 2, axis=1)
    if normalise:
        assert rel(o, vv) < 1e-14
    else:
        a = (phi(q) * phi(np.repeat(k, 2, axis=1))).sum(-1, keepdims=True)
        assert rel(o, a * vv) < 1e-14


def test_convex_shift_and_locality():
    B, H, Hkv, N, d, W = 1, 2, 1, 50, 8, 7
    q, k, v = inputs(B, H, Hkv, N, d, seed=6)
    o = oracle.ref_fwd_window(q, k, v, W, True)
    vv = v[:, 0]
    for t in range(N):
        band = vv[:, max(0, t - W + 1):t + 1]
        assert (o[:, :, t] >= band.min(axis=1)[:, None] - 1e-12).all()
        assert (o[:, :, t] <= band.max(axis=1)[:, None] + 1e-12).all()
    assert rel(oracle.ref_fwd_window(q, k, v + 3.5, W, True), o + 3.5) < 1e-12
    s = 20
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, s] += 1.0
    v2[0, 0, s] -= 2.0
    o2 = oracle.ref_fwd_window(q, k2, v2, W, True)
    changed = np.any(o2 != o, axis=-1)[0, 0]
    assert not changed[:s].any() and not changed[s + W:].any() and changed[s:s + W].all()


def test_invalid_window_refused():
    q, k, v = inputs(1, 1, 1, 4, 2, seed=7)
    with pytest.raises(ValueError):
        oracle.ref_fwd_window(q, k, v, 0)
