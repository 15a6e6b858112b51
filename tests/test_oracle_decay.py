"""Pins for the oracle's decayed sums (CPU only).

Reading (the pages give decay only for the scan of the Stream efficiency
essay, section 4.2, h_t = h_{t-1} a_t + b_t): with a log-decay g_t per
(batch, kv head, token) and a_t = exp(g_t), S_t = a_t S_{t-1} + phi(k_t) v_t^T
and z_t = a_t z_{t-1} + phi(k_t); o_t = phi(q_t)^T S_t (/ phi(q_t) . z_t).

Each test checks the recurrence against something else: the unrolled
quadratic form with an explicit decay matrix (products of a_u), the plain
method (g = 0), a reset (a_t = 0 forgets the past), the geometric series of a
constant key, continuation, decode, and the convexity of normalised rows.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from linattn_inputs import make_decay, make_qkv

REL = 1e-12


def phi_lib(x):
    return (F.elu(torch.from_numpy(np.asarray(x, dtype=np.float64)), alpha=1.0) + 1.0).numpy()


def decayed_quadratic(q, k, v, g, normalise):
    """Brute force: o_t = sum_{s<=t} w_ts (phi(q_t).phi(k_s)) v_s (/ the same sum without v),
    w_ts = prod_{s<u<=t} exp(g_u), built by multiplying the factors one at a time."""
    q, k, v, g = (np.asarray(t, dtype=np.float64) for t in (q, k, v, g))
    B, H, N, d = q.shape
    G = H // k.shape[1]
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            kv = h // G
            A = phi_lib(q[b, h]) @ phi_lib(k[b, kv]).T
            W = np.zeros((N, N))
            for t in range(N):
                w = 1.0
                for s in range(t, -1, -1):
                    W[t, s] = w
                    w *= np.exp(g[b, kv, s])
            M = A * W
            num = M @ v[b, kv]
            out[b, h] = num / M.sum(axis=1, keepdims=True) if normalise else num
    return out


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64).reshape(-1, np.shape(a)[-1])
    b = np.asarray(b, dtype=np.float64).reshape(-1, np.shape(b)[-1])
    den = np.abs(b).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(a - b).max(axis=1) / den).max()) if a.size else 0.0


def inputs(B, H, Hkv, N, d, seed, scale=1.0):
    q, k, v = make_qkv(B, H, Hkv, N, d, "f32", seed)
    g = make_decay(B, Hkv, N, seed + 1) * scale
    return q, k, v, g


def test_zero_decay_is_the_plain_method():
    q, k, v, _ = inputs(2, 4, 2, 37, 8, 11)
    g = torch.zeros(2, 2, 37)
    for normalise in (True, False):
        a, Sa, za = oracle.ref_fwd(q, k, v, normalise=normalise, want_state=True)
        b, Sb, zb = oracle.ref_fwd_decay(q, k, v, g, normalise=normalise, want_state=True)
        assert np.array_equal(a, b) and np.array_equal(Sa, Sb) and np.array_equal(za, zb)


@pytest.mark.parametrize("normalise", [True, False])
@pytest.mark.parametrize("scale", [1.0, 16.0])
def test_equals_decayed_quadratic_form(normalise, scale):
    # scale 16: g = logsigmoid(u), decays down to exp(-3) per token
    q, k, v, g = inputs(1, 4, 2, 29, 8, 21, scale)
    got = oracle.ref_fwd_decay(q, k, v, g, normalise=normalise)
    assert rel_err(got, decayed_quadratic(q, k, v, g, normalise)) < REL


def test_reset_token_forgets_the_past():
    """a_r = 0 (g_r = -inf): from token r on, the rows and final sums are those of a
    fresh pass over tokens r.."""
    q, k, v, g = inputs(1, 2, 2, 40, 8, 31)
    r = 17
    g[:, :, r] = -float("inf")
    out, S, z = oracle.ref_fwd_decay(q, k, v, g, want_state=True)
    tail, St, zt = oracle.ref_fwd_decay(q[:, :, r:], k[:, :, r:], v[:, :, r:], g[:, :, r:], want_state=True)
    assert rel_err(out[:, :, r:], tail) < REL
    assert rel_err(S, St) < REL and rel_err(z, zt) < REL
    # and the rows before the reset are untouched by it
    head = oracle.ref_fwd_decay(q[:, :, :r], k[:, :, :r], v[:, :, :r], g[:, :, :r])
    assert np.array_equal(out[:, :, :r], head)


def test_constant_key_geometric_series():
    """k_t = k, v_t = v, a_t = gamma: S_t = phi(k) v^T (1 - gamma^(t+1)) / (1 - gamma)."""
    N, d, gamma = 50, 4, 0.9
    q = torch.randn(1, 1, N, d, generator=torch.Generator().manual_seed(5), dtype=torch.float64)
    k = torch.tensor([0.3, -1.2, 2.0, -0.1], dtype=torch.float64).expand(1, 1, N, d).contiguous()
    v = torch.tensor([1.5, -0.5, 0.25, 3.0], dtype=torch.float64).expand(1, 1, N, d).contiguous()
    g = torch.full((1, 1, N), np.log(gamma), dtype=torch.float64)
    fk, vv = phi_lib(k[0, 0, 0]), v[0, 0, 0].numpy()
    geo = (1 - gamma ** (np.arange(N) + 1)) / (1 - gamma)
    num = oracle.ref_fwd_decay(q, k, v, g, normalise=False)
    expect = (phi_lib(q[0, 0]) @ fk)[:, None] * geo[:, None] * vv[None, :]
    assert rel_err(num[0, 0], expect) < REL
    o, S, z = oracle.ref_fwd_decay(q, k, v, g, want_state=True)
    assert rel_err(o[0, 0], np.broadcast_to(vv, (N, d))) < REL
    assert rel_err(S[0, 0], np.outer(fk, vv) * geo[-1]) < REL
    assert rel_err(z[0, 0][None], (fk * geo[-1])[None]) < REL


@pytest.mark.parametrize("cut", [1, 13, 32, 63])
def test_continuation_equals_one_pass(cut):
    q, k, v, g = inputs(2, 4, 2, 64, 8, 41)
    full, S, z = oracle.ref_fwd_decay(q, k, v, g, want_state=True)
    a, Sa, za = oracle.ref_fwd_decay(q[:, :, :cut], k[:, :, :cut], v[:, :, :cut], g[:, :, :cut], want_state=True)
    b, Sb, zb = oracle.ref_fwd_decay(q[:, :, cut:], k[:, :, cut:], v[:, :, cut:], g[:, :, cut:], want_state=True,
                                     state_in=Sa, z_in=za)
    assert np.array_equal(np.concatenate([a, b], axis=2), full)
    assert np.array_equal(Sb, S) and np.array_equal(zb, z)


@pytest.mark.parametrize("normalise", [True, False])
def test_decode_steps_equal_prefill_rows(normalise):
    B, H, Hkv, N, d = 2, 4, 2, 12, 8
    q, k, v, g = inputs(B, H, Hkv, N, d, 51)
    full = oracle.ref_fwd_decay(q, k, v, g, normalise=normalise)
    S = np.zeros((B, Hkv, d, d))
    z = np.zeros((B, Hkv, d))
    for t in range(N):
        o = oracle.ref_decode_step_decay(S, z, q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], normalise=normalise)
        assert rel_err(o, full[:, :, t]) < REL


def test_normalised_rows_are_convex_combinations():
    q, k, v, g = inputs(1, 2, 1, 60, 6, 61, 16.0)
    out = oracle.ref_fwd_decay(q, k, v, g)
    vv = v.double().numpy()[0, 0]
    for t in range(60):
        lo, hi = vv[: t + 1].min(axis=0), vv[: t + 1].max(axis=0)
        assert np.all(out[0, :, t] >= lo - 1e-12) and np.all(out[0, :, t] <= hi + 1e-12)


def test_gqa_heads_share_their_kv_heads_decay():
    """A group's query heads read the same decayed sums: GQA equals MHA with K, V and g repeated."""
    q, k, v, g = inputs(1, 6, 2, 25, 8, 71)
    G = 3
    a = oracle.ref_fwd_decay(q, k, v, g)
    b = oracle.ref_fwd_decay(q, k.repeat_interleave(G, 1), v.repeat_interleave(G, 1), g.repeat_interleave(G, 1))
    assert np.array_equal(a, b)


def test_decay_argument_checks():
    q, k, v, g = inputs(1, 2, 2, 5, 4, 81)
    with pytest.raises(AssertionError):
        oracle.ref_fwd_decay(q, k, v, g[:, :, :4])
