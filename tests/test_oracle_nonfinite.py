"""Non-finite inputs in the oracle: NaN and Inf propagate as the definition
says (LinearTile 1.0.0 README, "How It Works", with the causal running sums of
its "Features" list): a bad query spoils its own row only; a bad key or value
at token s spoils every causal row t >= s and no row before it; a non-causal
pass sees every key, so every row is spoiled; a decode step reads the carried
state, so a non-finite state spoils its outputs."""
import numpy as np
import pytest

import oracle

B, H, Hkv, N, d = 2, 4, 2, 40, 8


def inputs(seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    return q, k, v


def finite_rows(o):
    return np.isfinite(o).all(axis=-1)


@pytest.mark.parametrize("normalise", [1, 0])
def test_nan_query_spoils_its_row_only(normalise):
    q, k, v = inputs(1)
    q[1, 3, 17, 2] = np.nan
    o = oracle.ref_fwd(q, k, v, causal=True, normalise=normalise)
    bad = ~finite_rows(o)
    assert bad[1, 3, 17] and bad.sum() == 1
    clean = oracle.ref_fwd(*inputs(1), causal=True, normalise=normalise)
    ok = finite_rows(o)
    assert np.array_equal(o[ok], clean[ok])


@pytest.mark.parametrize("what,val", [("k", np.nan), ("v", np.nan), ("v", np.inf), ("k", np.inf)])
@pytest.mark.parametrize("normalise", [1, 0])
def test_bad_key_or_value_spoils_later_rows(what, val, normalise):
    q, k, v = inputs(2)
    s = 23
    (k if what == "k" else v)[0, 1, s, 5] = val
    o = oracle.ref_fwd(q, k, v, causal=True, normalise=normalise)
    fin = finite_rows(o)
    heads = slice(2, 4)  # query heads of kv head 1
    clean = oracle.ref_fwd(*inputs(2), causal=True, normalise=normalise)
    # before s: finite and unchanged, in every head; other kv groups untouched
    assert fin[0, heads, :s].all()
    assert np.array_equal(o[0, heads, :s], clean[0, heads, :s])
    assert np.array_equal(o[:, :2], clean[:, :2]) and np.array_equal(o[1], clean[1])
    # from s on every row of the group is non-finite (an infinite key feature
    # makes a normalised row inf / inf = NaN, an unnormalised one inf)
    assert (~fin[0, heads, s:]).all()


def test_noncausal_bad_key_spoils_every_row_of_its_group():
    q, k, v = inputs(3)
    k[1, 0, 31, 0] = np.nan
    o = oracle.ref_fwd(q, k, v, causal=False, normalise=True)
    fin = finite_rows(o)
    assert (~fin[1, :2]).all() and fin[1, 2:].all() and fin[0].all()


def test_decode_with_nonfinite_state():
    rng = np.random.default_rng(4)
    S = rng.standard_normal((1, 1, d, d))
    z = np.abs(rng.standard_normal((1, 1, d))) + 1.0
    S[0, 0, 3, 4] = np.inf
    q, k, v = rng.standard_normal((1, 2, d)), rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))
    o = oracle.ref_decode_step(S, z, q, k, v, normalise=True)
    # phi(q) > 0 weights every state row, so column 4 is infinite in both heads; the others stay finite
    assert np.isinf(o[0, :, 4]).all() and np.isfinite(np.delete(o[0], 4, axis=-1)).all()
    S[0, 0, 3, 4] = np.nan
    o = oracle.ref_decode_step(S, z, q, k, v, normalise=True)
    assert np.isnan(o[0, :, 4]).all()


@pytest.mark.parametrize("phi_map", ["elu1", "relu", "softplus"])
def test_feature_maps_keep_nan(phi_map):
    assert np.isnan(oracle.phi(float("nan"), phi_map))
    assert np.isnan(oracle.dphi(float("nan"), phi_map))
    assert oracle.phi(float("inf"), phi_map) == float("inf")
    assert oracle.phi(float("-inf"), phi_map) == 0.0
