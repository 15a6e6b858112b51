"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: a library
routine (torch's ELU), a different route to the same quantity (the quadratic
masked attention form, the cumulative sum of outer products), exact rational
arithmetic, closed forms, and invariants the method implies.  Together they
are chosen so that a plausible slip in the oracle (a dropped term, a wrong
index, an exclusive instead of inclusive mask, a different head map, a
transposed state) fails at least one of them; ``test_oracle_mutants.py``
plants such slips and checks that they are caught.

Method: LinearTile 1.0.0 README, "How It Works" (O = phi(Q)(phi(K)^T V),
phi = ELU + 1) and the causal / GQA items of its "Features" list.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import oracle
from linattn_inputs import make_qkv, randn

REL = 1e-12


def phi_lib(x: np.ndarray) -> np.ndarray:
    """phi via torch's ELU (alpha = 1) plus one, in fp64 - the library route."""
    return (F.elu(torch.from_numpy(np.asarray(x, dtype=np.float64)), alpha=1.0) + 1.0).numpy()


def quadratic_form(q, k, v, causal, normalise):
    """Brute force: (M * phi(Q) phi(K)^T) V with M the inclusive causal mask (or all ones)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    out = np.zeros_like(q)
    mask = np.tril(np.ones((N, N))) if causal else np.ones((N, N))
    for b in range(B):
        for h in range(H):
            g = h // G
            A = (phi_lib(q[b, h]) @ phi_lib(k[b, g]).T) * mask
            num = A @ v[b, g]
            out[b, h] = num / A.sum(axis=1, keepdims=True) if normalise else num
    return out


def within_rounding_bound(got, ref, q, k, v, causal, normalise):
    """True when |got - ref| stays under the forward error bound of the sums involved.

    Both routes add the same N products phi(q).phi(k) v (each a d-term dot
    product) in different orders, so in fp64 they may differ by about
    (N + d) eps times the sum of the terms' magnitudes (the standard bound for
    recursive summation, Higham, Accuracy and Stability of Numerical
    Algorithms, ch. 3-4).  That magnitude is the same form taken with |v|; a
    relative test against the row maximum alone fails rows that cancel.
    """
    N, d = q.shape[2], q.shape[3]
    scale = quadratic_form(q, k, np.abs(v), causal, normalise)
    bound = 4 * (N + d + 4) * np.finfo(np.float64).eps * scale + 1e-300
    return bool(np.all(np.abs(np.asarray(got) - ref) <= bound))


def cumsum_form(q, k, v, normalise):
    """Brute force, second route: S_t as the running sum of outer products phi(k_s) v_s^T."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, H, N, d = q.shape
    G = H // k.shape[1]
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            fk = phi_lib(k[b, h // G])
            S = np.cumsum(np.einsum("ti,tj->tij", fk, v[b, h // G]), axis=0)
            z = np.cumsum(fk, axis=0)
            fq = phi_lib(q[b, h])
            num = np.einsum("ti,tij->tj", fq, S)
            out[b, h] = num / np.einsum("ti,ti->t", fq, z)[:, None] if normalise else num
    return out


def rel_err(a, b):
    """Max over rows of max_j |a - b| / max_j |b| (absolute where a row of b is all zero)."""
    a = np.asarray(a, dtype=np.float64).reshape(-1, np.shape(a)[-1])
    b = np.asarray(b, dtype=np.float64).reshape(-1, np.shape(b)[-1])
    den = np.abs(b).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(a - b).max(axis=1) / den).max()) if a.size else 0.0


# ---------------------------------------------------------------- feature map

def test_phi_matches_library_elu():
    xs = np.concatenate([np.linspace(-40, 40, 4001), [0.0, -0.0, 1e-300, -1e-300, 5e-324, 1e-8, -1e-8]])
    ref = phi_lib(xs)
    got = np.array([oracle.phi(x) for x in xs])
    # torch forms exp(x) - 1 and adds 1 back, which costs absolute (not relative)
    # accuracy for very negative x; compare with both bounds.
    assert np.all(np.abs(got - ref) <= 1e-15 * np.abs(ref) + 4e-16)


def test_phi_positive_and_continuous():
    xs = np.linspace(-30, 30, 601)
    vals = np.array([oracle.phi(x) for x in xs])
    assert np.all(vals > 0)
    assert oracle.phi(0.0) == 1.0 and oracle.phi(-0.0) == 1.0
    assert abs(oracle.phi(1e-12) - 1.0) < 1e-11 and abs(oracle.phi(-1e-12) - 1.0) < 1e-11
    assert np.all(np.diff(vals) > 0)  # phi is strictly increasing


# ------------------------------------------------------- brute-force routes

shapes = st.tuples(
    st.integers(1, 2),            # B
    st.sampled_from([(1, 1), (2, 2), (2, 1), (4, 2), (3, 3), (6, 2)]),  # (H, Hkv)
    st.integers(1, 64),           # N
    st.sampled_from([1, 2, 4, 8, 32]),  # d
    st.integers(0, 2**31 - 1),    # seed
)


@settings(max_examples=40, deadline=None)
@given(shapes, st.booleans(), st.booleans())
def test_oracle_equals_quadratic_masked_form(shape, causal, normalise):
    B, (H, Hkv), N, d, seed = shape
    q, k, v = make_qkv(B, H, Hkv, N, d, "f32", seed)
    got = oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise, nthreads=2)
    ref = quadratic_form(q, k, v, causal, normalise)
    assert within_rounding_bound(got, ref, q, k, v, causal, normalise)


@settings(max_examples=25, deadline=None)
@given(shapes, st.booleans())
def test_oracle_equals_cumsum_of_outer_products(shape, normalise):
    B, (H, Hkv), N, d, seed = shape
    q, k, v = make_qkv(B, H, Hkv, N, d, "f32", seed)
    got = oracle.ref_fwd(q, k, v, causal=True, normalise=normalise, nthreads=2)
    assert within_rounding_bound(got, cumsum_form(q, k, v, normalise), q, k, v, True, normalise)


@pytest.mark.parametrize("normalise", [True, False])
def test_config1_full_against_quadratic_form(normalise):
    """The small fp32 workload (B1 H2 N256 d32) in full."""
    q, k, v = make_qkv(1, 2, 2, 256, 32, "f32", 1001)
    got = oracle.ref_fwd(q, k, v, causal=True, normalise=normalise)
    assert rel_err(got, quadratic_form(q, k, v, True, normalise)) <= REL


def test_bf16_inputs_are_read_exactly():
    q, k, v = make_qkv(1, 2, 1, 40, 8, "bf16", 7)
    got = oracle.ref_fwd(q, k, v)
    ref = quadratic_form(q.double().numpy(), k.double().numpy(), v.double().numpy(), True, True)
    assert rel_err(got, ref) <= REL


def test_exact_rational_arithmetic():
    """Positive dyadic inputs make phi(x) = x + 1 exact; compare with Fraction arithmetic."""
    rng = np.random.default_rng(3)
    N, d = 7, 3
    q = rng.integers(1, 9, size=(1, 1, N, d)) / 4.0
    k = rng.integers(1, 9, size=(1, 1, N, d)) / 8.0
    v = rng.integers(-8, 9, size=(1, 1, N, d)) / 2.0
    for normalise in (True, False):
        got = oracle.ref_fwd(q, k, v, causal=True, normalise=normalise)
        for t in range(N):
            fq = [Fraction(x) + 1 for x in q[0, 0, t]]
            num = [Fraction(0)] * d
            den = Fraction(0)
            for s in range(t + 1):
                w = sum(a * (Fraction(b) + 1) for a, b in zip(fq, k[0, 0, s]))
                den += w
                num = [n + w * Fraction(x) for n, x in zip(num, v[0, 0, s])]
            exact = [n / den for n in num] if normalise else num
            for j in range(d):
                assert abs(got[0, 0, t, j] - float(exact[j])) <= 1e-15 * max(1.0, abs(float(exact[j])))


# ---------------------------------------------------- associativity (non-causal)

@pytest.mark.parametrize("seed", [11, 12, 13])
def test_noncausal_associativity(seed):
    """(phi(Q) phi(K)^T) V == phi(Q) (phi(K)^T V) and rowsum(phi(Q)phi(K)^T) == phi(Q) . z_N."""
    q, k, v = make_qkv(2, 4, 2, 50, 8, "f32", seed)
    out, S, z = oracle.ref_fwd(q, k, v, causal=False, normalise=False, want_state=True)
    qq, kk, vv = (t.double().numpy() for t in (q, k, v))
    for b in range(2):
        for h in range(4):
            g = h // 2
            A = phi_lib(qq[b, h]) @ phi_lib(kk[b, g]).T
            assert rel_err(out[b, h], A @ vv[b, g]) <= REL
            assert np.allclose(A.sum(axis=1), phi_lib(qq[b, h]) @ z[b, g], rtol=1e-13, atol=0)
    outn = oracle.ref_fwd(q, k, v, causal=False, normalise=True)
    assert rel_err(outn, quadratic_form(q, k, v, False, True)) <= REL


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("normalise", [True, False])
def test_zero_keys_give_prefix_mean(normalise):
    """K = 0 makes phi(k) = 1: normalised o_t is the mean of v_0..v_t, independent of Q;
    unnormalised o_t is (sum_i phi(q_t)_i) * sum_{s<=t} v_s."""
    N, d = 33, 4
    q = randn((1, 1, N, d), 5).double().numpy()
    v = randn((1, 1, N, d), 6).double().numpy()
    k = np.zeros_like(v)
    got = oracle.ref_fwd(q, k, v, causal=True, normalise=normalise)[0, 0]
    csum = np.cumsum(v[0, 0], axis=0)
    if normalise:
        ref = csum / np.arange(1, N + 1)[:, None]
    else:
        ref = phi_lib(q[0, 0]).sum(axis=1, keepdims=True) * csum
    assert rel_err(got, ref) <= REL


def test_noncausal_zero_keys_give_global_mean():
    q = randn((1, 2, 20, 4), 8).double().numpy()
    v = randn((1, 2, 20, 4), 9).double().numpy()
    got = oracle.ref_fwd(q, np.zeros_like(v), v, causal=False, normalise=True)
    assert rel_err(got, np.broadcast_to(v.mean(axis=2, keepdims=True), got.shape)) <= REL


def test_single_token_returns_its_value():
    q, k, v = make_qkv(2, 4, 2, 1, 8, "f32", 21)
    got = oracle.ref_fwd(q, k, v, causal=True, normalise=True)
    ref = torch.repeat_interleave(v, 2, dim=1).double().numpy()
    assert rel_err(got, ref) <= REL


def test_d1_is_weighted_prefix_mean():
    """With d = 1, phi(q_t) cancels: o_t = sum_{s<=t} phi(k_s) v_s / sum_{s<=t} phi(k_s)."""
    q, k, v = make_qkv(1, 1, 1, 30, 1, "f32", 22)
    got = oracle.ref_fwd(q, k, v, causal=True, normalise=True)[0, 0, :, 0]
    fk = phi_lib(k.double().numpy()[0, 0, :, 0])
    vv = v.double().numpy()[0, 0, :, 0]
    ref = np.cumsum(fk * vv) / np.cumsum(fk)
    assert np.allclose(got, ref, rtol=1e-13, atol=0)


# --------------------------------------------------------------- invariants

def test_z_strictly_increasing_and_state_is_phiK_T_V():
    q, k, v = make_qkv(1, 2, 2, 24, 8, "f32", 31)
    prev = None
    for n in range(1, 25):
        _, S, z = oracle.ref_fwd(q[:, :, :n], k[:, :, :n], v[:, :, :n], want_state=True)
        fk = phi_lib(k.double().numpy()[:, :, :n])
        assert np.allclose(S, np.einsum("bgti,bgtj->bgij", fk, v.double().numpy()[:, :, :n]),
                           rtol=1e-13, atol=1e-13)
        assert np.allclose(z, fk.sum(axis=2), rtol=1e-14, atol=0)
        if prev is not None:
            assert np.all(z > prev)
        prev = z


def test_normalised_rows_are_convex_combinations():
    q, k, v = make_qkv(1, 2, 2, 64, 8, "f32", 32)
    got = oracle.ref_fwd(q, k, v, causal=True, normalise=True)
    vv = v.double().numpy()
    lo = np.minimum.accumulate(vv, axis=2)
    hi = np.maximum.accumulate(vv, axis=2)
    assert np.all(got >= lo - 1e-12) and np.all(got <= hi + 1e-12)


def test_shift_equivariance():
    q, k, v = make_qkv(1, 2, 1, 40, 8, "f32", 33)
    a = oracle.ref_fwd(q, k, v)
    b = oracle.ref_fwd(q, k, v.double() + 2.5)
    assert np.allclose(b, a + 2.5, rtol=0, atol=1e-12)


def test_causality_is_bitwise():
    q, k, v = make_qkv(1, 2, 2, 48, 8, "f32", 34)
    a = oracle.ref_fwd(q, k, v)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[:, :, 30:] += 3.0
    k2[:, :, 30:] -= 2.0
    v2[:, :, 30:] *= -5.0
    b = oracle.ref_fwd(q2, k2, v2)
    assert np.array_equal(a[:, :, :30], b[:, :, :30])
    assert not np.array_equal(a[:, :, 30:], b[:, :, 30:])


def test_last_causal_row_equals_noncausal_row():
    q, k, v = make_qkv(2, 2, 2, 37, 8, "f32", 35)
    for normalise in (True, False):
        c = oracle.ref_fwd(q, k, v, causal=True, normalise=normalise)
        n = oracle.ref_fwd(q, k, v, causal=False, normalise=normalise)
        assert rel_err(c[:, :, -1], n[:, :, -1]) <= REL


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = make_qkv(2, 8, 2, 40, 8, "f32", 36)
    G = 4
    a = oracle.ref_fwd(q, k, v)
    b = oracle.ref_fwd(q, torch.repeat_interleave(k, G, dim=1), torch.repeat_interleave(v, G, dim=1))
    assert np.array_equal(a, b)


# ------------------------------------------------------------------- decode

@pytest.mark.parametrize("normalise", [True, False])
def test_decode_continues_prefill(normalise):
    """Prefill(N) then decode steps N..N+m-1 reproduces rows N..N+m-1 of prefill(N+m)."""
    B, H, Hkv, N, d, m = 2, 4, 2, 20, 8, 5
    q, k, v = make_qkv(B, H, Hkv, N + m, d, "f32", 41)
    full = oracle.ref_fwd(q, k, v, causal=True, normalise=normalise)
    _, S, z = oracle.ref_fwd(q[:, :, :N], k[:, :, :N], v[:, :, :N], want_state=True)
    for t in range(N, N + m):
        o = oracle.ref_decode_step(S, z if normalise else None, q[:, :, t], k[:, :, t], v[:, :, t],
                                   normalise=normalise)
        assert rel_err(o, full[:, :, t]) <= REL


def test_decode_from_zero_state_is_prefill():
    B, H, Hkv, N, d = 1, 2, 1, 12, 4
    q, k, v = make_qkv(B, H, Hkv, N, d, "f32", 42)
    full = oracle.ref_fwd(q, k, v)
    S = np.zeros((B, Hkv, d, d))
    z = np.zeros((B, Hkv, d))
    for t in range(N):
        o = oracle.ref_decode_step(S, z, q[:, :, t], k[:, :, t], v[:, :, t])
        assert rel_err(o, full[:, :, t]) <= REL


# ---------------------------------------------------------------- arguments

def test_rejects_bad_head_split():
    q, k, v = make_qkv(1, 3, 2, 4, 4, "f32", 1)
    with pytest.raises(ValueError):
        oracle.ref_fwd(q, k, v)


def test_empty_sequence():
    q, k, v = make_qkv(1, 2, 2, 0, 4, "f32", 1)
    out, S, z = oracle.ref_fwd(q, k, v, want_state=True)
    assert out.shape == (1, 2, 0, 4) and not S.any() and not z.any()



# ------------------------------------------------------------- continuation

@settings(max_examples=25, deadline=None)
@given(shapes, st.booleans(), st.booleans(), st.floats(0.0, 1.0))
def test_continuation_from_state_equals_one_pass(shape, causal, normalise, frac):
    """Split a sequence anywhere: the second part run from the first part's
    (S, z) reproduces the one-pass rows, state and normaliser (the plain
    oracle being pinned above, this pins the continuation against it)."""
    B, (H, Hkv), N, d, seed = shape
    q, k, v = make_qkv(B, H, Hkv, N, d, "f32", seed)
    n1 = int(round(frac * N))
    whole, S, z = oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise, want_state=True, nthreads=2)
    _, S1, z1 = oracle.ref_fwd(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], causal=True, want_state=True, nthreads=2)
    o2, S2, z2 = oracle.ref_fwd(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], causal=causal, normalise=normalise,
                                want_state=True, nthreads=2, state_in=S1, z_in=z1)
    # The continuation performs the same additions in the same order as the
    # one-pass run, so the match is exact.
    assert np.array_equal(o2, whole[:, :, n1:])
    assert np.array_equal(S2, S) and np.array_equal(z2, z)


def test_continuation_from_zero_state_is_the_plain_pass():
    q, k, v = make_qkv(2, 4, 2, 37, 8, "f32", 5)
    Hkv, d = 2, 8
    plain = oracle.ref_fwd(q, k, v)
    from_zero = oracle.ref_fwd(q, k, v, state_in=np.zeros((2, Hkv, d, d)), z_in=np.zeros((2, Hkv, d)))
    assert np.array_equal(plain, from_zero)


def test_continuation_closed_form_constant_keys():
    """K = 0 (phi(k) = 1) after a start state (S0, z0): o_t = (phi(q_t)^T S0 + sum_{s<=t} v_s (phi(q_t).1))
    / (phi(q_t) . z0 + t |phi(q_t)|_1)."""
    rng = np.random.default_rng(11)
    B, H, N, d = 1, 1, 9, 4
    q = rng.standard_normal((B, H, N, d))
    v = rng.standard_normal((B, H, N, d))
    k = np.zeros((B, H, N, d))
    S0 = rng.random((B, H, d, d))
    z0 = rng.random((B, H, d)) + 0.5
    got = oracle.ref_fwd(q, k, v, state_in=S0, z_in=z0)
    fq = phi_lib(q[0, 0])
    cs = np.cumsum(v[0, 0], axis=0)
    for t in range(N):
        l1 = fq[t].sum()
        num = fq[t] @ S0[0, 0] + cs[t] * l1
        den = fq[t] @ z0[0, 0] + (t + 1) * l1
        assert np.allclose(got[0, 0, t], num / den, rtol=1e-13, atol=0)
