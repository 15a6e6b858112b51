"""GPU parity: the HIP library (called through the C ABI) against the fp64 oracle.

Bar (per output row r = (b, h, t)): e_r = max_j |O_gpu - O_ref| / max_j |O_ref|
must be <= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs with fp32
accumulation.  States and normalisers use the same metric per matrix / vector.

Sizes: small ragged shapes in full (several chunks, segments and a ragged
tail), every workload at its full size, with the oracle evaluated on sampled
(batch, kv head) sequences where a full oracle run would take minutes.
"""
import numpy as np
import pytest
import torch

import oracle
import sequence_mixing_amd as la
from linattn_inputs import DECODE, WORKLOADS, DecodeStream, make_qkv, workload_qkv
from sequence_mixing_amd import ops

pytestmark = pytest.mark.gpu

# fp16 rows enter the matrix cores as bf16 (fp16 only at the loads and
# stores), so they share bf16's bar.
TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 2e-2}


def rows_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    if g.size == 0:
        return 0.0
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(g - r).max(axis=1) / den).max())


def mat_rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    lead = got.shape[:2]
    g = got.reshape(int(np.prod(lead)), -1)
    r = ref.reshape(int(np.prod(lead)), -1)
    den = np.abs(r).max(axis=1)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(g - r).max(axis=1) / den).max())


def gpu(t):
    return t.contiguous().cuda()


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run_case(B, H, Hkv, N, d, dtype, causal, normalise, chunk=0, seed=0, check_state=True):
    q, k, v = make_qkv(B, H, Hkv, N, d, dtype, seed)
    print(f"case B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype} causal={causal} norm={normalise} chunk={chunk} seed={seed}",
          flush=True)
    out, S, z = ops.fwd(gpu(q), gpu(k), gpu(v), causal=causal, normalise=normalise, chunk=chunk, want_state=True)
    torch.cuda.synchronize()
    ref, Sr, zr = oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise, want_state=True)
    tol = TOL[dtype]
    e = rows_rel_err(host(out), ref)
    assert e <= tol, f"output rel err {e:.3e} > {tol}"
    if check_state and N > 0:
        es, ez = mat_rel_err(host(S), Sr), mat_rel_err(host(z), zr)
        assert es <= tol and ez <= tol, f"state rel err {es:.3e}, z rel err {ez:.3e}"
    return e


# ------------------------------------------------------------- small shapes

SMALL = [
    # B, H, Hkv, N, d, dtype
    (1, 2, 2, 256, 32, "f32"),
    (1, 1, 1, 1, 64, "f32"),
    (2, 2, 2, 7, 64, "bf16"),
    (1, 2, 1, 100, 64, "f32"),
    (2, 4, 2, 257, 64, "bf16"),
    (1, 4, 4, 1000, 32, "bf16"),
    (1, 4, 1, 333, 128, "bf16"),
    (1, 2, 2, 300, 128, "f32"),
    (3, 6, 3, 515, 64, "f32"),
    (1, 8, 2, 2049, 128, "bf16"),
    (2, 6, 2, 300, 64, "bf16"),     # G = 3: three one-head blocks per kv head
    (1, 6, 1, 777, 64, "bf16"),     # G = 6: head blocks of 2
    (1, 8, 1, 500, 64, "f32"),      # G = 8
    (1, 16, 2, 333, 128, "bf16"),   # G = 8 at d = 128: head blocks of 4
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dH%dK%dN%dd%d%s" % s)
@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_small_shapes(shape, causal, normalise):
    B, H, Hkv, N, d, dtype = shape
    run_case(B, H, Hkv, N, d, dtype, causal, normalise, seed=N + d)


@pytest.mark.parametrize("chunk", [32, 64, 128, 256])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_chunk_size(chunk, dtype):
    rc, _, _ = la.linattn_fwd_plan(2, 4, 2, 1100, 64, 1, ops.dtype_code(getattr(torch, {"f32": "float32", "bf16": "bfloat16"}[dtype])), chunk)
    if rc != 0:
        pytest.skip("chunk does not fit LDS for this dtype")
    run_case(2, 4, 2, 1100, 64, dtype, 1, 1, chunk=chunk, seed=chunk)


def test_config1_full():
    w = WORKLOADS["cfg1"]
    for normalise in (1, 0):
        for chunk in (0, 32, 64, 128, 256):
            run_case(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, 1, normalise, chunk=chunk, seed=w.seed)


def test_empty_and_zero_batch():
    q = torch.zeros(1, 2, 0, 64, device="cuda")
    out, S, z = ops.fwd(q, q.clone(), q.clone(), want_state=True)
    torch.cuda.synchronize()
    assert out.shape == (1, 2, 0, 64) and not S.any() and not z.any()
    q = torch.zeros(0, 2, 16, 64, device="cuda")
    assert ops.fwd(q, q.clone(), q.clone()).shape == (0, 2, 16, 64)


# ------------------------------------------------------- workloads, full size

@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_config2_full(causal, normalise):
    w = WORKLOADS["cfg2"]
    run_case(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, causal, normalise, seed=w.seed)


@pytest.mark.parametrize("normalise", [1, 0])
def test_config3_full(normalise):
    w = WORKLOADS["cfg3"]
    run_case(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, 1, normalise, seed=w.seed)


def full_check(w, out, S, z, ref, Sr, zr, label):
    """Every output row, state and normaliser of a full-size workload against the oracle."""
    tol = TOL[w.dtype]
    e = rows_rel_err(host(out), ref)
    es, ez = mat_rel_err(host(S), Sr), mat_rel_err(host(z), zr)
    print(f"  {label}: out {e:.2e} state {es:.2e} z {ez:.2e}", flush=True)
    assert e <= tol and es <= tol and ez <= tol, f"{label}: out {e:.3e} state {es:.3e} z {ez:.3e}"


_REF_CACHE = {}


def workload_ref(name, normalise):
    """The oracle's rows and final sums for a whole workload (every batch entry and kv head),
    computed once per (workload, normaliser) and shared by the chunk sizes."""
    key = (name, normalise)
    if key not in _REF_CACHE:
        for other in [k_ for k_ in _REF_CACHE if k_[0] != name]:
            del _REF_CACHE[other]  # the references of one workload held at a time
        q, k, v = workload_qkv(WORKLOADS[name])
        _REF_CACHE[key] = oracle.ref_fwd(q, k, v, causal=True, normalise=normalise, want_state=True)
    return _REF_CACHE[key]


@pytest.mark.parametrize("normalise", [1, 0])
@pytest.mark.parametrize("chunk", [64, 128, 256])
def test_config4_full(chunk, normalise):
    """bf16 B2 H8 N65536 d64 at every chunk size and both normaliser settings, all 16 sequences."""
    w = WORKLOADS["cfg4"]
    q, k, v = workload_qkv(w)
    print(f"cfg4 chunk={chunk} normalise={normalise}", flush=True)
    out, S, z = ops.fwd(gpu(q), gpu(k), gpu(v), causal=True, normalise=normalise, chunk=chunk, want_state=True)
    torch.cuda.synchronize()
    del q, k, v
    ref, Sr, zr = workload_ref("cfg4", normalise)
    full_check(w, out, S, z, ref, Sr, zr, f"cfg4 chunk {chunk} normalise {normalise}")


@pytest.mark.parametrize("normalise", [1, 0])
def test_config5_prefill_full(normalise):
    """GQA bf16 B1 H32 Hkv8 N32768 d128, both normaliser settings, all 8 kv heads and 32 query heads."""
    w = WORKLOADS["cfg5"]
    q, k, v = workload_qkv(w)
    print(f"cfg5 prefill normalise={normalise}", flush=True)
    out, S, z = ops.fwd(gpu(q), gpu(k), gpu(v), causal=True, normalise=normalise, want_state=True)
    torch.cuda.synchronize()
    del q, k, v
    ref, Sr, zr = workload_ref("cfg5", normalise)
    full_check(w, out, S, z, ref, Sr, zr, f"cfg5 prefill normalise {normalise}")


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("normalise", [1, 0])
def test_decode_step_same_start_state(dtype, d, normalise):
    """The decode kernel against the oracle from an identical (nonzero) start state."""
    B, H, Hkv = 3, 8, 2
    q0, k0, v0 = make_qkv(B, Hkv, Hkv, 50, d, dtype, 77 + d)
    _, S, z = ops.fwd(gpu(q0), gpu(k0), gpu(v0), want_state=True)
    Sr, zr = host(S).copy(), host(z).copy()
    stream = DecodeStream(B, H, Hkv, d, dtype, 5 + d)
    for step in range(4):
        q, k, v = stream.next()
        o = ops.decode_step(S, z if normalise else None, gpu(q), gpu(k), gpu(v), normalise=normalise)
        ref = oracle.ref_decode_step(Sr, zr if normalise else None, q, k, v, normalise=normalise)
        torch.cuda.synchronize()
        tol = 1e-5 if dtype == "f32" else TOL[dtype]
        assert rows_rel_err(host(o), ref) <= tol
        assert mat_rel_err(host(S), Sr) <= 1e-5
        if normalise:
            assert mat_rel_err(host(z), zr) <= 1e-6


@pytest.mark.parametrize("B,H,Hkv,d,dtype", [(2, 40, 1, 128, "bf16"), (3, 6, 2, 64, "f32"), (1, 3, 3, 32, "bf16"),
                                              (2, 70, 2, 64, "bf16")])
def test_decode_step_head_groups(B, H, Hkv, d, dtype):
    """Query-head groups that are not a multiple of 4, or larger than one staging pass (32 heads)."""
    q0, k0, v0 = make_qkv(B, Hkv, Hkv, 20, d, dtype, 31 + H)
    _, S, z = ops.fwd(gpu(q0), gpu(k0), gpu(v0), want_state=True)
    Sr, zr = host(S).copy(), host(z).copy()
    stream = DecodeStream(B, H, Hkv, d, dtype, 9 + H)
    for step in range(3):
        q, k, v = stream.next()
        o = ops.decode_step(S, z, gpu(q), gpu(k), gpu(v))
        ref = oracle.ref_decode_step(Sr, zr, q, k, v, normalise=True)
        torch.cuda.synchronize()
        tol = 1e-5 if dtype == "f32" else TOL[dtype]
        assert rows_rel_err(host(o), ref) <= tol
        assert mat_rel_err(host(S), Sr) <= 1e-5
        assert mat_rel_err(host(z), zr) <= 1e-6


@pytest.mark.parametrize("B,H,Hkv,d,dtype,decay", [(1024, 32, 8, 128, "bf16", False), (2050, 16, 8, 64, "f32", False),
                                                    (1024, 8, 8, 128, "bf16", True)])
def test_decode_step_state_beyond_cache(B, H, Hkv, d, dtype, decay):
    """A state larger than the 256 MiB memory-side cache, which the decode kernel streams
    with the non-temporal hint: two steps on the whole batch (plain or decayed sums),
    checked against the oracle on sampled slots (every kv head) and bitwise against the
    same steps taken in pieces of 256 slots (states small enough for the plain path)."""
    assert B * Hkv * d * d * 4 > 256 << 20
    print(f"decode beyond cache B{B} H{H} Hkv{Hkv} d{d} {dtype} decay={decay}", flush=True)
    gen = torch.Generator("cuda").manual_seed(61 + d)
    S = torch.randn(B, Hkv, d, d, device="cuda", generator=gen) * 0.05
    z = torch.rand(B, Hkv, d, device="cuda", generator=gen) + 1.0
    slots = [0, 1, B // 2 + 3, B - 1]
    Sr, zr = host(S[slots]).copy(), host(z[slots]).copy()
    S2, z2 = S.clone(), z.clone()
    stream = DecodeStream(B, H, Hkv, d, dtype, 17 + d)
    for step in range(2):
        q, k, v = stream.next()
        qg, kg, vg = gpu(q), gpu(k), gpu(v)
        g = -torch.rand(B, Hkv, generator=torch.Generator("cpu").manual_seed(step)) if decay else None

        def call(S_, z_, sl):
            a = (S_, z_, qg[sl].contiguous(), kg[sl].contiguous(), vg[sl].contiguous())
            return ops.decode_step_decay(*a, gpu(g[sl])) if decay else ops.decode_step(*a)

        o = call(S, z, slice(0, B))
        parts = []
        for b0 in range(0, B, 256):
            sl = slice(b0, min(B, b0 + 256))
            Sp, zp = S2[sl].contiguous(), z2[sl].contiguous()
            parts.append(call(Sp, zp, sl))
            S2[sl], z2[sl] = Sp, zp
        if decay:
            ref = oracle.ref_decode_step_decay(Sr, zr, q[slots], k[slots], v[slots], g[slots].numpy())
        else:
            ref = oracle.ref_decode_step(Sr, zr, q[slots], k[slots], v[slots], normalise=True)
        torch.cuda.synchronize()
        assert rows_rel_err(host(o[slots]), ref) <= (1e-5 if dtype == "f32" else TOL[dtype])
        assert torch.equal(o, torch.cat(parts)), f"step {step}: outputs differ from the pieces"
    assert torch.equal(S, S2) and torch.equal(z, z2)
    assert mat_rel_err(host(S[slots]), Sr) <= 1e-5
    assert mat_rel_err(host(z[slots]), zr) <= 1e-6


def test_decode_continues_prefill_on_gpu():
    """Prefill(N) then one decode step equals row N of prefill(N + 1)."""
    B, H, Hkv, N, d = 2, 8, 2, 777, 64
    q, k, v = make_qkv(B, H, Hkv, N + 1, d, "f32", 91)
    full = ops.fwd(gpu(q), gpu(k), gpu(v))
    _, S, z = ops.fwd(gpu(q[:, :, :N]), gpu(k[:, :, :N]), gpu(v[:, :, :N]), want_state=True)
    o = ops.decode_step(S, z, gpu(q[:, :, N]), gpu(k[:, :, N]), gpu(v[:, :, N]))
    torch.cuda.synchronize()
    assert rows_rel_err(host(o), host(full[:, :, N])) <= 1e-4


def test_config5_decode_1024_steps_sampled():
    """GQA prefill, its state replicated into 64 slots, then 1024 decode steps at batch 64.

    The GPU runs the whole batch; the oracle follows slots 0, 31 and 63 with all 8 kv
    heads and all 32 query heads end to end (its own prefill state, its own decode
    steps) over all 1024 steps, and compares their states and normalisers at the end.
    """
    w, dw = WORKLOADS["cfg5"], DECODE
    q, k, v = workload_qkv(w)
    _, S1, z1 = ops.fwd(gpu(q), gpu(k), gpu(v), want_state=True)
    _, Sr1, zr1 = workload_ref("cfg5", 1)
    del q, k, v
    S = S1.expand(dw.B, -1, -1, -1).contiguous()
    z = z1.expand(dw.B, -1, -1).contiguous()
    slots = [0, 31, 63]
    Sr = np.ascontiguousarray(np.repeat(Sr1, len(slots), axis=0))
    zr = np.ascontiguousarray(np.repeat(zr1, len(slots), axis=0))
    stream = DecodeStream(dw.B, dw.H, dw.Hkv, dw.d, dw.dtype, dw.seed)
    worst = 0.0
    for step in range(1024):
        qs, ks, vs = stream.next()
        o = ops.decode_step(S, z, gpu(qs), gpu(ks), gpu(vs))
        ref = oracle.ref_decode_step(Sr, zr, qs[slots], ks[slots], vs[slots], normalise=True)
        e = rows_rel_err(host(o[slots]), ref)
        worst = max(worst, e)
        assert e <= TOL["bf16"], f"step {step}: {e:.3e}"
    torch.cuda.synchronize()
    es, ez = mat_rel_err(host(S[slots]), Sr), mat_rel_err(host(z[slots]), zr)
    print(f"decode worst rel err over 1024 steps: {worst:.3e}; final state {es:.2e}, z {ez:.2e}", flush=True)
    # the start sums are the bf16 prefill's (phi(k) rounded to bf16 at the matrix core)
    assert es <= TOL["bf16"] and ez <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_unnormalised_steps_advance_z(dtype):
    """Steps with normalise = 0 and z given advance z, so a later normalised step (and a
    continued prefill) read the whole sums: three unnormalised steps, then a normalised one."""
    B, H, Hkv, d = 2, 8, 2, 64
    q0, k0, v0 = make_qkv(B, Hkv, Hkv, 40, d, dtype, 123)
    _, S, z = ops.fwd(gpu(q0), gpu(k0), gpu(v0), want_state=True)
    Sr, zr = host(S).copy(), host(z).copy()
    stream = DecodeStream(B, H, Hkv, d, dtype, 321)
    tol = 1e-5 if dtype == "f32" else TOL[dtype]
    for step, normalise in enumerate((0, 0, 0, 1)):
        q, k, v = stream.next()
        o = ops.decode_step(S, z, gpu(q), gpu(k), gpu(v), normalise=normalise)
        ref = oracle.ref_decode_step(Sr, zr, q, k, v, normalise=normalise)
        torch.cuda.synchronize()
        e = rows_rel_err(host(o), ref)
        assert e <= tol, f"step {step} normalise {normalise}: {e:.3e}"
        assert mat_rel_err(host(S), Sr) <= 1e-5
        assert mat_rel_err(host(z), zr) <= 1e-6, f"step {step}: z not advanced"


# ---------------------------------------------------------- structure on GPU

def test_causality_bitwise():
    q, k, v = make_qkv(1, 4, 2, 1500, 64, "bf16", 5)
    a = ops.fwd(gpu(q), gpu(k), gpu(v))
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[:, :, 900:] = 3.0
    k2[:, :, 900:] = -1.0
    v2[:, :, 900:] = 7.0
    b = ops.fwd(gpu(q2), gpu(k2), gpu(v2))
    torch.cuda.synchronize()
    assert torch.equal(a[:, :, :900], b[:, :, :900])


def test_deterministic():
    q, k, v = make_qkv(2, 8, 8, 4096, 64, "bf16", 6)
    a = ops.fwd(gpu(q), gpu(k), gpu(v))
    b = ops.fwd(gpu(q), gpu(k), gpu(v))
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_gqa_matches_repeated_kv():
    q, k, v = make_qkv(1, 8, 2, 1000, 64, "f32", 8)
    a = ops.fwd(gpu(q), gpu(k), gpu(v))
    b = ops.fwd(gpu(q), gpu(torch.repeat_interleave(k, 4, dim=1)), gpu(torch.repeat_interleave(v, 4, dim=1)))
    torch.cuda.synchronize()
    assert rows_rel_err(host(a), host(b)) <= 1e-5


def test_chunk_invariance():
    q, k, v = make_qkv(2, 8, 8, 3000, 64, "bf16", 9)
    outs = [host(ops.fwd(gpu(q), gpu(k), gpu(v), chunk=c)) for c in (64, 128, 256)]
    for o in outs[1:]:
        assert rows_rel_err(o, outs[0]) <= 2e-2


@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("d,G", [(64, 1), (128, 4)])
def test_fp32_kernel_vs_bf16_kernel(causal, d, G):
    # bf16-representable inputs: the fp32 path reads them exactly, so the two
    # kernels differ only by the bf16 path's operand and output roundings
    q, k, v = make_qkv(2, 2 * G, 2, 1500, d, "bf16", 12 + d)
    o16 = host(ops.fwd(gpu(q), gpu(k), gpu(v), causal=causal))
    o32 = host(ops.fwd(gpu(q.float()), gpu(k.float()), gpu(v.float()), causal=causal))
    torch.cuda.synchronize()
    ref = oracle.ref_fwd(q, k, v, causal=causal)
    assert rows_rel_err(o32, ref) <= TOL["f32"]
    assert rows_rel_err(o16, ref) <= TOL["bf16"]
    assert rows_rel_err(o16, o32) <= TOL["bf16"]


def test_last_causal_row_equals_noncausal():
    q, k, v = make_qkv(2, 4, 2, 999, 64, "f32", 10)
    c = ops.fwd(gpu(q), gpu(k), gpu(v), causal=True)
    n = ops.fwd(gpu(q), gpu(k), gpu(v), causal=False)
    torch.cuda.synchronize()
    assert rows_rel_err(host(c[:, :, -1]), host(n[:, :, -1])) <= 1e-4


@pytest.mark.parametrize("causal", [1, 0])
def test_timed_entry_point_with_repeats_matches_plain_call(causal):
    """linattn_fwd_timed (last stage launched 3 times) leaves exactly the output of linattn_fwd; with 0
    launches of the last stage it leaves the output untouched."""
    B, H, Hkv, N, d = 2, 8, 2, 900, 64
    q, k, v = (t.contiguous().cuda() for t in make_qkv(B, H, Hkv, N, d, "bf16", 333))
    ref, S_ref, z_ref = ops.fwd(q, k, v, causal=causal, want_state=True)
    out = torch.empty_like(q)
    S = torch.empty_like(S_ref)
    z = torch.empty_like(z_ref)
    ws = ops.workspace(B, H, Hkv, N, d, causal, q.dtype)
    nbytes = ws.numel() * 4 if ws is not None else 0
    hip = __import__("ctypes").CDLL("libamdhip64.so")
    evs = []
    for _ in range(4):
        e = __import__("ctypes").c_void_p()
        assert hip.hipEventCreate(__import__("ctypes").byref(e)) == 0
        evs.append(e.value)
    rc = la.linattn_fwd_timed(q, k, v, out, B, H, Hkv, N, d, causal, 1, la.LINATTN_BF16, S, z, 0, ws, nbytes,
                              None, events=evs, reps=3)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(S, S_ref) and torch.equal(z, z_ref)
    # reps = 0: the first two stages only, the output is left as it was
    out.fill_(7.0)
    assert la.linattn_fwd_timed(q, k, v, out, B, H, Hkv, N, d, causal, 1, la.LINATTN_BF16, S, z, 0, ws, nbytes,
                                None, events=evs, reps=0) == 0
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    assert la.linattn_fwd_timed(q, k, v, out, B, H, Hkv, N, d, causal, 1, la.LINATTN_BF16, S, z, 0, ws, nbytes,
                                None, events=evs, reps=-1) == -2


# ------------------------------------------- continuing from given start sums

def start_sums(B, Hkv, d, dtype, seed, n_prefix=300):
    """Sums of a seeded prefix of n_prefix tokens (oracle, fp64), rounded to fp32 for both sides."""
    qp, kp, vp = make_qkv(B, Hkv, Hkv, n_prefix, d, dtype, seed)
    _, S, z = oracle.ref_fwd(qp, kp, vp, causal=True, want_state=True)
    return torch.from_numpy(S).float(), torch.from_numpy(z).float()


@pytest.mark.parametrize("B,H,Hkv,N,d,dtype,chunk", [
    (1, 2, 2, 100, 64, "f32", 0),
    (2, 4, 2, 257, 64, "bf16", 0),
    (1, 4, 1, 333, 128, "bf16", 0),
    (1, 8, 2, 2049, 128, "bf16", 0),
    (3, 6, 3, 515, 64, "f32", 32),
    (1, 2, 2, 1, 32, "f32", 0),
    (2, 8, 8, 1000, 32, "bf16", 64),
    (1, 16, 2, 700, 128, "bf16", 0),
])
@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_continuation_matches_oracle(B, H, Hkv, N, d, dtype, chunk, causal, normalise):
    q, k, v = make_qkv(B, H, Hkv, N, d, dtype, 71 + N)
    S0, z0 = start_sums(B, Hkv, d, dtype, 5 + d)
    rc, c, P = la.linattn_fwd_plan(B, H, Hkv, N, d, causal, ops.dtype_code(q.dtype), chunk)
    print(f"continuation B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype} causal={causal} norm={normalise} "
          f"chunk={c} segments={P}", flush=True)
    assert rc == 0
    out, S, z = ops.fwd(gpu(q), gpu(k), gpu(v), causal=causal, normalise=normalise, chunk=chunk, want_state=True,
                        state_in=gpu(S0), z_in=gpu(z0) if normalise else None)
    torch.cuda.synchronize()
    ref, Sr, zr = oracle.ref_fwd(q, k, v, causal=causal, normalise=normalise, want_state=True,
                                 state_in=S0, z_in=z0 if normalise else None)
    tol = TOL[dtype]
    e = rows_rel_err(host(out), ref)
    assert e <= tol, f"output rel err {e:.3e} > {tol}"
    es = mat_rel_err(host(S), Sr)
    assert es <= tol, f"state rel err {es:.3e}"
    if normalise:
        ez = mat_rel_err(host(z), zr)
        assert ez <= tol, f"z rel err {ez:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_in_pieces_equals_one_pass(dtype):
    """A sequence run in four uneven pieces, each from the last piece's sums, gives the one-pass rows."""
    B, H, Hkv, N, d = 2, 8, 2, 3001, 128 if dtype == "bf16" else 64
    q, k, v = (gpu(t) for t in make_qkv(B, H, Hkv, N, d, dtype, 808))
    print(f"pieces B{B} H{H} Hkv{Hkv} N{N} d{d} {dtype}", flush=True)
    whole, S_w, z_w = ops.fwd(q, k, v, want_state=True)
    cuts = [0, 1, 1000, 1777, N]
    S = torch.zeros(B, Hkv, d, d, device="cuda")
    z = torch.zeros(B, Hkv, d, device="cuda")
    outs = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        sl = (slice(None), slice(None), slice(a, b))
        o, S, z = ops.fwd(q[sl].contiguous(), k[sl].contiguous(), v[sl].contiguous(), want_state=True,
                          state_in=S, z_in=z)
        outs.append(o)
    torch.cuda.synchronize()
    pieces = torch.cat(outs, dim=2)
    tol = TOL[dtype]
    assert rows_rel_err(host(pieces), host(whole)) <= tol
    assert mat_rel_err(host(S), host(S_w)) <= 1e-4 and mat_rel_err(host(z), host(z_w)) <= 1e-4
    ref = oracle.ref_fwd(*(t.cpu() for t in (q, k, v)), causal=True)
    assert rows_rel_err(host(pieces), ref) <= tol


def test_continuation_edge_cases():
    B, H, Hkv, d = 1, 4, 2, 64
    S0, z0 = start_sums(B, Hkv, d, "f32", 3)
    S0, z0 = gpu(S0), gpu(z0)
    # N == 0: the final sums are the start sums, bit for bit
    q = torch.zeros(B, H, 0, d, device="cuda")
    kv = torch.zeros(B, Hkv, 0, d, device="cuda")
    for causal in (1, 0):
        out, S, z = ops.fwd(q, kv, kv.clone(), causal=causal, want_state=True, state_in=S0, z_in=z0)
        torch.cuda.synchronize()
        assert out.shape == q.shape and torch.equal(S, S0) and torch.equal(z, z0)
    q, k, v = (gpu(t) for t in make_qkv(B, H, Hkv, 50, d, "f32", 4))
    out = torch.empty_like(q)
    S, z = torch.empty_like(S0), torch.empty_like(z0)
    ws = ops.workspace(B, H, Hkv, 50, d, 1, q.dtype)
    nbytes = ws.numel() * 4 if ws is not None else 0
    f32 = la.LINATTN_F32
    call = lambda si, zi, so, zo, norm: la.linattn_fwd_from_state(q, k, v, out, B, H, Hkv, 50, d, 1, norm, f32,
                                                                  si, zi, so, zo, 0, ws, nbytes)
    assert call(None, z0, S, z, 1) == -1          # state_in is required
    assert call(S0, None, S, z, 1) == -1          # z_in is required when normalising
    assert call(S0, z0, S0, z, 1) == -2           # outputs may not alias the start sums
    assert call(S0, z0, S, z0, 1) == -2
    assert call(S0, None, S, z, 0) == 0           # without normalisation z starts from zero
    torch.cuda.synchronize()
    _, Sr, zr = oracle.ref_fwd(*(t.cpu() for t in (q, k, v)), normalise=False, want_state=True, state_in=S0.cpu())
    assert mat_rel_err(host(S), Sr) <= 1e-4 and mat_rel_err(host(z), zr) <= 1e-4


# ------------------------------------------------------------------- fp16 rows

@pytest.mark.parametrize("B,H,Hkv,N,d", [(1, 2, 2, 256, 32), (2, 4, 2, 257, 64), (1, 8, 2, 2049, 128),
                                         (2, 6, 2, 300, 64), (1, 16, 2, 333, 128)])
@pytest.mark.parametrize("causal", [1, 0])
@pytest.mark.parametrize("normalise", [1, 0])
def test_fp16_small_shapes(B, H, Hkv, N, d, causal, normalise):
    run_case(B, H, Hkv, N, d, "f16", causal, normalise, seed=N + d + 3)


def test_fp16_long_sequence_sampled():
    """cfg3's shape with fp16 rows, the oracle on two sampled sequences end to end."""
    B, H, Hkv, N, d = 2, 8, 8, 16384, 64
    q, k, v = make_qkv(B, H, Hkv, N, d, "f16", 1703)
    print("fp16 B2 H8 N16384 d64", flush=True)
    out, S, z = ops.fwd(gpu(q), gpu(k), gpu(v), want_state=True)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 7)):
        ref, Sr, zr = oracle.ref_fwd(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], want_state=True)
        assert rows_rel_err(host(out[b:b + 1, h:h + 1]), ref) <= TOL["f16"]
        assert mat_rel_err(host(S[b:b + 1, h:h + 1]), Sr) <= TOL["f16"]


def test_fp16_decode_step():
    B, H, Hkv, d = 3, 8, 2, 128
    S0 = torch.randn(B, Hkv, d, d, generator=torch.Generator().manual_seed(1)).abs() * 3
    z0 = torch.rand(B, Hkv, d, generator=torch.Generator().manual_seed(2)) * 50 + 1
    st = DecodeStream(B, H, Hkv, d, "f16", 4)
    q, k, v = st.next()
    S, z = gpu(S0.clone()), gpu(z0.clone())
    out = ops.decode_step(S, z, gpu(q), gpu(k), gpu(v))
    torch.cuda.synchronize()
    Sr, zr = S0.double().numpy(), z0.double().numpy()
    ref = oracle.ref_decode_step(Sr, zr, q, k, v, normalise=True)
    assert out.dtype == torch.float16
    assert rows_rel_err(host(out), ref) <= TOL["f16"]
    assert mat_rel_err(host(S), Sr) <= 1e-5


# ------------------------------------------------------------- maximum size

def test_head_block_past_two_gib():
    """bf16, G = 4, d = 128, N just over 2^21: four query heads of q span more than
    2 GiB, so the plan halves the heads per workgroup (32-bit offsets inside a block).
    With k = 0 (phi(k) = 1) every normalised row is the prefix mean of v whatever q is,
    a property that holds at any size; sampled rows (incl. the block's last ones, past
    the 1 GiB and 2 GiB offsets) are checked against it in fp64 on the host."""
    B, H, Hkv, d = 1, 4, 1, 128
    N = (1 << 21) + 1000
    assert H * N * d * 2 > 2**31 - 1
    print(f"max-size case B{B} H{H} Hkv{Hkv} N{N} d{d} bf16", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(4242)
    q = torch.randn(B, H, N, d, generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn(B, Hkv, N, d, generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.zeros_like(v)
    out = ops.fwd(q, k, v)
    torch.cuda.synchronize()
    vh = v[0, 0].double().cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, 64), np.linspace(0, N - 1, 200).astype(np.int64),
                                     np.arange(N - 64, N)]))
    csum = np.cumsum(vh, axis=0)
    ref = csum[rows] / (rows + 1)[:, None]
    del q
    o = out[0][:, torch.from_numpy(rows).cuda()].double().cpu().numpy()  # [H, rows, d]
    for h in range(H):
        e = rows_rel_err(o[h], ref)
        assert e <= TOL["bf16"], f"head {h}: {e:.3e}"
