"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and validates arguments / plans launches on the host.

Only calls that return before any HIP call are made here (argument errors,
workspace sizing, planning); nothing is launched.
"""
import ctypes
import os
import re
import subprocess

import pytest

import sequence_mixing_amd as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")
F32, BF16 = la.LINATTN_F32, la.LINATTN_BF16


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(linattn_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("linattn_fwd", "linattn_decode_step", "linattn_fwd_workspace_bytes", "linattn_fwd_plan",
              "linattn_status_string", "linattn_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = la.load()
    for n in declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", la.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (linattn_\w+)", out))
    assert set(declared_functions()) <= exported


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-fsyntax-only", "-x", "c", "-std=c99", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", HEADER], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_version_and_status_strings():
    import re

    declared = int(re.search(r"#define LINATTN_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert la.linattn_abi_version() == declared
    for code in [0, -1, -2, -3, -4, -5, -6, -7]:
        assert la.linattn_status_string(code) and la.linattn_status_string(code) != "unknown status"
    assert la.linattn_status_string(12345) == "unknown status"


@pytest.mark.parametrize("args,code", [
    ((1, 3, 2, 16, 64, 1, F32, 0), -2),     # H % Hkv != 0
    ((-1, 2, 2, 16, 64, 1, F32, 0), -2),    # B < 0
    ((1, 2, 2, -5, 64, 1, F32, 0), -2),     # N < 0
    ((1, 0, 1, 16, 64, 1, F32, 0), -2),     # H == 0
    ((1, 2, 2, 16, 48, 1, F32, 0), -4),     # d unsupported
    ((1, 2, 2, 16, 256, 1, BF16, 0), -4),   # d unsupported
    ((1, 2, 2, 16, 64, 1, F32, 96), -4),    # chunk unsupported
    ((1, 2, 2, 16, 128, 1, BF16, 256), -4), # bf16 d=128 chunk 256 exceeds LDS
    ((1, 2, 2, 16, 64, 1, 7, 0), -3),       # dtype
])
def test_plan_rejects(args, code):
    rc, _, _ = la.linattn_fwd_plan(*args)
    assert rc == code
    assert la.linattn_fwd_workspace_bytes(*args) == -1


def test_fwd_rejects_before_launch():
    # Argument errors return before anything touches the GPU.
    assert la.linattn_fwd(None, None, None, None, 1, 3, 2, 16, 64, 1, 1, F32, stream=0) == -2
    assert la.linattn_fwd(None, None, None, None, 1, 2, 2, 16, 64, 1, 1, F32, stream=0) == -1
    assert la.linattn_fwd(16, 16, 16, 16, 1, 2, 2, 16, 64, 1, 1, 9, stream=0) == -3
    assert la.linattn_fwd(16, 16, 16, 16, 1, 2, 2, 16, 40, 1, 1, F32, stream=0) == -4
    assert la.linattn_fwd(17, 16, 16, 16, 1, 2, 2, 16, 64, 1, 1, F32, stream=0) == -7
    # 4096 tokens need a workspace; none given.
    assert la.linattn_fwd(16, 16, 16, 16, 2, 8, 8, 4096, 64, 1, 1, F32, stream=0) == -5
    need = la.linattn_fwd_workspace_bytes(2, 8, 8, 4096, 64, 1, F32)
    assert la.linattn_fwd(16, 16, 16, 16, 2, 8, 8, 4096, 64, 1, 1, F32, workspace=16, workspace_bytes=need - 4,
                          stream=0) == -5
    # B == 0 is a valid no-op.
    assert la.linattn_fwd(None, None, None, None, 0, 2, 2, 16, 64, 1, 1, F32, stream=0) == 0


def test_decode_rejects_before_launch():
    assert la.linattn_decode_step(16, 16, 16, 16, 16, 16, 1, 3, 2, 64, 1, F32, stream=0) == -2
    assert la.linattn_decode_step(16, 16, 16, 16, 16, 16, 1, 2, 2, 48, 1, F32, stream=0) == -4
    assert la.linattn_decode_step(16, 16, 16, 16, 16, 16, 1, 2, 2, 64, 1, 9, stream=0) == -3
    assert la.linattn_decode_step(16, None, 16, 16, 16, 16, 1, 2, 2, 64, 1, F32, stream=0) == -1
    assert la.linattn_decode_step(None, 16, 16, 16, 16, 16, 1, 2, 2, 64, 1, F32, stream=0) == -1
    assert la.linattn_decode_step(16, 16, 24, 16, 16, 16, 1, 2, 2, 64, 1, F32, stream=0) == -7
    assert la.linattn_decode_step(None, None, None, None, None, None, 0, 2, 2, 64, 1, F32, stream=0) == 0


def plan(B, H, Hkv, N, d, causal, dtype, chunk=0):
    rc, c, p = la.linattn_fwd_plan(B, H, Hkv, N, d, causal, dtype, chunk)
    assert rc == 0
    return c, p


def test_plan_covers_every_token_with_whole_chunks():
    for N in [1, 7, 31, 32, 33, 100, 257, 4096, 4097, 65536]:
        for chunk in [32, 64, 128, 256]:
            for nseq in [1, 2, 16, 64]:
                c, P = plan(nseq, 1, 1, N, 64, 1, BF16, chunk)
                assert c == chunk
                nch = -(-N // c)
                assert 1 <= P <= nch
                # Segments are whole chunks: some segment length s chunks covers N
                # with P segments, the last one non-empty.
                assert any((P - 1) * s * c < N <= P * s * c for s in range(1, nch + 1))
                # Enough workgroups to spread over the chip (one or two per CU),
                # never more than two per CU.
                assert nseq * P <= 512 + nseq
                assert nseq * P >= min(nseq * nch, 128)


def test_workspace_formula():
    for (B, H, Hkv, N, d, causal, dt) in [(2, 8, 8, 4096, 64, 1, F32), (2, 8, 8, 65536, 64, 1, BF16),
                                          (1, 32, 8, 32768, 128, 1, BF16), (2, 8, 8, 4096, 64, 0, F32),
                                          (1, 2, 2, 256, 32, 1, F32), (3, 4, 2, 7, 64, 0, BF16)]:
        c, P = plan(B, H, Hkv, N, d, causal, dt)
        slots = P - 1 if causal else P
        assert la.linattn_fwd_workspace_bytes(B, H, Hkv, N, d, causal, dt) == B * Hkv * slots * d * (d + 1) * 4
    assert la.linattn_fwd_workspace_bytes(1, 1, 1, 0, 64, 1, F32) == 0
    assert la.linattn_fwd_workspace_bytes(0, 1, 1, 100, 64, 1, F32) == 0


def test_auto_chunk_choices():
    for args in [(2, 8, 8, 65536, 64, 1, BF16), (1, 32, 8, 32768, 128, 1, BF16), (2, 8, 8, 4096, 64, 1, F32),
                 (1, 2, 2, 256, 32, 1, F32), (1, 2, 2, 256, 128, 1, F32)]:
        c, _ = plan(*args)
        assert c in (32, 64, 128, 256)
        # the automatic choice is always one the explicit argument accepts
        assert la.linattn_fwd_plan(*args, c)[0] == 0
    # every group size, head dimension and dtype (planning runs on the host:
    # a bad automatic choice would show up here, not on the GPU)
    for dt in (F32, BF16, la.LINATTN_F16):
        for d in (32, 64, 128):
            for G in (1, 2, 3, 4, 5, 6, 8, 12, 16, 32):
                for causal in (0, 1):
                    rc, c, P = la.linattn_fwd_plan(2, 2 * G, 2, 1000, d, causal, dt, 0)
                    assert rc == 0 and c in (32, 64, 128, 256), (dt, d, G, causal, rc, c)
                    assert la.linattn_fwd_workspace_bytes(2, 2 * G, 2, 1000, d, causal, dt) >= 0


def test_bwd_workspace_and_validation_without_gpu():
    """Argument checks of the backward run before any launch."""
    f32, bf = la.LINATTN_F32, la.LINATTN_BF16
    assert la.linattn_bwd_workspace_bytes(1, 2, 2, 64, 48, 1, f32) == -1       # d not supported
    assert la.linattn_bwd_workspace_bytes(1, 3, 2, 64, 64, 1, f32) == -1       # H % Hkv != 0
    assert la.linattn_bwd_workspace_bytes(1, 2, 2, 64, 64, 1, 7) == -1         # dtype
    # causal: forward sums, den and the suffix sums of (P - 1) segments; grows with B*H*N for den
    a = la.linattn_bwd_workspace_bytes(2, 8, 8, 4096, 64, 1, f32)
    b = la.linattn_bwd_workspace_bytes(2, 8, 8, 8192, 64, 1, bf)
    assert 0 < a < b
    assert la.linattn_bwd(None, None, None, None, None, None, None, None, 0, 2, 2, 64, 64, 1, 1, f32, stream=0) == 0
    assert la.linattn_bwd(None, None, None, None, None, None, None, None, 1, 2, 2, 64, 64, 1, 1, f32, stream=0) == -1
    assert la.linattn_bwd(None, None, None, None, None, None, None, None, 1, 2, 2, 64, 40, 1, 1, f32, stream=0) == -4


def test_packed_argtypes_match_header():
    """Every exported call's ctypes argument count equals the header's parameter count."""
    hdr = open(os.path.join(ROOT, "include", "linattn.h")).read()
    lib = la.load()
    for name in ("linattn_fwd", "linattn_fwd_from_state", "linattn_fwd_packed", "linattn_fwd_timed",
                 "linattn_bwd", "linattn_decode_step", "linattn_fwd_packed_workspace_bytes",
                 "linattn_bwd_workspace_bytes", "linattn_fwd_workspace_bytes", "linattn_fwd_plan",
                 "linattn_fwd_decay", "linattn_fwd_decay_workspace_bytes", "linattn_decode_step_decay"):
        m = re.search(r"\b" + name + r"\(([^)]*)\);", hdr)
        assert m, name
        nparams = len([p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"])
        assert len(getattr(lib, name).argtypes) == nparams, name


def test_fp16_plans_like_bf16():
    """fp16 rows take the 16-bit kernels: the same chunk, segments and workspace as bf16."""
    for args in [(2, 8, 8, 4096, 64, 1), (1, 32, 8, 32768, 128, 1), (2, 8, 8, 4096, 64, 0), (3, 6, 2, 777, 32, 1)]:
        assert la.linattn_fwd_plan(*args, la.LINATTN_F16) == la.linattn_fwd_plan(*args, la.LINATTN_BF16)
        assert la.linattn_fwd_workspace_bytes(*args, la.LINATTN_F16) == la.linattn_fwd_workspace_bytes(*args, la.LINATTN_BF16)
        assert la.linattn_bwd_workspace_bytes(*args, la.LINATTN_F16) == la.linattn_bwd_workspace_bytes(*args, la.LINATTN_BF16)
    assert la.linattn_fwd_plan(1, 2, 2, 16, 64, 1, 9)[0] == -3


def test_decay_validation_without_gpu():
    """linattn_fwd_decay / its workspace size: argument checks before any launch."""
    f32, bf = la.LINATTN_F32, la.LINATTN_BF16
    relu = f32 | (1 << 8)
    assert la.linattn_fwd_decay_workspace_bytes(1, 2, 2, 64, 64, relu, 0) == -1     # feature map
    assert la.linattn_fwd_decay_workspace_bytes(1, 2, 2, 4096, 64, f32, 128) == -1  # shifted fp32 copies
    for args in [(2, 8, 8, 4096, 64), (1, 32, 8, 32768, 128), (2, 8, 8, 16384, 64), (3, 6, 2, 777, 32)]:
        for dt in (f32, bf):
            rc, c, P = la.linattn_fwd_plan(*args, 1, dt, 0)
            # the automatic chunk, at most 64 tokens for 16-bit rows at d <= 64
            ch = 64 if dt == bf and args[4] <= 64 and c > 64 else c
            rc, c, P = la.linattn_fwd_plan(*args, 1, dt, ch)
            plain = la.linattn_fwd_workspace_bytes(*args, 1, dt, ch)
            B, H, Hkv = args[:3]
            # one float more per segment partial (the segment's summed log-decay)
            assert la.linattn_fwd_decay_workspace_bytes(*args, dt, 0) == plain + B * Hkv * (P - 1) * 4
            assert la.linattn_fwd_decay_workspace_bytes(*args, dt, 0) == la.linattn_fwd_decay_workspace_bytes(*args, dt, ch)
    assert la.linattn_fwd_decay(None, None, None, None, None, 0, 2, 2, 64, 64, 1, f32, stream=0) == 0
    assert la.linattn_fwd_decay(16, 16, 16, None, 16, 1, 2, 2, 64, 64, 1, f32, stream=0) == -1
    assert la.linattn_fwd_decay(16, 16, 16, 16, 16, 1, 2, 2, 64, 64, 1, relu, stream=0) == -4
    need = la.linattn_fwd_decay_workspace_bytes(2, 8, 8, 4096, 64, f32, 0)
    assert la.linattn_fwd_decay(16, 16, 16, 16, 16, 2, 8, 8, 4096, 64, 1, f32, workspace=16,
                                workspace_bytes=need - 4, stream=0) == -5
    assert la.linattn_fwd_decay(16, 16, 16, 18, 16, 1, 2, 2, 64, 64, 1, f32, stream=0) == -7  # g misaligned
    assert la.linattn_decode_step_decay(16, 16, 16, 16, 16, None, 16, 1, 2, 2, 64, 1, f32, stream=0) == -1
    assert la.linattn_decode_step_decay(16, 16, 16, 16, 16, 18, 16, 1, 2, 2, 64, 1, f32, stream=0) == -7


def test_plan_size_limits():
    """One head's q past 2 GiB is rejected; just below it plans (with fewer heads per block)."""
    bf = la.LINATTN_BF16
    assert la.linattn_fwd_plan(1, 1, 1, 1 << 23, 128, 1, bf, 0)[0] == -2
    assert la.linattn_fwd_plan(1, 4, 1, (1 << 21) + 1000, 128, 1, bf, 0)[0] == 0
    assert la.linattn_fwd_plan(1, 1, 1, (1 << 23) - 16, 128, 1, bf, 0)[0] == 0
