"""Planted-mistake check for the oracle's pins (CPU only).

Each case copies ``oracle/linattn_ref.c``, plants one plausible slip (a dropped
term, a wrong index, an exclusive mask, a different GQA head map, a
transposed state read, a flipped gradient sign, ...), compiles the copy into a
temporary library and runs the oracle pin suites (forward and backward)
against it in a child process.  The suite must fail
for every mutant; a mutant that survives means the pins have a blind spot.
The real oracle source is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "linattn_ref.c")

CAUSAL_ABSORB = """            /* Absorb token t before reading: query t sees keys s <= t. */
            for (int i = 0; i < d; ++i) f[i] = linattn_ref_phi(kb[(size_t)t * d + i]);
            for (int i = 0; i < d; ++i) {
                for (int jj = 0; jj < w; ++jj) S[(size_t)i * w + jj] += f[i] * vb[(size_t)t * d + j0 + jj];
                z[i] += f[i];
            }
"""


def _exclusive_mask(src: str) -> str:
    """Move the causal absorb after the reads: query t would see only s < t."""
    assert CAUSAL_ABSORB in src
    src = src.replace(CAUSAL_ABSORB, "")
    anchor = """                ot[j0 + jj] = J->normalise ? num / den : num;
            }
        }
"""
    assert anchor in src
    return src.replace(anchor, anchor + "        if (J->causal) {\n" + CAUSAL_ABSORB + "        }\n", 1)


DECODE_UPDATE = """            for (int i = 0; i < d; ++i) {
                for (int j = 0; j < d; ++j) S[(size_t)i * d + j] += f[i] * vt[j];
                if (zz) zz[i] += f[i];
            }
"""


def _decode_reads_before_update(src: str) -> str:
    """Apply the decode update after the queries read the state (exclusive decode)."""
    assert DECODE_UPDATE in src
    src = src.replace(DECODE_UPDATE, "")
    anchor = """                    ot[j] = normalise ? num / den : num;
                }
            }
"""
    assert anchor in src
    return src.replace(anchor, anchor + DECODE_UPDATE, 1)


DECAY_BLOCK = """            if (gb) {
                const double a = exp(gb[t]);
                for (int i = 0; i < d; ++i) {
                    for (int jj = 0; jj < w; ++jj) S[(size_t)i * w + jj] *= a;
                    z[i] *= a;
                }
            }
"""


def _decay_after_absorb(src: str) -> str:
    """Decay after token t is added: S_t = a_t (S_{t-1} + phi(k_t) v_t^T)."""
    assert DECAY_BLOCK in src
    src = src.replace(DECAY_BLOCK, "", 1)
    anchor = """                z[i] += f[i];
            }
        }
        for (int h = g * G; h < (g + 1) * G; ++h) {"""
    assert anchor in src
    return src.replace(anchor, anchor.replace("        }\n        for (int h", DECAY_BLOCK.replace("            ", "            ", 1)
                                               + "        }\n        for (int h", 1), 1)


BWD_GATHER = "        if (J->causal) GATHER(s);\n"
BWD_DK_STORE = """            dkb[(size_t)s * d + i] = acc * linattn_ref_dphi(ks[i]);
        }
"""


def _bwd_exclusive_reverse_walk(src: str) -> str:
    """Gather query s into (R, r) after key s is read: key s would miss query s."""
    assert BWD_GATHER in src and BWD_DK_STORE in src
    return src.replace(BWD_GATHER, "", 1).replace(BWD_DK_STORE, BWD_DK_STORE + BWD_GATHER, 1)


MUTANTS = {
    "phi_drops_plus_one": lambda s: s.replace("x > 0.0 ? x + 1.0 : exp(x)", "x > 0.0 ? x : exp(x)"),
    "phi_negative_branch_is_plain_elu": lambda s: s.replace("x > 0.0 ? x + 1.0 : exp(x)",
                                                           "x > 0.0 ? x + 1.0 : exp(x) - 1.0"),
    "exclusive_causal_mask": _exclusive_mask,
    "denominator_drops_query": lambda s: s.replace("for (int i = 0; i < d; ++i) den += p[i] * z[i];",
                                                   "for (int i = 0; i < d; ++i) den += z[i];", 1),
    "value_column_offset_lost": lambda s: s.replace("vb[(size_t)t * d + j0 + jj]", "vb[(size_t)t * d + jj]"),
    "interleaved_head_map": lambda s: s.replace(
        "for (int h = g * G; h < (g + 1) * G; ++h) {\n            const double *qt = J->q",
        "for (int h = g; h < J->H; h += J->Hkv) {\n            const double *qt = J->q"),
    "state_read_transposed": lambda s: s.replace("num += p[i] * S[(size_t)i * w + jj];",
                                                 "num += p[i] * S[(size_t)jj * w + i];"),
    "noncausal_drops_last_token": lambda s: s.replace(
        "for (int t = 0; t < N; ++t) {\n            for (int i = 0; i < d; ++i) f[i] = linattn_ref_phi(kb",
        "for (int t = 0; t < N - 1; ++t) {\n            for (int i = 0; i < d; ++i) f[i] = linattn_ref_phi(kb"),
    "decode_skips_z_update": lambda s: s.replace("if (zz) zz[i] += f[i];", ""),
    "decode_reads_before_update": _decode_reads_before_update,
    "continuation_ignores_z_in": lambda s: s.replace("for (int i = 0; i < d; ++i) z[i] = zi[i];",
                                                     "for (int i = 0; i < d; ++i) z[i] = 0.0 * zi[i];"),
    "continuation_state_in_transposed": lambda s: s.replace(
        "S[(size_t)i * w + jj] = si[(size_t)i * d + j0 + jj];", "S[(size_t)i * w + jj] = si[(size_t)(j0 + jj) * d + i];"),
    "bwd_normaliser_gradient_sign": lambda s: s.replace("hval = -dov / den;", "hval = dov / den;"),
    "bwd_dq_drops_normaliser_term": lambda s: s.replace("double da = hval * z[i];", "double da = 0.0 * z[i];"),
    "bwd_exclusive_reverse_walk": _bwd_exclusive_reverse_walk,
    "bwd_dphi_branches_swapped": lambda s: s.replace("return x > 0.0 ? 1.0 : exp(x);",
                                                     "return x > 0.0 ? exp(x) : 1.0;"),
    "bwd_dk_drops_normaliser_sum": lambda s: s.replace("double acc = r[i];", "double acc = 0.0 * r[i];"),
    "bwd_dv_reads_R_transposed": lambda s: s.replace("acc += R[(size_t)i * d + j] * f[i];",
                                                     "acc += R[(size_t)j * d + i] * f[i];"),
    "bwd_gradient_not_divided_by_denominator": lambda s: s.replace("gt[j] = dot[j] / den;", "gt[j] = dot[j];"),
    "softplus_positive_branch_sign": lambda s: s.replace("x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x))",
                                                         "x > 0.0 ? x + log1p(exp(x)) : log1p(exp(x))"),
    "relu_keeps_negatives": lambda s: s.replace("if (g_feature_map == 1) return x > 0.0 || x != x ? x : 0.0;",
                                                "if (g_feature_map == 1) return x > -0.5 || x != x ? x : 0.0;"),
    "softplus_derivative_sign": lambda s: s.replace("return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    "window_one_key_too_many": lambda s: s.replace("const int s0 = t - J->W + 1 > 0 ? t - J->W + 1 : 0;",
                                                   "const int s0 = t - J->W > 0 ? t - J->W : 0;"),
    "window_without_diagonal": lambda s: s.replace("for (int s = s0; s <= t; ++s) {", "for (int s = s0; s < t; ++s) {"),
    "decay_applied_after_absorb": _decay_after_absorb,
    "decay_skips_z": lambda s: s.replace("S[(size_t)i * w + jj] *= a;\n                    z[i] *= a;",
                                         "S[(size_t)i * w + jj] *= a;\n"),
    "decay_sign_flipped": lambda s: s.replace("const double a = exp(gb[t]);", "const double a = exp(-gb[t]);"),
    "decay_reads_next_token": lambda s: s.replace("const double a = exp(gb[t]);",
                                                  "const double a = exp(gb[t + 1 < N ? t + 1 : t]);"),
    "decode_decay_skipped": lambda s: s.replace("const double a = exp(gd[(size_t)b * Hkv + g]);",
                                                "const double a = 1.0 + 0.0 * gd[(size_t)b * Hkv + g];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = open(SRC).read()
    mutated = MUTANTS[name](src)
    assert mutated != src, f"mutation {name} did not apply"
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-w", str(c_path), "-o", str(so_path),
                    "-lm", "-lpthread"], check=True)
    env = dict(os.environ, LINATTN_REF_LIB=str(so_path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py"), os.path.join(ROOT, "tests", "test_oracle_bwd.py"),
                        os.path.join(ROOT, "tests", "test_oracle_phi.py"),
                        os.path.join(ROOT, "tests", "test_oracle_decay.py"),
                        os.path.join(ROOT, "tests", "test_oracle_window.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the oracle pins:\n{r.stdout[-2000:]}"
