"""Oracle against the hand-derived fixtures in tests/golden/hand_examples.txt (CPU only)."""
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _cases():
    cases, cur = [], None
    for line in open(os.path.join(HERE, "golden", "hand_examples.txt")):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        tag, *vals = line.split()
        if tag == "case":
            cur = {"name": vals[0], "N": int(vals[1]), "d": int(vals[2]), "norm": bool(int(vals[3])),
                   "q": [], "k": [], "v": [], "o": []}
            cases.append(cur)
        else:
            cur[tag].append([float(x) for x in vals])
    return cases


def test_hand_examples():
    cases = _cases()
    assert len(cases) == 4
    for c in cases:
        q, k, v, o = (np.array(c[t])[None, None] for t in "qkvo")
        assert q.shape == (1, 1, c["N"], c["d"]) and o.shape == q.shape
        got = oracle.ref_fwd(q, k, v, causal=True, normalise=c["norm"])
        assert np.allclose(got, o, rtol=1e-15, atol=1e-15), c["name"]
