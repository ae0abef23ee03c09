"""The oracle's α-entmax against hand-derived closed forms stored in
tests/golden/entmax_closed_forms.txt (each line carries its derivation from the
α-entmax definition of the paper review, section 三 background)."""
import os

import numpy as np
import pytest

from oracle import dash_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _cases():
    out = []
    for line in open(os.path.join(HERE, "golden", "entmax_closed_forms.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        alpha, s, p, tau, why = [f.strip() for f in line.split("|")]
        out.append((float(alpha), [float(v) for v in s.split(",")], [float(v) for v in p.split(",")],
                    None if tau == "-" else float(tau), why))
    return out


CASES = _cases()


def test_fixture_is_complete():
    assert len(CASES) >= 9
    assert {c[0] for c in CASES} >= {1.0, 1.5, 2.0, 3.0}


@pytest.mark.parametrize("case", CASES, ids=[f"a{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_entmax_closed_form(case):
    alpha, s, p_ref, tau_ref, why = case
    p, tau, _ = O.entmax(np.array([s]), alpha=alpha)
    assert np.abs(p[0] - np.array(p_ref)).max() <= 1e-12, why
    assert abs(p[0].sum() - 1.0) <= 1e-12
    if tau_ref is not None:
        assert abs(float(tau[0]) - tau_ref) <= 1e-12, why
