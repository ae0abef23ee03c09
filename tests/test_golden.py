"""The oracle against hand-derived closed forms stored under tests/golden/ (each line
carries its derivation): α-entmax (the paper review, section 三 background formula) and
the Stage-0 summaries (section 三, Eq. 4)."""
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


def _stage0_cases():
    out = []
    for line in open(os.path.join(HERE, "golden", "stage0_closed_forms.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        d, B, keys, qbar, kbar, why = [f.strip() for f in line.split("|")]
        K = np.array([[float(v) for v in row.split(",")] for row in keys.split(";")])
        out.append((int(d), int(B), K, np.array([float(v) for v in qbar.split(",")]),
                    np.array([float(v) for v in kbar.split(",")]), why))
    return out


S0 = _stage0_cases()


@pytest.mark.parametrize("case", S0, ids=[f"s0-{i}" for i in range(len(S0))])
def test_stage0_closed_form(case):
    d, B, K, qbar, kbar_ref, why = case
    assert K.shape == (B, d)
    kb = O.stage0_summaries(K[None, None], qbar[None], B)          # [1, 1, 1, d]
    assert kb.shape == (1, 1, 1, d)
    assert np.abs(kb[0, 0, 0] - kbar_ref).max() <= 1e-12, why


def _ra_cases():
    import json
    f = json.load(open(os.path.join(HERE, "golden", "route_attend_closed_forms.json")))
    return f["common"], f["cases"]


RA_COMMON, RA = _ra_cases()


@pytest.mark.parametrize("case", RA, ids=[c["name"].replace(" ", "_") for c in RA])
def test_route_attend_closed_form(case):
    c = RA_COMMON
    Q = np.array(case["Q"], dtype=np.float64)[None, :, None, :]            # [1, h_q, 1, d]
    kbar = np.array(case["kbar"], dtype=np.float64)[None, None]            # [1, 1, T, d]
    pos = np.array([[c["pos"]]])
    rt = O.route(Q, pos, kbar, c["B"], c["alpha"], c["gamma"], c["sigma"], c["causal"], c["n_kv"])
    tv = len(case["w"])                                  # visible chunks; the rest is the query's own
    assert np.abs(rt["w"][0, 0, 0, :tv] - np.array(case["w"])).max() <= 1e-12, case["derivation"]
    assert rt["support"][0, 0, 0, :tv].all() and not rt["support"][0, 0, 0, tv:].any()
    assert np.abs(rt["bias"][0, 0, 0, :tv] - np.array(case["bias"])).max() <= 1e-12, case["derivation"]
    K = np.array(c["K"], dtype=np.float64)[None, None]
    V = np.array(c["V"], dtype=np.float64)[None, None]
    out = O.attend(Q, pos, K, V, rt, c["B"], c["causal"], c["n_kv"])
    assert np.abs(out[0, :, 0] - np.array(case["O"])).max() <= 1e-12, case["derivation"]
