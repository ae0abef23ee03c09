"""The seeded workload generator: determinism, bf16 rounding and planted structure."""
import numpy as np
import pytest
import torch

from long_context_amd import inputs


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3e-39], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(inputs.round_bf16(x), ref)


def test_seeded_and_deterministic():
    a = inputs.make_prefill(b=1, h_q=2, h_kv=1, d=16, n=64, B=16, seed=3)
    b = inputs.make_prefill(b=1, h_q=2, h_kv=1, d=16, n=64, B=16, seed=3)
    c = inputs.make_prefill(b=1, h_q=2, h_kv=1, d=16, n=64, B=16, seed=4)
    np.testing.assert_array_equal(a.Q, b.Q)
    np.testing.assert_array_equal(a.qbar, b.qbar)
    assert not np.array_equal(a.Q, c.Q)


def test_prefill_1k_fp32_shapes():
    w = inputs.prefill_1k_fp32()
    assert w.Q.shape == (1, 1, 1024, 64) and w.K.shape == (1, 1, 1024, 64)
    assert w.dtype == "f32" and w.B == 64 and w.alpha == 1.5 and w.gamma == 1.0
    assert abs(w.qbar.std() - 0.1) < 0.03


def test_needles_have_cosine_point_eight():
    w = inputs.prefill_8k_gqa8_needles()
    assert w.Q.shape == (1, 16, 8192, 128)
    assert np.array_equal(inputs.round_bf16(w.Q), w.Q)
    # the aligned query rows: all heads of a group share the direction u
    K = w.K[0, 0].astype(np.float64)
    Q = w.Q[0, 0].astype(np.float64)
    qn = Q / np.linalg.norm(Q, axis=-1, keepdims=True)
    Kn = K / np.linalg.norm(K, axis=-1, keepdims=True)
    cos = Kn @ qn.T                        # [n, n]
    hits = np.abs(cos - 0.8) < 0.01        # bf16 rounding moves cosines by ~1e-3
    assert hits.sum() >= 8 * 64 * 64 * 0.95


def test_decode_128k_flat_and_sharp_groups():
    w = inputs.decode_128k_b4()
    norms = np.linalg.norm(w.Q[:, :, 0].astype(np.float64), axis=-1).reshape(4, 2, 16)
    assert np.allclose(norms[w.sharp == 1], 4.0, rtol=1e-2)
    assert np.allclose(norms[w.sharp == 0], 0.2, rtol=1e-2)
    assert w.sharp.sum() == 4
    assert w.seq_len.tolist() == [131072] * 4


@pytest.mark.slow
def test_calibrated_gamma_gives_three_quarters_sparsity():
    """The frozen γ of the 8K needle workload reproduces 75% +- 1% group sparsity
    under the oracle's routing on every 16th row."""
    from oracle import dash_oracle as O
    w = inputs.prefill_8k_gqa8_needles()
    kb = O.stage0_summaries(w.K, w.qbar, w.B)
    rows = np.arange(0, w.n, 16)
    rt = O.route(w.Q[:, :, rows], rows[None], kb, w.B, w.alpha, w.gamma, w.sigma, True, w.n)
    assert abs(O.group_sparsity(rt) - 0.75) <= 0.01
