"""Pins of the fp64 oracle against mathematics it does not share code with.

The paper (arXiv:2609.21594) prints no worked example of the Muon step (its
section 2.3 has no body in the page text), so the oracle is pinned by:
  * the closed form of the quintic NS iteration through the SVD:
    NS(G) = U phi(S / (||G||_F + eps)) V^T, phi = p composed `steps` times,
    p(s) = a s + b s^3 + c s^5, evaluated here with scalar arithmetic;
  * special cases with no SVD (orthonormal rows, a row vector, a scalar);
  * invariants (transpose and orthogonal equivariance, scale invariance,
    zero in -> zero out, zero steps -> normalized input, the singular-value
    band the composed quintic maps into);
  * momentum, scale and apply values worked by hand;
  * torch.optim.Muon, a library implementation of the same step (loose for
    the update, since it iterates in bf16; tight for the momentum buffer).
Planted-mistake tests at the bottom check that each pin would catch a
plausible error in the oracle.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import muon as om

A_, B_, C_ = 3.4445, -4.7750, 2.0315


def p_scalar(s, a=A_, b=B_, c=C_):
    return a * s + b * s ** 3 + c * s ** 5


def phi(s, steps=5, coeffs=None):
    for k in range(steps):
        a, b, c = coeffs[k] if coeffs is not None else (A_, B_, C_)
        s = p_scalar(s, a, b, c)
    return s


def closed_form(g, steps=5, eps=1e-7, coeffs=None):
    g = np.asarray(g, np.float64)
    u, s, vt = np.linalg.svd(g, full_matrices=False)
    fro = math.sqrt(float(np.sum(g * g)))
    x = s / (fro + eps)
    return (u * np.array([phi(v, steps, coeffs) for v in x])) @ vt


def rel(a, b):
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def check_closed_form(ns, g, tol=1e-10, **kw):
    return rel(ns(g, **kw), closed_form(g, **kw)) <= tol


def _cases():
    rng = np.random.default_rng(123)
    q = rng.standard_normal((3, 6))
    rank2 = q[:2].T @ rng.standard_normal((2, 6))  # 6x6 of rank 2 ...
    return {
        "3x5_seed0": np.random.default_rng(0).standard_normal((3, 5)),
        "5x3_tall": rng.standard_normal((5, 3)),
        "4x4_square": rng.standard_normal((4, 4)),
        "rank2_3x6": rank2[:3],
        "16x40": rng.standard_normal((16, 40)),
        "40x16_tall": rng.standard_normal((40, 16)),
        "small_norm_8x12": 1e-4 * rng.standard_normal((8, 12)) / math.sqrt(96),
    }


@pytest.mark.parametrize("name", list(_cases()))
def test_closed_form(name):
    g = _cases()[name]
    err = rel(oracle.newton_schulz(g), closed_form(g))
    assert err <= 1e-10, (name, err)


def test_closed_form_3x5_values():
    # The 3x5 seed-0 input of the tiny configuration: the normalized singular
    # values and their images under phi, computed from the SVD alone.
    g = np.random.default_rng(0).standard_normal((3, 5))
    s = np.linalg.svd(g, compute_uv=False)
    x = s / (np.linalg.norm(g) + 1e-7)
    o = oracle.newton_schulz(g)
    so = np.linalg.svd(o, compute_uv=False)
    np.testing.assert_allclose(np.sort(so), np.sort([phi(v) for v in x]), rtol=1e-11)


@pytest.mark.parametrize("steps", [0, 1, 2, 5, 7])
def test_closed_form_steps(steps):
    g = np.random.default_rng(5).standard_normal((6, 9))
    assert rel(oracle.newton_schulz(g, steps), closed_form(g, steps)) <= 1e-10


def test_coefficient_table():
    g = np.random.default_rng(6).standard_normal((5, 8))
    table = [(3.0, -3.2, 1.2), (3.4445, -4.775, 2.0315), (2.9, -3.0, 1.1), (3.4, -4.7, 2.0), (1.875, -1.25, 0.375)]
    o = oracle.newton_schulz(g, 5, coeffs=table)
    assert rel(o, closed_form(g, 5, coeffs=table)) <= 1e-10
    # a table of identical triples is the fixed set
    same = oracle.newton_schulz(g, 5, coeffs=[(A_, B_, C_)] * 5)
    assert np.array_equal(same, oracle.newton_schulz(g, 5))


@pytest.mark.parametrize("m", [1, 3, 8, 64])
@pytest.mark.parametrize("alpha", [1.0, 1e-4])
def test_orthonormal_rows(m, alpha):
    # X = alpha Q with orthonormal rows: every singular value is alpha, the
    # Frobenius norm alpha sqrt(m), so NS(X) = phi(alpha sqrt(m) / (alpha sqrt(m) + eps)/sqrt(m)) Q
    rng = np.random.default_rng(m)
    q, _ = np.linalg.qr(rng.standard_normal((2 * m + 3, m)))
    q = q.T  # m x (2m+3), orthonormal rows
    x = alpha * q
    s0 = alpha / (alpha * math.sqrt(m) + 1e-7)
    np.testing.assert_allclose(oracle.newton_schulz(x), phi(s0) * q, rtol=0, atol=1e-12)


def test_phi_exact_rational():
    # phi at 1/sqrt(4) = 1/2 in exact rational arithmetic vs float scalar
    a, b, c = Fraction("3.4445"), Fraction("-4.7750"), Fraction("2.0315")
    s = Fraction(1, 2)
    for _ in range(5):
        s = a * s + b * s ** 3 + c * s ** 5
    q, _ = np.linalg.qr(np.random.default_rng(9).standard_normal((10, 4)))
    x = q.T  # 4 x 10 orthonormal rows, ||X||_F = 2
    o = oracle.newton_schulz(x, eps=0.0)
    np.testing.assert_allclose(o, float(s) * q.T, atol=1e-13)


def test_row_vector_and_scalar():
    g = np.array([[3.0, -4.0, 12.0]])  # norm 13
    expect = phi(13.0 / (13.0 + 1e-7)) * g / 13.0
    np.testing.assert_allclose(oracle.newton_schulz(g), expect, atol=1e-14)
    np.testing.assert_allclose(oracle.newton_schulz(g.T), expect.T, atol=1e-14)
    s = np.array([[-0.25]])
    np.testing.assert_allclose(oracle.newton_schulz(s), [[-phi(0.25 / (0.25 + 1e-7))]], atol=1e-14)


def test_transpose_equivariance_bitwise():
    g = np.random.default_rng(1).standard_normal((7, 19))
    assert np.array_equal(oracle.newton_schulz(g.T), oracle.newton_schulz(g).T)
    assert oracle.newton_schulz(g.T).shape == (19, 7)


def test_orthogonal_equivariance():
    rng = np.random.default_rng(2)
    g = rng.standard_normal((6, 11))
    qa, _ = np.linalg.qr(rng.standard_normal((6, 6)))
    qb, _ = np.linalg.qr(rng.standard_normal((11, 11)))
    lhs = qa @ oracle.newton_schulz(g) @ qb
    rhs = oracle.newton_schulz(qa @ g @ qb)
    assert rel(lhs, rhs) <= 1e-12


def test_scale_invariance():
    # Without eps the iteration is exactly scale invariant; eps moves the
    # result by a relative amount of order eps / ||G||.
    g = np.random.default_rng(3).standard_normal((9, 13))
    ref = oracle.newton_schulz(g, eps=0.0)
    assert rel(oracle.newton_schulz(1e5 * g, eps=0.0), ref) <= 1e-13
    for c in (1.0, 1e3):
        assert rel(oracle.newton_schulz(c * g), ref) <= 100 * 1e-7 / (c * np.linalg.norm(g))


def test_zero_in_zero_out():
    z = np.zeros((4, 9))
    assert np.array_equal(oracle.newton_schulz(z), z)
    p, buf, o = oracle.muon_matrix_step(np.ones((4, 9)), z, z, 0.02, 0.95)
    assert np.array_equal(o, z) and np.array_equal(p, np.ones((4, 9))) and np.array_equal(buf, z)


def test_zero_steps_is_normalized_input():
    g = np.random.default_rng(4).standard_normal((5, 7))
    np.testing.assert_allclose(oracle.newton_schulz(g, 0), g / (np.linalg.norm(g) + 1e-7), rtol=1e-15)


def test_singular_value_band():
    # phi maps [2e-3, 1] into [0.68, 1.21] (scanned on a fine grid), so for a
    # Gaussian 64x128 input, whose normalized singular values all exceed
    # 2e-3, every output singular value lies in that band.
    grid = np.concatenate([np.linspace(2e-3, 1.0, 200001)])
    vals = np.array([phi(v) for v in grid[::7]])
    assert vals.min() >= 0.68 and vals.max() <= 1.21
    g = np.random.default_rng(7).standard_normal((64, 128))
    x = np.linalg.svd(g, compute_uv=False) / np.linalg.norm(g)
    assert x.min() >= 2e-3
    so = np.linalg.svd(oracle.newton_schulz(g), compute_uv=False)
    assert so.min() >= 0.68 and so.max() <= 1.21


def test_momentum_hand_values():
    b, u = oracle.momentum_update(np.zeros(1), np.full(1, 2.0), 0.95)
    assert math.isclose(b[0], 0.1, rel_tol=1e-15) and math.isclose(u[0], 0.195, rel_tol=1e-14)
    b, u = oracle.momentum_update(np.ones(1), np.full(1, 2.0), 0.95)
    assert math.isclose(b[0], 1.05, rel_tol=1e-15) and math.isclose(u[0], 1.0975, rel_tol=1e-14)
    b, u = oracle.momentum_update(np.ones(1), np.full(1, 2.0), 0.95, form="sgd")
    assert math.isclose(b[0], 2.95, rel_tol=1e-15) and math.isclose(u[0], 4.8025, rel_tol=1e-14)
    b, u = oracle.momentum_update(np.ones(1), np.full(1, 2.0), 0.95, nesterov=False)
    assert u[0] == b[0]


def test_zero_init_momentum_forms_agree_after_normalization():
    # With zero-initialized momentum the EMA NS input is (1-beta) times the
    # heavy-ball one at every step, so the orthogonalized update agrees.
    rng = np.random.default_rng(8)
    be, bs = np.zeros((4, 6)), np.zeros((4, 6))
    for _ in range(3):
        g = rng.standard_normal((4, 6))
        be, ue = oracle.momentum_update(be, g, 0.9)
        bs, us = oracle.momentum_update(bs, g, 0.9, form="sgd")
        assert rel(oracle.newton_schulz(ue), oracle.newton_schulz(us)) <= 1e-6


def test_update_scale_hand_values():
    assert math.isclose(oracle.update_scale(64, 128), 0.2 * math.sqrt(128))
    assert math.isclose(oracle.update_scale(2048, 1408), 0.2 * math.sqrt(2048))
    assert oracle.update_scale(64, 128, "original") == 1.0
    assert math.isclose(oracle.update_scale(128, 64, "original"), math.sqrt(2))
    assert oracle.update_scale(5, 3, "none") == 1.0


def test_apply_hand_values():
    p = oracle.apply_update(np.ones(1), np.full(1, 0.5), lr=0.1, scale=2.0, weight_decay=0.1)
    assert math.isclose(p[0], 0.89, rel_tol=1e-15)


def test_nominal_flops():
    assert oracle.nominal_ns_flops(2048, 2048) == 30 * 2048 ** 3
    assert oracle.nominal_ns_flops(2048, 1408) == oracle.nominal_ns_flops(1408, 2048)
    assert oracle.nominal_ns_flops(1408, 2048) == 5 * (4 * 1408 ** 2 * 2048 + 2 * 1408 ** 3)


def test_expert_bank_is_not_flattened():
    # An [E, M, N] weight is E matrices; orthogonalizing the flattened
    # [E, M*N] matrix is a different result.
    rng = np.random.default_rng(10)
    w = rng.standard_normal((3, 4, 5))
    per = np.stack([oracle.newton_schulz(w[e]) for e in range(3)])
    flat = oracle.newton_schulz(w.reshape(3, 20)).reshape(3, 4, 5)
    assert rel(per, flat) > 0.1
    for e in range(3):  # each expert's update has singular values near 1
        s = np.linalg.svd(per[e], compute_uv=False)
        assert s.min() > 0.5


def test_batch_is_per_matrix():
    rng = np.random.default_rng(11)
    mats = [(rng.standard_normal((r, c)), rng.standard_normal((r, c)), rng.standard_normal((r, c)))
            for r, c in [(3, 5), (5, 3), (4, 4)]]
    out = oracle.muon_step(mats, 0.02, 0.95)
    for (p, g, b), (p1, b1, o1) in zip(mats, out):
        p2, b2, o2 = oracle.muon_matrix_step(p, g, b, 0.02, 0.95)
        assert np.array_equal(p1, p2) and np.array_equal(b1, b2) and np.array_equal(o1, o2)


# ---------------------------------------------------------------------------
# torch.optim.Muon (library routine, run as a black box on the CPU)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("adjust, rule", [("match_rms_adamw", "rms"), ("original", "original")])
def test_against_torch_muon(adjust, rule):
    torch = pytest.importorskip("torch")
    if not hasattr(torch.optim, "Muon"):
        pytest.skip("torch.optim.Muon not available")
    rng = np.random.default_rng(12)
    shapes = [(16, 24), (24, 16), (20, 20)]
    lr, beta, wd = 0.02, 0.95, 0.05
    ps = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    bufs = [np.zeros(s, np.float32) for s in shapes]
    tparams = [torch.nn.Parameter(torch.from_numpy(p.copy())) for p in ps]
    opt = torch.optim.Muon(tparams, lr=lr, momentum=beta, weight_decay=wd, adjust_lr_fn=adjust)
    for step in range(2):
        gs = [rng.standard_normal(s).astype(np.float32) for s in shapes]
        for tp, g in zip(tparams, gs):
            tp.grad = torch.from_numpy(g.copy())
        before = [tp.detach().numpy().astype(np.float64).copy() for tp in tparams]
        opt.step()
        for i, (tp, g) in enumerate(zip(tparams, gs)):
            p1, b1, o = oracle.muon_matrix_step(before[i], g, bufs[i], lr, beta, 5,
                                                weight_decay=wd, scale_rule=rule)
            tb = opt.state[tp]["momentum_buffer"].numpy()
            assert rel(tb, b1) <= 1e-6, (step, i)
            d_t = tp.detach().numpy().astype(np.float64) - before[i]
            d_o = p1 - before[i]
            assert rel(d_t, d_o) <= 3e-2, (step, i, rel(d_t, d_o))
            bufs[i] = tb.astype(np.float64)


# ---------------------------------------------------------------------------
# Planted mistakes: each pin above must reject a plausible error.
# ---------------------------------------------------------------------------

def _mutant(kind):
    def ns(g, steps=5, coeffs=om.QUINTIC_COEFFS, eps=1e-7):
        x = np.asarray(g, np.float64)
        t = x.shape[0] > x.shape[1]
        if t:
            x = x.T
        x = x / (np.linalg.norm(x) + (0.0 if kind == "no_eps" else eps))
        for k in range(steps):
            a, b, c = coeffs
            if kind == "swap_bc":
                b, c = c, b
            A = x @ x.T
            B = b * A + c * (A @ A) if kind != "drop_cubic" else c * (A @ A)
            x = a * x + (x @ B if kind == "right_side" else B @ x)
        return x.T if t else x
    return ns


@pytest.mark.parametrize("kind, case", [("no_eps", "small_norm_8x12"), ("swap_bc", "16x40"),
                                        ("drop_cubic", "16x40"), ("right_side", "4x4_square")])
def test_planted_mistakes_are_caught(kind, case):
    g = _cases()[case]
    assert check_closed_form(oracle.newton_schulz, g)
    assert not check_closed_form(_mutant(kind), g)


def test_planted_momentum_mistake_is_caught():
    # a look-ahead that uses the old buffer instead of the updated one
    buf, g, beta = np.zeros(1), np.full(1, 2.0), 0.95
    wrong_u = (1 - beta) * g + beta * buf
    _, u = oracle.momentum_update(buf, g, beta)
    assert not math.isclose(wrong_u[0], 0.195) and math.isclose(u[0], 0.195)


def test_golden_tiny_fp32_regression():
    # Oracle-written anchor (tests/golden/make_golden.py); a change here
    # means the oracle's arithmetic changed.
    import json
    import os
    import workloads
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_fp32_seed0.json")
    gold = json.load(open(path))
    w = workloads.WORKLOADS["tiny_fp32"]
    for rec, (gi, j, r, c) in zip(gold["matrices"], w.matrices()):
        g = workloads.grad(w, gi, j).as_f64()
        b = workloads.momentum(w, gi, j).astype(np.float64)
        p = workloads.params(w, gi, j).as_f64()
        p1, b1, o = oracle.muon_matrix_step(p, g, b, w.lr, w.beta, w.ns_steps)
        np.testing.assert_allclose(p1[0, :8], rec["p1_first_row_8"], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(b1[0, :8], rec["momentum1_first_row_8"], rtol=1e-12)
        assert math.isclose(np.linalg.norm(p1), rec["p1_frobenius"], rel_tol=1e-12)
