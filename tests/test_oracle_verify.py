"""Pins for the oracle's softmax, acceptance, scan, redraw and emit steps (CPU only).

Against: SciPy's logsumexp and closed forms for the softmax; hand-derived
cases (tests/golden/verify_hand.json); exact integration over every draft
sequence and every decision region at V=8, L=3, showing that the emitted
tokens follow the AR distribution exactly (the pages' lossless property),
in both bonus modes and with masked tokens; the closed forms
P(accept) = sum_k min(p_k, q_k) and E[n_emitted]; the special cases
q = p, disjoint supports and one-hot drafts; and a grid test of the
inverse CDF.
"""

import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle import verify as ov


# ---------------------------------------------------------------- softmax


def test_log_softmax_matches_scipy_logsumexp():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((5, 37)) * 4
    for T in (0.6, 1.0, 2.5):
        ref = z / T - logsumexp(z / T, axis=-1, keepdims=True)
        np.testing.assert_allclose(ov.log_softmax(z, T), ref, rtol=0, atol=1e-13)


def test_log_softmax_closed_forms():
    # two tokens: p_0 = sigmoid(z0 - z1)
    z = np.array([[1.5, -0.5]])
    p = np.exp(ov.log_softmax(z))
    assert abs(p[0, 0] - 1 / (1 + np.exp(-2.0))) < 1e-15
    # equal logits: uniform
    np.testing.assert_allclose(np.exp(ov.log_softmax(np.full((1, 10), 3.0))), 0.1, atol=1e-16)
    # shift invariance and temperature as a logit scale
    z = np.random.default_rng(1).standard_normal((3, 20))
    np.testing.assert_allclose(ov.log_softmax(z + 7.0), ov.log_softmax(z), atol=1e-13)
    np.testing.assert_allclose(ov.log_softmax(z, 0.5), ov.log_softmax(2 * z, 1.0), atol=1e-13)
    # masked tokens get probability zero
    zm = np.array([[0.0, -np.inf, 0.0]])
    np.testing.assert_array_equal(np.exp(ov.log_softmax(zm)), [[0.5, 0.0, 0.5]])


# ---------------------------------------------------------------- golden


def test_hand_derived_cases(repo_root):
    with open(os.path.join(repo_root, "tests", "golden", "verify_hand.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        p = [list(r) for r in g["p"]]
        if "p0_override" in case:
            p[0] = case["p0_override"]
        with np.errstate(divide="ignore"):
            z = np.log(np.array(p, float))[None]
            d = np.log(np.array(g["q"], float))[None]
        res = ov.block_verify(z, d, np.array([case["x"]]), np.array([case["u"]]), 1.0,
                              case["has_bonus"])
        assert res["n_accepted"][0] == case["n_accepted"], case["name"]
        assert list(res["out_tokens"][0]) == case["out_tokens"], case["name"]
        assert res["n_emitted"][0] == case["n_emitted"], case["name"]


def _residual_golden_failures(fn, repo_root):
    """Hand-derived residual laws (tests/golden/verify_hand.json) that fn gets wrong."""
    with open(os.path.join(repo_root, "tests", "golden", "verify_hand.json")) as f:
        g = json.load(f)
    fails = []
    for case in g["residual_cases"]:
        with np.errstate(divide="ignore"):
            lp = np.log(np.array(case["p"], float))
            lq = np.log(np.array(case["q"], float))
        w, fb = fn(lp, lq, with_fallback=True)
        if not (np.allclose(w, case["residual"], rtol=0, atol=1e-15) and bool(fb) == case["fallback"]):
            fails.append(case["name"])
        if not np.allclose(fn(lp, lq), case["residual"], rtol=0, atol=1e-15):
            fails.append(case["name"] + " (weights only)")
    return fails


def test_residual_weights_hand_derived(repo_root):
    assert _residual_golden_failures(ov.residual_weights, repo_root) == []


def test_residual_pins_catch_planted_mistakes(repo_root):
    """Plausible mistakes in the residual (sign, |p - q|, no clamp, no fallback) each fail a pin."""
    def plant(kind):
        def fn(lp, lq, with_fallback=False):
            p, q = np.exp(lp), np.exp(lq)
            r = {"q-p": np.maximum(0.0, q - p), "abs": np.abs(p - q),
                 "nofallback": np.maximum(0.0, p - q), "nomax": p - q}[kind]
            zero = np.sum(r, axis=-1, keepdims=True) == 0.0
            if kind == "nofallback":
                w = r
            else:
                w = np.where(zero, p, r)
            return (w, zero[..., 0]) if with_fallback else w
        return fn
    for kind in ("q-p", "abs", "nofallback", "nomax"):
        assert _residual_golden_failures(plant(kind), repo_root), kind


# ---------------------------------------------------------------- exact integration


def _rational_rows(rng, rows, V, zero_frac=0.0):
    out = []
    for _ in range(rows):
        w = rng.integers(1, 10, V)
        if zero_frac:
            w[rng.random(V) < zero_frac] = 0
            if w.sum() == 0:
                w[0] = 1
        s = int(w.sum())
        out.append([Fraction(int(v), s) for v in w])
    return out


def _exact_output_law(p, q, L, has_bonus):
    """Integrate the oracle's decisions over every draft and every uniform cell.

    The oracle's output is piecewise constant in the uniforms: acceptance of
    position i changes only at a_i = min(1, p_i(x_i)/q_i(x_i)), and the redraw
    changes only at the boundaries C_k/R of the redraw distribution.  Each cell
    is evaluated once, at its midpoint, and weighted by its exact measure.
    """
    V = len(p[0])
    with np.errstate(divide="ignore"):
        z = np.log(np.array([[float(v) for v in r] for r in p]))[None]
        d = np.log(np.array([[float(v) for v in r] for r in q]))[None]
    X, U, W = [], [], []
    for x in itertools.product(range(V), repeat=L):
        wq = Fraction(1)
        for i in range(L):
            wq *= q[i][x[i]]
        if wq == 0:
            continue
        a = [min(Fraction(1), p[i][x[i]] / q[i][x[i]]) for i in range(L)]
        for choice in itertools.product((True, False), repeat=L):
            w = wq
            for i, c in enumerate(choice):
                w *= a[i] if c else 1 - a[i]
            if w == 0:
                continue
            u = [float(a[i] / 2) if c else float((1 + a[i]) / 2) for i, c in enumerate(choice)]
            n = choice.index(False) if False in choice else L
            if n < L:
                r = [max(Fraction(0), p[n][k] - q[n][k]) for k in range(V)]
                if sum(r) == 0:
                    r = list(p[n])
            elif has_bonus:
                r = list(p[L])
            else:
                r = None
            if r is None:
                cells = [(Fraction(1, 2), Fraction(1))]
            else:
                R = sum(r)
                cells, c = [], Fraction(0)
                for k in range(V):
                    if r[k] > 0:
                        cells.append(((2 * c + r[k]) / (2 * R), r[k] / R))
                    c += r[k]
            for mid, width in cells:
                X.append(x)
                U.append(u + [float(mid)])
                W.append(w * width)
    res = ov.block_verify(z, d, np.array(X), np.array(U), 1.0, has_bonus)
    law = {}
    for b in range(len(X)):
        n = int(res["n_emitted"][b])
        key = tuple(int(t) for t in res["out_tokens"][b][:n])
        law[key] = law.get(key, Fraction(0)) + W[b]
    return law


@pytest.mark.parametrize("has_bonus", [False, True])
@pytest.mark.parametrize("zero_frac", [0.0, 0.3])
def test_exact_output_law_is_the_ar_distribution(has_bonus, zero_frac):
    V, L = 8, 3
    rng = np.random.default_rng(100 + int(has_bonus) + int(10 * zero_frac))
    p = _rational_rows(rng, L + 1, V, zero_frac)
    q = _rational_rows(rng, L, V, zero_frac)
    law = _exact_output_law(p, q, L, has_bonus)
    assert abs(float(sum(law.values())) - 1.0) < 1e-12
    n_pos = L + (1 if has_bonus else 0)
    # (i) the first emitted token is distributed as p_0
    first = np.zeros(V)
    for key, pr in law.items():
        first[key[0]] += float(pr)
    np.testing.assert_allclose(first, [float(v) for v in p[0]], rtol=0, atol=1e-12)
    # (ii) the emitted prefix completed with fresh AR draws has joint prod_j p_j
    for w in itertools.product(range(V), repeat=n_pos):
        want = 1.0
        for j in range(n_pos):
            want *= float(p[j][w[j]])
        got = 0.0
        for key, pr in law.items():
            n = len(key)
            if tuple(w[:n]) == key:
                tail = 1.0
                for j in range(n, n_pos):
                    tail *= float(p[j][w[j]])
                got += float(pr) * tail
        assert abs(got - want) < 1e-12, (w, got, want)
    # expected emitted length: sum over m of prod_{i<m} alpha_i, alpha_i = sum_k min(p_ik, q_ik)
    alpha = [float(sum(min(p[i][k], q[i][k]) for k in range(V))) for i in range(L)]
    expect = sum(np.prod(alpha[:m]) for m in range(L + (1 if has_bonus else 0)))
    mean = sum(len(k) * float(pr) for k, pr in law.items())
    assert abs(mean - expect) < 1e-12


def test_acceptance_identity_is_one_minus_tv():
    rng = np.random.default_rng(5)
    for _ in range(20):
        V = int(rng.integers(2, 50))
        p = rng.dirichlet(np.ones(V))
        q = rng.dirichlet(np.ones(V))
        a = ov.acceptance_probability(np.log(p), np.log(q))
        assert abs(np.sum(q * a) - np.sum(np.minimum(p, q))) < 1e-14
        assert abs(np.sum(q * a) - (1 - 0.5 * np.sum(np.abs(p - q)))) < 1e-14


# ---------------------------------------------------------------- special cases


def test_q_equal_p_accepts_everything():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((4, 6, 30))
    x = rng.integers(0, 30, (4, 6))
    u = np.full((4, 7), 1 - 2.0 ** -24)
    res = ov.block_verify(z, z, x, u, 0.8, False)
    assert np.all(res["n_accepted"] == 6) and np.all(res["n_emitted"] == 6)
    np.testing.assert_array_equal(res["out_tokens"][:, :6], x)


def test_disjoint_supports_reject_first_and_redraw_from_p():
    V = 10
    z = np.full((1, 2, V), -np.inf)
    z[0, :, :5] = np.log(np.arange(1, 6) / 15.0)
    d = np.full((1, 2, V), -np.inf)
    d[0, :, 5:] = 0.0
    n = 4000
    x = np.tile([[7, 8]], (n, 1))
    u = np.column_stack([np.zeros(n), np.zeros(n), (np.arange(n) + 0.5) / n])
    res = ov.block_verify(z, d, x, u, 1.0, False)
    assert np.all(res["n_accepted"] == 0) and np.all(res["n_emitted"] == 1)
    counts = np.bincount(res["out_tokens"][:, 0], minlength=V)
    np.testing.assert_allclose(counts / n, [1 / 15, 2 / 15, 3 / 15, 4 / 15, 5 / 15, 0, 0, 0, 0, 0],
                               atol=1.0 / n)


def test_one_hot_draft_accepts_with_probability_p_of_x():
    V = 6
    p = np.array([0.1, 0.2, 0.3, 0.15, 0.15, 0.1])
    z = np.log(p)[None, None]
    d = np.full((1, 1, V), -np.inf)
    d[0, 0, 2] = 0.0
    assert ov.acceptance_probability(np.log(p[2]), 0.0) == pytest.approx(0.3, abs=1e-15)
    n = 10000
    u = np.column_stack([(np.arange(n) + 0.5) / n, np.full(n, 0.5)])
    res = ov.block_verify(z, d, np.full((n, 1), 2), u, 1.0, False)
    assert abs(np.mean(res["n_accepted"] == 1) - 0.3) <= 1.0 / n


def test_single_token_vocabulary():
    res = ov.block_verify(np.zeros((1, 4, 1)), np.zeros((1, 3, 1)), np.zeros((2, 3), int),
                          np.full((2, 4), 0.7), 1.0, True)
    np.testing.assert_array_equal(res["n_accepted"], [3, 3])
    np.testing.assert_array_equal(res["out_tokens"], [[0, 0, 0, 0], [0, 0, 0, 0]])
    np.testing.assert_array_equal(res["n_emitted"], [4, 4])


def test_out_of_range_draft_token_sets_sentinel():
    z = np.zeros((2, 2, 4))
    res = ov.block_verify(z, z, np.array([[0, 4], [1, -1]]), np.full((2, 3), 0.5), 1.0, False)
    np.testing.assert_array_equal(res["n_accepted"], [-1, -1])
    np.testing.assert_array_equal(res["n_emitted"], [0, 0])
    assert np.all(res["out_tokens"] == -1)


# ---------------------------------------------------------------- inverse CDF


def test_inverse_cdf_strict_rule_on_exact_weights():
    w = np.array([1.0, 1.0, 2.0])          # C = (1, 2, 4), R = 4
    assert ov.inverse_cdf(w, 0.0) == 0
    assert ov.inverse_cdf(w, 0.25) == 1    # u R = 1 = C_0, not > 1
    assert ov.inverse_cdf(w, 0.5) == 2
    assert ov.inverse_cdf(w, 1 - 2.0 ** -24) == 2
    w0 = np.array([0.0, 3.0, 0.0, 1.0])
    assert ov.inverse_cdf(w0, 0.0) == 1    # zero-mass token 0 is never chosen
    assert ov.inverse_cdf(w0, 0.75) == 3


def test_inverse_cdf_grid_frequencies():
    rng = np.random.default_rng(9)
    w = rng.random(40)
    w[rng.random(40) < 0.25] = 0.0
    G = 1 << 20
    u = np.arange(G) / G
    tok = ov.inverse_cdf(np.broadcast_to(w, (G, 40)), u)
    counts = np.bincount(tok, minlength=40)
    expect = w / w.sum() * G
    assert np.all(np.abs(counts - expect) <= 1.0)
    assert np.all(counts[w == 0] == 0)


def test_draft_sample_frequencies():
    z = np.array([[0.0, np.log(3.0), -np.inf, np.log(4.0)]])
    G = 1 << 16
    u = np.arange(G) / G
    tok = ov.draft_sample(np.broadcast_to(z, (G, 4)), u)
    counts = np.bincount(tok, minlength=4)
    assert np.all(np.abs(counts - np.array([1, 3, 0, 4]) / 8 * G) <= 1)
