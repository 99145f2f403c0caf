"""Pins for the tree-verification oracle (CPU only).

The emitted sequence must follow the AR law: the first token has law p_root,
and each later token, given that the tokens before it walk a tree path to
node v, has law p_v.  This is checked exactly (every inverse-CDF cell of
every depth enumerated, the weights summed per emitted sequence, against
the product of the AR probabilities along the sequence), by a chi-square
test over random uniforms, on a grid of first draws against inverse_cdf,
and on degenerate trees (certain tokens, impossible children, duplicates,
malformed trees).
"""

import itertools

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import tree

BIN_TREE = (np.array([-1, 0, 0, 1, 1, 2, 2]), np.array([0, 1, 3, 0, 2, 1, 3]))  # depth 2, two children per node


def _softmax(z, T=1.0):
    return np.exp(oracle.log_softmax(z, T))


def _ar_probability(seq, z, parents, tokens, T):
    """AR probability of an emitted sequence on the tree: product of p_v(y)
    along the path the sequence takes (computed from tokens, not uniforms)."""
    prob, v = 1.0, 0
    for j, y in enumerate(seq):
        prob *= _softmax(z[v], T)[y]
        kids = [c for c in range(len(parents)) if parents[c] == v and tokens[c] == y and c > v]
        if j == len(seq) - 1:
            assert not kids, "an emitted sequence ends where the tree has no matching child"
        else:
            v = kids[0]
    return prob


def _cells(p):
    """Midpoint uniform of each positive-mass inverse-CDF cell, and its width."""
    c = np.cumsum(p)
    lo = np.concatenate([[0.0], c[:-1]]) / c[-1]
    hi = c / c[-1]
    return [((a + b) / 2, b - a) for a, b in zip(lo, hi) if b > a]


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_exact_law_by_cell_enumeration(T):
    rng = np.random.default_rng(2)
    par, tok = BIN_TREE
    N, V = len(par), 4
    z = rng.standard_normal((N, V)) * 1.5
    depth_max = int(tree.tree_depths(par).max()) + 1
    law = {}

    def child(v, y):
        return [c for c in range(N) if par[c] == v and tok[c] == y and c > v][0]

    # depth by depth: the cells of depth d are those of the node the path has
    # reached; the oracle runs with those uniforms (later ones arbitrary), and a
    # sequence that stops at depth d adds the product of its cells' widths
    def walk(v, depth, weight, u_sofar):
        for u, w in _cells(_softmax(z[v], T)):
            us = u_sofar + [u] + [0.5] * (N - depth - 1)
            out = tree.tree_verify(z[None], par[None], tok[None], np.array([us]), T)
            e = int(out["n_emitted"][0])
            seq = tuple(int(t) for t in out["out_tokens"][0, :e])
            if e == depth + 1:
                law[seq] = law.get(seq, 0.0) + weight * w
            else:
                walk(child(v, seq[depth]), depth + 1, weight * w, u_sofar + [u])

    walk(0, 0, 1.0, [])
    assert abs(sum(law.values()) - 1.0) < 1e-12
    for seq, pr in law.items():
        assert len(seq) <= depth_max + 1
        assert abs(pr - _ar_probability(seq, z, par, tok, T)) < 1e-12, seq


def test_first_draw_is_inverse_cdf_of_the_root():
    rng = np.random.default_rng(5)
    par, tok = BIN_TREE
    z = rng.standard_normal((len(par), 9))
    p = _softmax(z[0])
    for u0 in np.linspace(0, 1, 257, endpoint=False):
        out = tree.tree_verify(z[None], par[None], tok[None], np.array([[u0] + [0.3] * 6]))
        assert out["out_tokens"][0, 0] == oracle.inverse_cdf(p, u0)


def test_chi_square_two_levels():
    rng = np.random.default_rng(9)
    par = np.array([-1, 0, 0, 0])
    tok = np.array([0, 2, 5, 7])
    V, trials = 8, 60000
    z = rng.standard_normal((4, V))
    u = rng.random((trials, 4))
    out = tree.tree_verify(np.broadcast_to(z, (trials, 4, V)), np.broadcast_to(par, (trials, 4)),
                           np.broadcast_to(tok, (trials, 4)), u)
    p0 = _softmax(z[0])
    child_of = {2: 1, 5: 2, 7: 3}
    cells, expect = {}, {}
    for y in range(V):
        if y in child_of:
            for y2 in range(V):
                expect[(y, y2)] = p0[y] * _softmax(z[child_of[y]])[y2]
        else:
            expect[(y,)] = p0[y]
    for s in range(trials):
        e = out["n_emitted"][s]
        key = tuple(int(t) for t in out["out_tokens"][s, :e])
        cells[key] = cells.get(key, 0) + 1
    keys = sorted(expect)
    obs = np.array([cells.get(k, 0) for k in keys], dtype=float)
    exp = np.array([expect[k] for k in keys]) * trials
    assert obs.sum() == trials
    assert stats.chisquare(obs, exp).pvalue > 1e-4


def test_certain_and_impossible_children():
    V = 6
    par = np.array([-1, 0, 1, 2])
    tok = np.array([0, 3, 1, 4])
    z = np.full((4, V), -np.inf)
    z[0, 3] = z[1, 1] = z[2, 4] = 0.0   # each node certainly draws its child's token
    z[3, 2] = 0.0                       # the leaf's bonus
    out = tree.tree_verify(z[None], par[None], tok[None], np.array([[0.9, 0.1, 0.5, 0.99]]))
    assert out["n_accepted"][0] == 3 and out["last_node"][0] == 3
    assert list(out["out_tokens"][0]) == [3, 1, 4, 2] and out["n_emitted"][0] == 4
    z2 = np.zeros((4, V))
    z2[0, 3] = -np.inf                  # the root's only child is impossible
    out = tree.tree_verify(z2[None], par[None], tok[None], np.array([[0.7, 0.1, 0.5, 0.99]]))
    assert out["n_accepted"][0] == 0 and out["out_tokens"][0, 0] != 3 and list(out["out_tokens"][0, 1:]) == [-1] * 3


def test_duplicate_siblings_take_the_lowest_index_and_malformed_trees_are_flagged():
    V = 4
    z = np.full((4, V), -np.inf)
    z[:, 2] = 0.0
    par = np.array([-1, 0, 0, 1])
    tok = np.array([0, 2, 2, 2])
    out = tree.tree_verify(z[None], par[None], tok[None], np.full((1, 4), 0.5))
    assert out["last_node"][0] == 3 and out["n_accepted"][0] == 2   # via node 1, not node 2
    bad = [(np.array([0, 0, 0, 1]), tok), (np.array([-1, 0, 3, 1]), tok), (par, np.array([0, 2, 4, 2]))]
    for p_, t_ in bad:
        out = tree.tree_verify(z[None], p_[None], t_[None], np.full((1, 4), 0.5))
        assert out["n_accepted"][0] == -1 and out["last_node"][0] == -1 and out["n_emitted"][0] == 0
        assert np.all(out["out_tokens"][0] == -1)
