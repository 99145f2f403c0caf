"""Statistical pins of the oracle's sampler on the tiny workload (CPU only).

10**6 independent trials of one block (V = 64, L = 4, T = 1, z ~ N(0,1),
d = z + N(0, 0.5^2)), with drafts drawn from q by the oracle's inverse CDF
(Philox stream 1) and acceptance/redraw uniforms from Philox stream 0:

* the first emitted token must pass a chi-square test against p_0 at
  alpha = 0.01 (63 degrees of freedom);
* the prefix completed with fresh AR draws must pass the same test at every
  later position (Bonferroni alpha/4);
* the mean number of emitted tokens must lie within 5 standard errors of
  sum_m prod_{i<m} alpha_i with alpha_i = sum_k min(p_ik, q_ik).
"""

import numpy as np
from scipy import stats

import oracle
from synthetic import WORKLOADS, verify_inputs

TRIALS = 1_000_000
CHUNK = 200_000


def _run_trials(z, d, L, T, has_bonus, seed=0):
    V = z.shape[-1]
    first = np.zeros(V, np.int64)
    emitted = np.zeros(TRIALS, np.int64)
    tokens = np.zeros((TRIALS, L + 1), np.int64)
    for c0 in range(0, TRIALS, CHUNK):
        n = min(CHUNK, TRIALS - c0)
        ud = oracle.philox_uniforms(seed, 1, c0 * L, n * L).reshape(n, L)
        x = np.stack([oracle.draft_sample(d[:, i, :], ud[:, i], T) for i in range(L)], axis=1)
        u = oracle.philox_uniforms(seed, 0, c0 * (L + 1), n * (L + 1)).reshape(n, L + 1)
        res = oracle.block_verify(z, d, x, u, T, has_bonus)
        first += np.bincount(res["out_tokens"][:, 0], minlength=V)
        emitted[c0:c0 + n] = res["n_emitted"]
        tokens[c0:c0 + n] = res["out_tokens"]
    return first, emitted, tokens


def test_tiny_workload_is_lossless_on_the_oracle():
    wl = WORKLOADS["tiny"]
    L, V, T = wl.block, wl.vocab, wl.temperatures[0]
    z, d = verify_inputs(1, L, V, wl.seed, "normal", wl.target_sigma, wl.draft_sigmas[0],
                         has_bonus=False, dtype="f32")
    p = np.exp(oracle.log_softmax(z[0], T))
    q = np.exp(oracle.log_softmax(d[0], T))
    first, emitted, tokens = _run_trials(z, d, L, T, False)

    expected = p[0] * TRIALS
    assert expected.min() >= 5
    chi0 = stats.chisquare(first, expected)
    assert chi0.pvalue >= 0.01, chi0

    # completed marginals: positions not emitted are filled with fresh draws from p_j
    rng = np.random.default_rng(77)
    for j in range(1, L):
        col = tokens[:, j].copy()
        missing = emitted <= j
        col[missing] = rng.choice(V, size=int(missing.sum()), p=p[j] / p[j].sum())
        res = stats.chisquare(np.bincount(col, minlength=V), p[j] * TRIALS)
        assert res.pvalue >= 0.01 / 4, (j, res)

    alpha = np.minimum(p, q).sum(axis=1)
    expect = sum(np.prod(alpha[:m]) for m in range(L))
    se = emitted.std() / np.sqrt(TRIALS)
    assert abs(emitted.mean() - expect) < 5 * se, (emitted.mean(), expect, se)
