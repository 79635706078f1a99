"""Pins of the oracle's sampler variants (CPU only): the Gumbel-max token
draw, the sorted cumulative entropy bound and the stability count."""
import numpy as np
import scipy.stats

from oracle import dg_oracle as O


def _scfg(V, **kw):
    c = dict(vocab=V, tau=1.0, t_max=1.0, t_min=1.0, n_steps=48, step=0, canvas_idx=0, seed=1, final_step=False)
    c.update(kw)
    return c


def test_gumbel_noise_has_gumbel_distribution():
    g = O.gumbel_noise(np.arange(8), 4096, seed=5, step=3, canvas_idx=1).ravel()
    # Gumbel(0,1): mean = Euler-Mascheroni constant, variance = pi^2 / 6; and a KS test
    assert abs(g.mean() - np.euler_gamma) < 0.03
    assert abs(g.var() - np.pi ** 2 / 6) < 0.06
    assert scipy.stats.kstest(g, "gumbel_r").pvalue > 1e-3


def test_gumbel_max_draws_follow_the_tempered_softmax():
    """Gumbel-max property: argmax(l/t + g) ~ softmax(l/t).  Independent draws
    come from distinct (step, canvas) counters."""
    logits = np.array([[0.3, -1.0, 2.0, 0.0, 1.2, -0.4]])
    t = 0.8
    p = np.exp(logits[0] / t) / np.exp(logits[0] / t).sum()
    counts = np.zeros(6)
    for canvas in range(3000):
        r = O.sample_renoise(logits, _scfg(6, t_max=t, t_min=t, step=canvas % 48, canvas_idx=canvas,
                                           token_rule="gumbel"))
        counts[r["pred"][0]] += 1
    assert scipy.stats.chisquare(counts, p * counts.sum()).pvalue > 1e-3


def test_gumbel_at_low_temperature_is_the_argmax_and_shift_invariant():
    g = np.random.default_rng(4)
    logits = g.normal(0, 3, size=(16, 500))
    cold = O.sample_renoise(logits, _scfg(500, t_max=1e-4, t_min=1e-4, token_rule="gumbel"))
    assert np.array_equal(cold["pred"], np.argmax(logits, axis=1))
    a = O.sample_renoise(logits, _scfg(500, token_rule="gumbel", seed=9))
    b = O.sample_renoise(logits + 7.5, _scfg(500, token_rule="gumbel", seed=9))
    clear = a["gumbel_margin"] > 1e-9
    assert np.array_equal(a["pred"][clear], b["pred"][clear])


def test_sorted_cumulative_worked_example():
    # ascending order: pos 0 (0.1), pos 2 (0.2), pos 1 (0.5), pos 3 (3.0), pos 4 (3.0)
    H = np.array([0.1, 0.5, 0.2, 3.0, 3.0])
    commit, prior = O.sorted_cumulative_commit(H, 0.35)
    assert list(commit) == [True, True, True, False, False]
    assert np.allclose(prior, [0.0, 0.3, 0.1, 0.8, 3.8])
    # ties go to the lower position: pos 3 ranks before pos 4
    commit, _ = O.sorted_cumulative_commit(H, 3.8)
    assert list(commit) == [True, True, True, True, True]
    commit, _ = O.sorted_cumulative_commit(H, 3.79)
    assert list(commit) == [True, True, True, True, False]


def test_sorted_cumulative_is_a_sorted_prefix_and_monotone():
    g = np.random.default_rng(8)
    for trial in range(50):
        n = int(g.integers(1, 40))
        H = np.round(g.exponential(1.0, size=n), 2)     # ties happen
        bound = float(g.uniform(0, 10))
        commit, prior = O.sorted_cumulative_commit(H, bound)
        order = sorted(range(n), key=lambda j: (H[j], j))
        flags = commit[order]
        k = int(flags.sum())
        assert k >= 1 and flags[:k].all() and not flags[k:].any()       # a prefix, never empty
        # brute force: the largest prefix U with sum(U) - max(U) <= bound
        best = max(kk for kk in range(1, n + 1) if H[order[:kk]].sum() - H[order[kk - 1]] <= bound + 1e-12)
        assert k == best
        bigger, _ = O.sorted_cumulative_commit(H, bound + 1.0)
        assert (bigger | ~commit).all()                  # monotone in the bound


def test_variants_final_step_and_stability_count():
    g = np.random.default_rng(2)
    logits = g.normal(0, 1, size=(12, 64)) * np.linspace(0, 8, 12)[:, None]
    s = _scfg(64, tau=5.0, commit_rule="sorted_cumulative", token_rule="gumbel")
    r0 = O.sample_renoise(logits, s)
    assert r0["n_renoised"] == int((~r0["commit"]).sum()) and r0["n_changed"] is None
    committed = r0["commit"]
    assert np.array_equal(r0["tokens"][committed], r0["pred"][committed])
    r1 = O.sample_renoise(logits, dict(s, step=1), pred_prev=r0["pred"])
    assert r1["n_changed"] == int((r1["pred"] != r0["pred"]).sum())
    r2 = O.sample_renoise(logits, dict(s, step=1), pred_prev=r1["pred"])
    assert r2["n_changed"] == 0
    fin = O.sample_renoise(logits, dict(s, final_step=True))
    assert fin["commit"].all() and np.array_equal(fin["tokens"], fin["pred"])
