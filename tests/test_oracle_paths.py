"""Pins for the oracle's exact best path and sampled commit (CPU only).

Exact best path (LiLiCorr paper, Appendix E, Eq. (12)): pinned by brute force
over every path of tiny lattices (maximum float32 total; among equal totals
the path that is smallest compared from the last slot backward), by hand-worked
fixtures in tests/golden/paths_hand.json, by its relation to the greedy walk
(never a lower total; identical for two slots, for alpha = 0 and for K = 1).

Sampled commit (SGLang PR, "Sampling the committed path (opt-in)"): pinned by a
hand-worked draw fixture, by a chi-square test of the draw frequencies against
scipy's softmax, by greedy rows reproducing the greedy walk bit for bit, and by
the vanishing-temperature limit.
"""
import itertools
import json
import os

import numpy as np
import pytest
from scipy import special, stats

from oracle.paths import best_path, path_total, sample_path
from oracle.walk import greedy_walk, step_scores

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fixture():
    return json.load(open(os.path.join(GOLDEN, "paths_hand.json")))


def _arrays(c):
    return (np.array(c["idx"]), np.array(c["logp"], dtype=np.float32),
            np.array(c["cos"], dtype=np.float32))


def test_hand_fixture_exact_and_greedy():
    for c in _fixture()["cases"]:
        idx, logp, cos = _arrays(c)
        r = best_path(idx, logp, cos, c["alpha"])
        assert r.choice.tolist() == c["exact_choice"], c["name"]
        assert r.tokens.tolist() == c["exact_tokens"], c["name"]
        assert r.score.tolist() == c["exact_score"], c["name"]
        assert float(r.total) == c["exact_total"], c["name"]
        g = greedy_walk(idx, logp, cos, c["alpha"])
        assert g.choice.tolist() == c["greedy_choice"], c["name"]
        assert float(path_total(logp, cos, g.choice, c["alpha"])) == c["greedy_total"], c["name"]


def _lattice(rng, B, K, kind):
    if kind == "dyadic":     # few distinct values: many exact ties, every float32 sum exact
        logp = rng.choice([-1.0, -0.5, 0.0], size=(B, K)).astype(np.float32)
        cos = rng.choice([-0.5, 0.0, 0.5], size=(B - 1, K, K)).astype(np.float32)
    else:
        logp = -np.abs(rng.standard_normal((B, K))).astype(np.float32)
        cos = rng.uniform(-1, 1, size=(B - 1, K, K)).astype(np.float32)
    return rng.integers(0, 1000, size=(B, K)), logp, cos


@pytest.mark.parametrize("B,K", [(2, 3), (3, 2), (3, 4), (4, 3), (5, 2), (5, 4), (6, 3)])
@pytest.mark.parametrize("kind", ["dyadic", "random"])
@pytest.mark.parametrize("alpha,use_logp", [(1.0, True), (0.5, True), (8.0, False)])
def test_brute_force_best_path(B, K, kind, alpha, use_logp):
    rng = np.random.default_rng(1000 * B + 10 * K + len(kind) + int(alpha * 4))
    for _ in range(4):
        idx, logp, cos = _lattice(rng, B, K, kind)
        best, best_key = None, None
        for tail in itertools.product(range(K), repeat=B - 1):
            path = (0,) + tail
            g = float(path_total(logp, cos, path, alpha, use_logp))
            # larger total first; on equal totals the path smallest when read
            # from the last slot backward
            key = (g, tuple(-c for c in reversed(path)))
            if best_key is None or key > best_key:
                best_key, best = key, path
        r = best_path(idx, logp, cos, alpha, use_logp)
        assert float(r.total) == best_key[0]
        assert tuple(r.choice.tolist()) == best
        assert r.tokens.tolist() == [int(idx[s][best[s]]) for s in range(B)]


def test_exact_never_below_greedy():
    rng = np.random.default_rng(17)
    for _ in range(200):
        B, K = int(rng.integers(2, 17)), int(rng.integers(1, 9))
        idx, logp, cos = _lattice(rng, B, K, "random")
        g = greedy_walk(idx, logp, cos, 1.0)
        e = best_path(idx, logp, cos, 1.0)
        assert float(e.total) >= float(path_total(logp, cos, g.choice, 1.0))


def test_two_slots_alpha_zero_and_k1_equal_greedy():
    rng = np.random.default_rng(18)
    for _ in range(50):
        K = int(rng.integers(1, 9))
        idx, logp, cos = _lattice(rng, 2, K, "dyadic")
        assert np.array_equal(best_path(idx, logp, cos).choice, greedy_walk(idx, logp, cos).choice)
        B = int(rng.integers(2, 17))
        idx, logp, cos = _lattice(rng, B, K, "random")
        # alpha = 0 decouples the slots: every slot's own argmax, as the greedy walk
        assert np.array_equal(best_path(idx, logp, cos, 0.0).choice,
                              greedy_walk(idx, logp, cos, 0.0).choice)
        idx, logp, cos = _lattice(rng, B, 1, "random")
        assert best_path(idx, logp, cos).choice.tolist() == [0] * B


@pytest.mark.parametrize("case", ["sample", "sample_boundary"])
def test_sample_hand_fixture(case):
    f = _fixture()[case]
    idx, logp, cos = _arrays(f)
    for u, expect in f["draws"]:
        r = sample_path(idx, logp, cos, f["temperature"], [0.0, u], f["alpha"])
        assert r.choice.tolist() == [0, expect]
        assert r.tokens.tolist() == [5, [7, 8][expect]]
        assert np.allclose(r.proposal[1], f["q1"], rtol=0, atol=1e-15)
        assert r.proposal[0].tolist() == [1.0, 0.0]


def test_sample_frequencies_match_softmax():
    # one drafted slot with fixed scores; 20000 draws at T = 0.7
    rng = np.random.default_rng(19)
    K, T, n = 5, 0.7, 20000
    logp = np.stack([np.zeros(K), -np.abs(rng.standard_normal(K))]).astype(np.float32)
    cos = rng.uniform(-1, 1, size=(1, K, K)).astype(np.float32)
    idx = np.arange(2 * K).reshape(2, K)
    z = step_scores(logp[1], cos[0][0], 1.0, True)
    q = special.softmax(z.astype(np.float64) / T)
    u = rng.random(n, dtype=np.float32)
    counts = np.zeros(K)
    for x in u:
        counts[sample_path(idx, logp, cos, T, [0.0, x]).choice[1]] += 1
    chi2, p = stats.chisquare(counts, q * n)
    assert p > 1e-4, (counts, q * n)
    r = sample_path(idx, logp, cos, T, [0.0, 0.5])
    assert np.allclose(r.proposal[1], q, rtol=1e-12)


def test_greedy_rows_and_cold_limit():
    rng = np.random.default_rng(20)
    for _ in range(40):
        B, K = int(rng.integers(2, 17)), int(rng.integers(1, 9))
        idx, logp, cos = _lattice(rng, B, K, "dyadic")
        u = rng.random(B, dtype=np.float32)
        g = greedy_walk(idx, logp, cos)
        for T in (0.0, -1.0):
            r = sample_path(idx, logp, cos, T, u)
            assert np.array_equal(r.choice, g.choice)
            assert np.array_equal(r.proposal, np.eye(K)[g.choice])
        idx, logp, cos = _lattice(rng, B, K, "random")    # no ties: distinct scores
        g = greedy_walk(idx, logp, cos)
        # at a temperature far below every score gap the draw is the argmax
        # unless u falls in the (underflowed) tail
        r = sample_path(idx, logp, cos, 1e-4, np.full(B, 0.5, dtype=np.float32))
        assert np.array_equal(r.choice, g.choice)


def test_sample_proposals_are_distributions():
    rng = np.random.default_rng(21)
    idx, logp, cos = _lattice(rng, 16, 8, "random")
    u = rng.random(16, dtype=np.float32)
    r = sample_path(idx, logp, cos, 1.3, u)
    assert np.allclose(r.proposal.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(r.proposal >= 0)
    # the drawn candidate's cumulative interval contains u
    for s in range(1, 16):
        c = r.choice[s]
        lo = r.cdf[s][c - 1] if c > 0 else 0.0
        assert lo <= u[s] < r.cdf[s][c]
