"""Pins for the oracle's greedy walk and pair scores (CPU only).

The walk (LiLiCorr paper, Eq. (8)) is pinned by: a hand-worked fixture; the
alpha = 0 and K = 1 reductions to the per-slot argmax; an exhaustive
enumeration of all paths on tiny lattices, where the greedy path must be the
lexicographic maximum of the interleaved key (z_1, -c_1, z_2, -c_2, ...);
Markov invariance; and independence of blocks.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.walk import greedy_walk, step_scores
from oracle.scores import pair_scores
from oracle.bf16 import round_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_fixture():
    g = json.load(open(os.path.join(GOLDEN, "walk_hand.json")))
    idx = np.array(g["idx"])
    logp = np.array(g["logp"], dtype=np.float32)
    cos = np.array(g["cos"], dtype=np.float32)
    for case in g["cases"]:
        r = greedy_walk(idx, logp, cos, case["alpha"])
        assert r.choice.tolist() == case["choice"]
        assert r.tokens.tolist() == case["tokens"]
        assert r.score.tolist() == case["score"]
        assert r.gap.tolist() == case["gap"]


def _random_lattice(rng, B, K, coarse):
    if coarse:   # few distinct values -> many exact ties
        logp = rng.choice([-1.0, -0.5, 0.0], size=(B, K)).astype(np.float32)
        cos = rng.choice([-0.5, 0.0, 0.5], size=(B - 1, K, K)).astype(np.float32)
    else:
        logp = -np.abs(rng.standard_normal((B, K))).astype(np.float32)
        cos = rng.uniform(-1, 1, size=(B - 1, K, K)).astype(np.float32)
    idx = rng.integers(0, 1000, size=(B, K))
    return idx, logp, cos


@pytest.mark.parametrize("B,K", [(2, 1), (2, 4), (3, 3), (4, 2), (5, 3), (6, 4)])
@pytest.mark.parametrize("coarse", [True, False])
@pytest.mark.parametrize("alpha", [1.0, 0.5, 8.0])
def test_exhaustive_greedy_enumeration(B, K, coarse, alpha):
    rng = np.random.default_rng(B * 100 + K * 10 + int(coarse) + int(alpha * 3))
    for _ in range(4):
        idx, logp, cos = _random_lattice(rng, B, K, coarse)
        best_key, best_path = None, None
        for tail in itertools.product(range(K), repeat=B - 1):
            path = (0,) + tail
            key = []
            for s in range(1, B):
                z = step_scores(logp[s], cos[s - 1][path[s - 1]], alpha, True)[path[s]]
                key += [float(z), -path[s]]
            if best_key is None or key > best_key:
                best_key, best_path = key, path
        r = greedy_walk(idx, logp, cos, alpha)
        assert tuple(r.choice.tolist()) == best_path


def test_alpha_zero_is_per_slot_argmax():
    rng = np.random.default_rng(5)
    for _ in range(20):
        idx, logp, cos = _random_lattice(rng, 16, 8, coarse=True)
        r = greedy_walk(idx, logp, cos, 0.0)
        expect = np.argmax(logp, axis=1)
        expect[0] = 0
        # logp rows are sorted descending in the real path; here they are not,
        # so slot 0 (fixed to candidate 0) is excluded from the comparison
        assert np.array_equal(r.choice[1:], expect[1:])


def test_k1_is_trivial():
    rng = np.random.default_rng(6)
    idx, logp, cos = _random_lattice(rng, 16, 1, coarse=False)
    r = greedy_walk(idx, logp, cos, 1.0)
    assert np.array_equal(r.choice, np.zeros(16, dtype=np.int64))
    assert np.array_equal(r.tokens, idx[:, 0])


def test_markov_invariance():
    # Rows of cos_s other than the committed c_{s-1} must not matter.
    rng = np.random.default_rng(8)
    for _ in range(20):
        idx, logp, cos = _random_lattice(rng, 12, 6, coarse=False)
        r = greedy_walk(idx, logp, cos, 1.0)
        cos2 = rng.uniform(-1, 1, size=cos.shape).astype(np.float32)
        for s in range(1, 12):
            cos2[s - 1][r.choice[s - 1]] = cos[s - 1][r.choice[s - 1]]
        r2 = greedy_walk(idx, logp, cos2, 1.0)
        assert np.array_equal(r.choice, r2.choice)


def test_blocks_are_independent():
    rng = np.random.default_rng(9)
    blocks = [_random_lattice(rng, 8, 4, coarse=True) for _ in range(5)]
    alone = [greedy_walk(*b, 1.0).tokens for b in blocks]
    order = [3, 1, 4, 0, 2]
    permuted = [greedy_walk(*blocks[i], 1.0).tokens for i in order]
    for j, i in enumerate(order):
        assert np.array_equal(permuted[j], alone[i])


def test_paper_rule_is_scaled_cosine_argmax():
    # use_logp = 0 with alpha = sigma is the paper's phi = sigma * cos rule.
    rng = np.random.default_rng(10)
    idx, logp, cos = _random_lattice(rng, 10, 8, coarse=False)
    r = greedy_walk(idx, logp, cos, 8.0, use_logp=False)
    c = 0
    for s in range(1, 10):
        c_next = int(np.argmax(cos[s - 1][c]))
        assert r.choice[s] == c_next
        c = c_next


def test_walk_arithmetic_is_float32_without_fma():
    # logp + alpha*cos rounded twice in float32: pick values where a fused
    # multiply-add would round differently than the two-step form.
    logp = np.array([[0.0, 0.0], [np.float32(1.0), np.float32(1.0 + 2 ** -23)]], dtype=np.float32)
    cos = np.array([[[np.float32(1 + 2 ** -23), np.float32(1.0)], [0, 0]]], dtype=np.float32)
    alpha = np.float32(1 - 2 ** -24)
    z = step_scores(logp[1], cos[0][0], alpha, True)
    prod0 = np.float32(alpha * np.float32(1 + 2 ** -23))
    assert z[0] == np.float32(np.float32(1.0) + prod0)
    assert z.dtype == np.float32


def _unit_bf16(rng, n, d):
    v = rng.standard_normal((n, d))
    return round_bf16(v / np.linalg.norm(v, axis=1, keepdims=True))


@pytest.mark.parametrize("d", [32, 128, 256])
def test_pair_scores_invariants(d):
    rng = np.random.default_rng(d)
    B, K = 6, 8
    outv = np.stack([_unit_bf16(rng, K, d) for _ in range(B)])
    inv = np.stack([_unit_bf16(rng, K, d) for _ in range(B)])
    # bf16 rounding of each unit-vector component moves the norm by at most 2^-8
    n = np.linalg.norm(outv, axis=-1)
    assert np.all(np.abs(n - 1) <= 2 ** -8)
    c = pair_scores(outv, inv)
    assert c.shape == (B - 1, K, K) and c.dtype == np.float32
    assert np.all(np.abs(c) <= 1.01)
    # duplicated vectors give cos ~ 1; orientation: out of slot s-1 against in of slot s
    inv2 = inv.copy()
    inv2[3, 5] = outv[2, 1]
    c2 = pair_scores(outv, inv2)
    assert abs(c2[2, 1, 5] - 1.0) <= 2 ** -7
    assert np.array_equal(c2[2, 1, :5], c[2, 1, :5])


def test_pair_scores_hand_example():
    outv = np.zeros((2, 2, 4))
    inv = np.zeros((2, 2, 4))
    outv[0, 0] = [1, 0, 0, 0]
    outv[0, 1] = [0, 0.5, 0.5, 0]
    inv[1, 0] = [0.5, 0.5, 0, 0]
    inv[1, 1] = [0, 0, 1, 0]
    c = pair_scores(outv, inv)
    assert c[0].tolist() == [[0.5, 0.0], [0.25, 0.5]]
