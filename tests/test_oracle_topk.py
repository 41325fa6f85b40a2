"""Pins for the oracle's top-K and log-partition (CPU only).

Top-K order is (value descending, index ascending) on the raw logits; the
log-partition is log sum_v exp(x_v). Both have plain definitions, so the pins
are a different selection algorithm (full lexicographic sort), closed forms
and an independent library routine.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

from oracle.topk_lse import topk_lse_row, topk_lse
from synth import f32_to_bf16_bits_rne, bf16_bits_to_f32


def brute_topk(x, K):
    return np.lexsort((np.arange(x.size), -x.astype(np.float64)))[:K]


@pytest.mark.parametrize("V,K", [(1024, 4), (1024, 32), (37, 37), (8, 1), (7, 3), (2000, 64)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topk_matches_full_sort_f32(V, K, seed):
    x = np.random.default_rng(seed).standard_normal(V).astype(np.float32)
    idx, logp, lse = topk_lse_row(x, K)
    assert np.array_equal(idx, brute_topk(x, K))


@pytest.mark.parametrize("scale", [0.05, 1.0, 4.0])
def test_topk_bf16_ties_match_full_sort(scale):
    # bfloat16 has 8 significant bits, so rows of a few thousand draws hold many
    # exact ties, including at the K-th / (K+1)-th boundary.
    rng = np.random.default_rng(7)
    boundary_ties = 0
    for r in range(60):
        bits = f32_to_bf16_bits_rne(rng.standard_normal(3000).astype(np.float32) * np.float32(scale))
        x = bf16_bits_to_f32(bits)
        for K in (8, 16, 32):
            idx, _, _ = topk_lse_row(bits, K)
            assert np.array_equal(idx, brute_topk(x, K))
            srt = np.sort(x)[::-1]
            boundary_ties += int(srt[K - 1] == srt[K])
    assert boundary_ties > 0


def test_topk_python_sorted_small():
    vals = [0.5, -1.0, 0.5, 2.0, 0.5, -0.0, 0.0, 2.0]
    x = np.array(vals, dtype=np.float32)
    expect = [i for _, i in sorted(((-v, i) for i, v in enumerate(vals)))][:5]
    idx, _, _ = topk_lse_row(x, 5)
    assert idx.tolist() == expect == [3, 7, 0, 2, 4]


def test_constant_row_ids_and_lse():
    V, K, c = 5000, 16, 1.75
    x = np.full(V, c, dtype=np.float32)
    idx, logp, lse = topk_lse_row(x, K)
    assert idx.tolist() == list(range(K))
    assert lse == pytest.approx(c + math.log(V), rel=0, abs=1e-12)
    assert np.all(logp == np.float32(np.float32(c) - np.float32(c + math.log(V))))


def test_signed_zero_ties_by_index():
    x = np.array([-0.0, 0.0, -0.0, -1.0, 0.0], dtype=np.float32)
    idx, _, _ = topk_lse_row(x, 4)
    assert idx.tolist() == [0, 1, 2, 4]


def test_k_equals_v_is_full_sort():
    x = np.array([3, 1, 2, 3, 0], dtype=np.float32)
    idx, _, _ = topk_lse_row(x, 5)
    assert idx.tolist() == [0, 3, 2, 1, 4]


def test_k1_is_first_argmax():
    rng = np.random.default_rng(3)
    for _ in range(50):
        bits = f32_to_bf16_bits_rne(rng.integers(-3, 3, 200).astype(np.float32))
        idx, _, _ = topk_lse_row(bits, 1)
        assert idx[0] == int(np.argmax(bf16_bits_to_f32(bits)))


def test_lse_single_spike():
    x = np.zeros(100_000, dtype=np.float32)
    x[12345] = 100.0
    _, _, lse = topk_lse_row(x, 1)
    assert lse == pytest.approx(100.0 + math.log1p((x.size - 1) * math.exp(-100.0)), abs=1e-12)


def test_lse_against_scipy_and_logp_rounding():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((6, 151936)) * 2.5).astype(np.float32)
    idx, logp, lse = topk_lse(x, 8)
    ref = logsumexp(x.astype(np.float64), axis=1)
    assert np.allclose(lse, ref, rtol=0, atol=1e-10)
    for r in range(6):
        expect = (x[r, idx[r]] - np.float32(ref[r])).astype(np.float32)
        assert np.array_equal(logp[r], expect)
    # logp are log-probabilities: non-positive and sum of their exp below 1
    assert np.all(logp <= 0) and np.all(np.exp(logp.astype(np.float64)).sum(1) < 1)


def test_golden_lse_fixture():
    # tests/golden/lse_closed_form.txt: constant rows have lse = c + log V.
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "lse_closed_form.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    for c, V, expect in rows:
        x = np.full(int(V), np.float32(float(c)), dtype=np.float32)
        _, _, lse = topk_lse_row(x, 1)
        assert lse == pytest.approx(float(expect), abs=1e-9)
