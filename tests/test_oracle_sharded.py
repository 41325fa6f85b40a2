"""Pins for the oracle's vocabulary-sharded top-K and log-partition (CPU only).

The sharded reduction must give the unsplit definition back for any number of
shards: identical top-K ids (an exact selection), the same log-partition to
float64 rounding, hence the same float32 log-probabilities. Rows with many
exact ties straddling shard boundaries, uneven shards, shards shorter than K
and single-element shards are included.
"""
import numpy as np
import pytest

from oracle.sharded import shard_bounds, topk_lse_sharded_row, shard_partial, merge_partials
from oracle.topk_lse import topk_lse_row
from synth import f32_to_bf16_bits_rne


@pytest.mark.parametrize("V,G", [(1000, 1), (1000, 2), (1000, 7), (151936, 8), (10, 10), (67, 64)])
def test_bounds_cover_the_vocabulary(V, G):
    b = shard_bounds(V, G)
    assert b[0][0] == 0 and b[-1][1] == V
    assert all(a[1] == c[0] for a, c in zip(b, b[1:]))
    assert max(h - l for l, h in b) - min(h - l for l, h in b) <= 1


@pytest.mark.parametrize("V,K,G", [(1024, 4, 1), (1024, 8, 2), (1024, 32, 8), (4099, 16, 7), (40, 8, 8),
                                   (64, 64, 64), (300, 17, 5)])
@pytest.mark.parametrize("kind", ["f32", "bf16", "coarse"])
def test_sharded_equals_unsplit(V, K, G, kind):
    rng = np.random.default_rng(V + K + G)
    for _ in range(5):
        if kind == "coarse":        # few distinct values: ties across every shard boundary
            row = rng.integers(-3, 3, size=V).astype(np.float32)
        else:
            row = rng.standard_normal(V).astype(np.float32)
            if kind == "bf16":
                row = f32_to_bf16_bits_rne(row)
        i0, l0, s0 = topk_lse_row(row, K)
        i1, l1, s1 = topk_lse_sharded_row(row, K, G)
        assert np.array_equal(i0, i1)
        assert abs(s0 - s1) <= 1e-12 * max(1.0, abs(s0))
        assert np.array_equal(l0, l1)


def test_constant_row_closed_form():
    # every value equal: ids 0..K-1 and lse = c + log V whatever the split
    V, K = 1000, 8
    row = np.full(V, 2.5, dtype=np.float32)
    for G in (1, 3, 8, 1000):
        idx, logp, lse = topk_lse_sharded_row(row, K, G)
        assert idx.tolist() == list(range(K))
        assert abs(lse - (2.5 + np.log(V))) < 1e-12


def test_merge_needs_only_the_partials():
    # a shard whose slice is all below the others contributes only to the partition
    row = np.concatenate([np.full(50, -20.0), np.linspace(0, 1, 50)]).astype(np.float32)
    parts = [shard_partial(row, 0, 50, 4), shard_partial(row, 50, 100, 4)]
    idx, logp, lse = merge_partials(parts, 4)
    assert idx.tolist() == [99, 98, 97, 96]
    assert abs(lse - np.log(np.sum(np.exp(row.astype(np.float64))))) < 1e-12
