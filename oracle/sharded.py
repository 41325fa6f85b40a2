"""Top-K and log-partition of rows whose vocabulary is split across shards.
TEST INFRASTRUCTURE ONLY.

When the logits come from a tensor-parallel LM head (the SGLang PR leaves the
tp > 1 case open), each shard g holds a contiguous range of vocabulary ids
[o_g, o_g + V_g). Each shard reduces its slice of a row to
  * its K best (value, global id) pairs in (value desc, id asc) order
    (fewer if V_g < K), and
  * a (m_g, s_g) pair with s_g = sum_{v in shard} exp(x_v - m_g), m_g its max;
and the row's answer is recovered from those alone:
  * top-K: the K best of the union of the shard lists, in the same order.
    Exact, by the argument the PR gives for its tile pre-selection: a global
    top-K element of shard g is preceded (in the global order) by fewer than K
    elements, hence by fewer than K of its own shard, so it is in that shard's
    list;
  * lse = M + log(sum_g s_g exp(m_g - M)), M = max_g m_g (the log-sum-exp of
    the shard partitions);
  * logp = fl32(fl32(x) - fl32(lse)) as for an unsplit row.
Float64 throughout, as the unsplit oracle.
"""
from __future__ import annotations

import numpy as np

from .topk_lse import _row_values


def shard_bounds(V: int, G: int):
    """Contiguous split of [0, V) into G ranges, the first V % G one longer."""
    base, extra = divmod(V, G)
    bounds, o = [], 0
    for g in range(G):
        n = base + (1 if g < extra else 0)
        bounds.append((o, o + n))
        o += n
    return bounds


def shard_partial(row: np.ndarray, lo: int, hi: int, K: int):
    """One shard's reduction of row[lo:hi]: (values f64[k], global ids int64[k], m, s), k = min(K, hi - lo)."""
    x = _row_values(row)[lo:hi].astype(np.float64)
    order = np.lexsort((np.arange(x.size), -x))[:K]
    m = float(x.max())
    s = float(np.sum(np.exp(x - m)))
    return x[order], order.astype(np.int64) + lo, m, s


def merge_partials(parts, K: int):
    """Combine shard partials into (idx int64[K], logp float32[K], lse float64)."""
    vals = np.concatenate([p[0] for p in parts])
    ids = np.concatenate([p[1] for p in parts])
    order = np.lexsort((ids, -vals))[:K]
    M = max(p[2] for p in parts)
    lse = M + np.log(sum(p[3] * np.exp(p[2] - M) for p in parts))
    idx = ids[order]
    logp = (vals[order].astype(np.float32) - np.float32(lse)).astype(np.float32)
    return idx, logp, float(lse)


def topk_lse_sharded_row(row: np.ndarray, K: int, G: int):
    parts = [shard_partial(row, lo, hi, K) for lo, hi in shard_bounds(row.shape[-1], G)]
    return merge_partials(parts, K)
