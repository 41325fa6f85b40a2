"""Per-slot top-K candidates and the full-vocabulary log-partition.

LiLiCorr paper, Section 3.2: each slot keeps the drafter's K most probable
tokens. Appendix A ("Architecture", "Serving"): candidates carry their
log-probability under the full vocabulary, and candidate extraction and the
vocabulary-wide normalisation are one fused step. SGLang PR, "Why the custom
kernels": the kernel returns the exact top-k and the log-partition of each row.

Ordering: value descending, then vocabulary index ascending, on the raw input
values (selecting on logits or on log-probs gives the same order, since the
subtraction of the row's log-partition is monotone). -0 and +0 compare equal.

Definition (oracle, float64):
  lse  = m + log(sum_v exp(x_v - m)),  m = max_v x_v
  logp = fl32(fl32(x) - fl32(lse))     the final subtraction in float32
"""
from __future__ import annotations

import numpy as np


def _row_values(row: np.ndarray) -> np.ndarray:
    if row.dtype == np.uint16:      # bfloat16 bit patterns: widen exactly
        return (row.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.asarray(row, dtype=np.float32)


def topk_lse_row(row: np.ndarray, K: int):
    """Return (idx int64[K], logp float32[K], lse float64) for one row."""
    x = _row_values(row)
    V = x.shape[0]
    if not (1 <= K <= V):
        raise ValueError("need 1 <= K <= V")
    if not np.all(np.isfinite(x)):
        raise ValueError("logits must be finite")
    kth = np.partition(x, V - K)[V - K]            # K-th largest value
    above = np.nonzero(x > kth)[0]
    equal = np.nonzero(x == kth)[0]                 # ascending index
    chosen = np.concatenate([above, equal[: K - above.size]])
    # Sort the chosen candidates by (value desc, index asc).
    order = np.lexsort((chosen, -x[chosen].astype(np.float64)))
    idx = chosen[order].astype(np.int64)
    x64 = x.astype(np.float64)
    m = x64.max()
    lse = m + np.log(np.sum(np.exp(x64 - m)))
    logp = (x[idx].astype(np.float32) - np.float32(lse)).astype(np.float32)
    return idx, logp, float(lse)


def topk_lse(rows: np.ndarray, K: int):
    """Row-wise top-K over a [..., V] array; returns idx, logp, lse with leading dims kept."""
    lead = rows.shape[:-1]
    flat = rows.reshape(-1, rows.shape[-1])
    idx = np.empty((flat.shape[0], K), dtype=np.int64)
    logp = np.empty((flat.shape[0], K), dtype=np.float32)
    lse = np.empty((flat.shape[0],), dtype=np.float64)
    for r in range(flat.shape[0]):
        idx[r], logp[r], lse[r] = topk_lse_row(flat[r], K)
    return idx.reshape(lead + (K,)), logp.reshape(lead + (K,)), lse.reshape(lead)
