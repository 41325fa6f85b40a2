"""Pair scores between adjacent slots.

LiLiCorr paper, Eq. (1) and Section 3.5: adjacent slots are coupled by the
cosine similarity of the earlier candidate's out vector with the later
candidate's in vector; each slot pair is one matrix product, batched over the
block. The vectors are unit norm, so the cosine is their dot product:

  cos_s[a][b] = sum_d out[s-1, a, d] * in[s, b, d]     s = 1 .. B-1

Products of bfloat16 values are exact; the sum is float64 and the result is
reported as float32.
"""
import numpy as np


def pair_scores(outv: np.ndarray, inv: np.ndarray) -> np.ndarray:
    """outv, inv: [B, K, d_e] -> cos float32 [B-1, K, K]."""
    B = outv.shape[0]
    c = np.empty((B - 1, outv.shape[1], inv.shape[1]), dtype=np.float64)
    for s in range(1, B):
        c[s - 1] = outv[s - 1] @ inv[s].T
    return c.astype(np.float32)
