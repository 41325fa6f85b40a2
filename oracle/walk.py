"""Greedy left-to-right commit over the candidate lattice.

LiLiCorr paper, Eq. (8) and Section 3.5: slot s commits the argmax of its
node score conditioned on the candidate committed at slot s-1; only this walk
is sequential. SGLang PR, "Why the custom kernels": argmax ties go to the
lower candidate index.

Rule used here (the paper's anchor slot has no candidates; in this path slot 0
carries logits too and commits its top candidate):

  c_0 = 0
  z_s[j] = fl32(logp[s][j] + fl32(alpha * cos_s[c_{s-1}][j]))   (use_logp = 1)
  z_s[j] = fl32(alpha * cos_s[c_{s-1}][j])                       (use_logp = 0,
            the paper's sigma * cos rule of Eq. (1) with alpha = sigma)
  c_s = lowest j with z_s[j] = max_j z_s[j]
  token[s] = idx[s][c_s]

All arithmetic is single-precision IEEE with no fused multiply-add.
Also reported per slot: the committed score z_s[c_s] and the gap to the best
other candidate (0 for K = 1, and for slot 0).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class WalkResult:
    choice: np.ndarray      # int64 [B]
    tokens: np.ndarray      # int64 [B]
    score: np.ndarray       # float32 [B]
    gap: np.ndarray         # float32 [B]
    z: np.ndarray           # float32 [B, K] (row 0: slot 0 logp)


def step_scores(logp_row: np.ndarray, cos_row: np.ndarray, alpha: float, use_logp: bool) -> np.ndarray:
    a = np.float32(alpha)
    prod = (a * cos_row.astype(np.float32)).astype(np.float32)
    if use_logp:
        return (logp_row.astype(np.float32) + prod).astype(np.float32)
    return prod


def greedy_walk(idx_block, logp_block, cos_block, alpha: float = 1.0, use_logp: bool = True) -> WalkResult:
    B, K = logp_block.shape
    choice = np.zeros(B, dtype=np.int64)
    score = np.zeros(B, dtype=np.float32)
    gap = np.zeros(B, dtype=np.float32)
    z = np.zeros((B, K), dtype=np.float32)
    z[0] = logp_block[0]
    score[0] = logp_block[0][0]
    for s in range(1, B):
        zs = step_scores(logp_block[s], cos_block[s - 1][choice[s - 1]], alpha, use_logp)
        z[s] = zs
        best = int(np.argmax(zs))                 # first occurrence of the max
        choice[s] = best
        score[s] = zs[best]
        if K > 1:
            others = np.delete(zs, best)
            gap[s] = np.float32(zs[best] - others.max())
    tokens = np.asarray(idx_block)[np.arange(B), choice].astype(np.int64)
    return WalkResult(choice, tokens, score, gap, z)
