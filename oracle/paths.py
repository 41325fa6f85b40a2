"""Two further commit rules over the candidate lattice.  TEST INFRASTRUCTURE ONLY.

Both use the same per-step score as the greedy walk (oracle.walk.step_scores):
  z_s(i, j) = fl32(logp[s][j] + fl32(alpha * cos_s[i][j]))   (use_logp = 1)
  z_s(i, j) = fl32(alpha * cos_s[i][j])                       (use_logp = 0)
and the same anchor: c_0 = 0 (slot 0 commits its top candidate).

best_path -- LiLiCorr paper, Appendix E ("Greedy Selection Versus the
Highest-Scoring Path", Eq. (12)): a path c = (c_1, ..., c_{B-1}) scores
g(c) = sum_s z_s(c_{s-1}, c_s); the maximiser is found by dynamic programming
in O(B K^2): sweep left to right keeping, per candidate, the score of the best
path ending there and its predecessor, then trace the predecessors back from
the best final candidate.
  Readings taken here. The sum is accumulated left to right in float32,
  G_s(j) = fl32(G_{s-1}(i) + z_s(i, j)); float32 addition is monotone, so the
  recursion still yields the maximum float32 total over all paths. Every
  maximum breaks ties toward the lower index (the greedy rule's tie rule),
  both when choosing a predecessor and when choosing the final candidate, so
  among equally scoring paths the trace-back returns the one that is smallest
  when compared from the last slot backward.

sample_path -- SGLang PR, "Sampling the committed path (opt-in)" and
"lilicorr_sample_path": the greedy walk with each slot drawn from
softmax(z / T) over that slot's candidates at the block's temperature T,
publishing the distribution drawn from (the proposal). A block whose T <= 0 is
a greedy row: it takes the argmax on the same float32 scores (the greedy walk's
path, bit for bit) and reports a one-hot proposal.
  Readings taken here. Slot 0 is the anchor: c_0 = 0 with a one-hot proposal.
  The random draw is an input: one uniform u_s in [0, 1) per slot, and the
  draw is the inverse CDF, c_s = #{j : C_j <= u_s} with C_j = sum_{i <= j} q_i
  (the smallest j whose cumulative probability exceeds u_s), clamped to K - 1.
  q = softmax(z / T) is evaluated in float64 from the float32 scores.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .walk import greedy_walk, step_scores


@dataclass
class PathResult:
    choice: np.ndarray      # int64 [B]
    tokens: np.ndarray      # int64 [B]
    score: np.ndarray       # float32 [B]: z_s(c_{s-1}, c_s); slot 0: its top logp
    total: np.float32       # float32 left-to-right sum of score[1:]


def path_total(logp, cos, choice, alpha: float = 1.0, use_logp: bool = True) -> np.float32:
    """g(c) of Eq. (12), summed left to right in float32."""
    g = np.float32(0.0)
    for s in range(1, logp.shape[0]):
        z = step_scores(logp[s], cos[s - 1][choice[s - 1]], alpha, use_logp)[choice[s]]
        g = np.float32(g + z)
    return g


def best_path(idx_block, logp_block, cos_block, alpha: float = 1.0,
              use_logp: bool = True) -> PathResult:
    B, K = logp_block.shape
    choice = np.zeros(B, dtype=np.int64)
    score = np.zeros(B, dtype=np.float32)
    score[0] = logp_block[0][0]
    if B == 1:
        return PathResult(choice, np.asarray(idx_block)[0:1, 0].astype(np.int64), score, np.float32(0))
    # forward sweep: G[j] = best float32 total of a path ending at candidate j
    # of the current slot; pred[s][j] = its predecessor at slot s - 1
    G = step_scores(logp_block[1], cos_block[0][0], alpha, use_logp).astype(np.float32)
    pred = np.zeros((B, K), dtype=np.int64)
    for s in range(2, B):
        newG = np.full(K, -np.inf, dtype=np.float32)
        for j in range(K):
            for i in range(K):          # ascending i, strict '>' keeps the lowest i on a tie
                z = step_scores(logp_block[s], cos_block[s - 1][i], alpha, use_logp)[j]
                cand = np.float32(G[i] + z)
                if cand > newG[j]:
                    newG[j] = cand
                    pred[s][j] = i
        G = newG
    # trace back from the best final candidate (lowest index on a tie)
    choice[B - 1] = int(np.argmax(G))
    for s in range(B - 1, 1, -1):
        choice[s - 1] = pred[s][choice[s]]
    choice[0] = 0
    for s in range(1, B):
        score[s] = step_scores(logp_block[s], cos_block[s - 1][choice[s - 1]], alpha, use_logp)[choice[s]]
    tokens = np.asarray(idx_block)[np.arange(B), choice].astype(np.int64)
    return PathResult(choice, tokens, score, path_total(logp_block, cos_block, choice, alpha, use_logp))


@dataclass
class SampleResult:
    choice: np.ndarray      # int64 [B]
    tokens: np.ndarray      # int64 [B]
    proposal: np.ndarray    # float64 [B, K]: distribution slot s was drawn from
    cdf: np.ndarray         # float64 [B, K]: its cumulative sums (for boundary checks)


def softmax_t(z: np.ndarray, temperature: float) -> np.ndarray:
    """softmax(z / T) in float64 from float32 scores."""
    t = (np.asarray(z, dtype=np.float64) - float(np.max(z))) / float(temperature)
    e = np.exp(t)
    return e / e.sum()


def sample_path(idx_block, logp_block, cos_block, temperature: float, uniforms,
                alpha: float = 1.0, use_logp: bool = True) -> SampleResult:
    B, K = logp_block.shape
    choice = np.zeros(B, dtype=np.int64)
    proposal = np.zeros((B, K), dtype=np.float64)
    cdf = np.ones((B, K), dtype=np.float64)
    proposal[0, 0] = 1.0
    if temperature <= 0:            # greedy row: the greedy walk's own path
        r = greedy_walk(idx_block, logp_block, cos_block, alpha, use_logp)
        proposal[np.arange(B), r.choice] = 1.0
        cdf = np.cumsum(proposal, axis=1)
        return SampleResult(r.choice, r.tokens, proposal, cdf)
    for s in range(1, B):
        z = step_scores(logp_block[s], cos_block[s - 1][choice[s - 1]], alpha, use_logp)
        q = softmax_t(z, temperature)
        c = np.cumsum(q)
        proposal[s] = q
        cdf[s] = c
        choice[s] = min(int(np.sum(c <= float(uniforms[s]))), K - 1)
    tokens = np.asarray(idx_block)[np.arange(B), choice].astype(np.int64)
    return SampleResult(choice, tokens, proposal, cdf)
