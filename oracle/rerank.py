"""The whole reranking path for one draft block, step by step.

LiLiCorr paper, Section 3.5: one network pass produces every in and out
vector, the pair scores are batched products, and a greedy walk commits the
block left to right. Blocks are independent.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .topk_lse import topk_lse
from .encoder import encode_block
from .paper_head import encode_block_paper
from .scores import pair_scores
from .walk import greedy_walk, WalkResult
from .paths import best_path, sample_path, PathResult, SampleResult
from .weights import OracleWeights


@dataclass
class BlockResult:
    idx: np.ndarray        # int64 [B, K]
    logp: np.ndarray       # float32 [B, K]
    lse: np.ndarray        # float64 [B]
    outv: np.ndarray       # float64 [B, K, d_e] (bf16 values)
    inv: np.ndarray        # float64 [B, K, d_e]
    cos: np.ndarray        # float32 [B-1, K, K]
    walk: WalkResult                     # the greedy walk (computed for every rule)
    exact: PathResult | None = None      # rule "exact"
    sample: SampleResult | None = None   # rule "sample"

    @property
    def tokens(self) -> np.ndarray:
        if self.exact is not None:
            return self.exact.tokens
        if self.sample is not None:
            return self.sample.tokens
        return self.walk.tokens


def rerank_block(logits_block: np.ndarray, K: int, w: OracleWeights, alpha: float = 1.0,
                 use_logp: bool = True, trace: dict | None = None, rule: str = "greedy",
                 temperature: float = 0.0, uniforms=None, hidden=None, target=None) -> BlockResult:
    """logits_block: [B, V] float32 values or uint16 bfloat16 bit patterns.

    rule: "greedy" (Eq. (8)), "exact" (best path, Appendix E) or "sample"
    (draws from softmax(z / temperature) with the given per-slot uniforms).
    With the paper's head (w.dims.paper_head) hidden [B, H_d] and target [H_t]
    are the block's drafter hidden states and target state (bf16 values)."""
    idx, logp, lse = topk_lse(logits_block, K)
    if w.dims.paper_head:
        outv, inv = encode_block_paper(idx, logp, hidden, target, w, trace)
    else:
        outv, inv = encode_block(idx, logp, w, trace)
    cos = pair_scores(outv, inv)
    walk = greedy_walk(idx, logp, cos, alpha, use_logp)
    res = BlockResult(idx, logp, lse, outv, inv, cos, walk)
    if rule == "exact":
        res.exact = best_path(idx, logp, cos, alpha, use_logp)
    elif rule == "sample":
        res.sample = sample_path(idx, logp, cos, temperature, uniforms, alpha, use_logp)
    elif rule != "greedy":
        raise ValueError(f"unknown rule {rule!r}")
    return res
