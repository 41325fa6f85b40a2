"""Seeded synthetic inputs and the workload table.

This module is shared by the oracle and the HIP path. It holds none of the
reranker's arithmetic: only shapes, seeds and the recipe that draws the draft
logits. Both sides receive the identical bytes it produces.

Workload shapes follow the pages' serving setup: block size 16 with 15 drafted
slots (LiLiCorr paper, Table 4), the Qwen3 vocabulary of 151,936 entries and
concurrency 1 and 32 (SGLang PR "[Spec] Add LiLiCorr", review thread on the
fused top-k), K = 8 (LiLiCorr paper, Table 4) and larger pools, and three output
entropy tiers (LiLiCorr paper, Section 4.1 / Table 2 throughput sweep). The
pages measure on public prompt suites; these seeded blocks stand in for their
shapes only.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WEIGHTS_SEED = 42


@dataclass(frozen=True)
class Workload:
    name: str
    num_blocks: int          # N independent draft blocks
    slots: int               # B slots per block (slot 0 plus B-1 drafted)
    vocab: int               # V
    topk: int                # K candidates per slot
    hidden: int              # encoder width H
    heads: int
    ffn: int                 # F
    d_e: int                 # in/out vector width
    dtype: str               # "f32" or "bf16" logits
    recipe: str              # "normal", "spiked" or "tempered"
    temperatures: tuple = field(default=(1.0,))
    alpha: float = 1.0
    layers: int = 2
    use_logp: bool = True
    # the paper's own head (drafter hidden states and a target state as inputs)
    target_hidden: int = 0
    drafter_hidden: int = 0

    @property
    def tokens_per_block(self) -> int:
        return self.slots * self.topk

    def logits_seed(self, tier: int = 0) -> int:
        index = WORKLOADS_ORDER.index(self.name)
        return 1000 * index + tier


WORKLOADS = {
    # Small case the oracle finishes in seconds.
    "tiny": Workload("tiny", 1, 16, 1024, 4, 64, 2, 256, 32, "f32", "normal"),
    # Concurrency 1, Qwen3-8B-like vocabulary.
    "c1_qwen3_8b": Workload("c1_qwen3_8b", 1, 16, 151936, 8, 1024, 8, 4096, 128,
                            "bf16", "spiked"),
    # Concurrency 32.
    "c32": Workload("c32", 32, 16, 151936, 8, 1024, 8, 4096, 128, "bf16", "spiked"),
    # 256 blocks, K = 16.
    "c256_k16": Workload("c256_k16", 256, 16, 151936, 16, 1024, 8, 4096, 128,
                         "bf16", "spiked"),
    # Entropy sweep: 64 blocks per temperature tier, K = 32, wider encoder.
    "entropy_k32": Workload("entropy_k32", 64, 16, 151936, 32, 2048, 16, 8192, 256,
                            "bf16", "tempered", temperatures=(0.3, 1.0, 3.0)),
    # Odd shapes for the test suite: an odd token count above 4096 (the
    # many-token node-build path with a ragged last block), 15 slots, a width
    # above 2048 and d_h = 128.
    "odd_h2560": Workload("odd_h2560", 41, 15, 4096, 7, 2560, 20, 512, 128, "bf16", "spiked"),
    # The paper's own head (LiLiCorr paper, Table 4: width 1024, 8 heads, FFN
    # 2048, d_e 1024, sigma = 8 with the sigma * cos rule; drafter and target
    # widths of a Qwen3-8B target, 4096), with a small CPU-checkable twin.
    "paper_tiny": Workload("paper_tiny", 1, 16, 1024, 4, 64, 2, 128, 32, "f32", "normal",
                           alpha=8.0, use_logp=False, target_hidden=128, drafter_hidden=128),
    "paper_qwen3_8b": Workload("paper_qwen3_8b", 1, 16, 151936, 8, 1024, 8, 2048, 1024, "bf16",
                               "spiked", alpha=8.0, use_logp=False, target_hidden=4096,
                               drafter_hidden=4096),
    "paper_c32": Workload("paper_c32", 32, 16, 151936, 8, 1024, 8, 2048, 1024, "bf16", "spiked",
                          alpha=8.0, use_logp=False, target_hidden=4096, drafter_hidden=4096),
}
WORKLOADS_ORDER = ["tiny", "c1_qwen3_8b", "c32", "c256_k16", "entropy_k32", "odd_h2560",
                   "paper_tiny", "paper_qwen3_8b", "paper_c32"]


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Input conversion only: the draft logits arrive as bfloat16, the storage
    format the pages serve them in. Finite inputs only.
    """
    bits = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return rounded.astype(np.uint16)


def make_logits(w: Workload, tier: int = 0, num_blocks: int | None = None) -> np.ndarray:
    """Draw the logits of a workload as a host array of shape [N, B, V].

    Returns float32 values for "f32" workloads and uint16 bfloat16 bit
    patterns for "bf16" workloads.

    Recipe (numpy default_rng seeded with logits_seed(tier)):
      1. standard_normal(float32) of shape [N, B, V];
      2. "spiked": per row, 3 distinct positions drawn with integers(0, V)
         (duplicates redrawn), then amplitudes uniform(8, 12) in float32
         added to the normal value at those positions;
      3. "tempered": the normal value divided by the tier's temperature;
      4. bf16 rounding (round to nearest even) for "bf16" workloads.
    ``num_blocks`` draws only the first blocks of the same stream order
    (the normal draw is generated block by block, so a prefix is identical).
    """
    n = w.num_blocks if num_blocks is None else num_blocks
    rng = np.random.default_rng(w.logits_seed(tier))
    rows_per_block = w.slots
    out_dtype = np.float32 if w.dtype == "f32" else np.uint16
    out = np.empty((n, w.slots, w.vocab), dtype=out_dtype)
    # Normal values block by block so that a prefix of blocks is reproducible.
    normals = []
    for b in range(w.num_blocks):
        blk = rng.standard_normal((rows_per_block, w.vocab), dtype=np.float32)
        if b < n:
            normals.append(blk)
    rows = w.num_blocks * rows_per_block
    if w.recipe == "spiked":
        pos = rng.integers(0, w.vocab, size=(rows, 3))
        while True:
            dup = (pos[:, 0] == pos[:, 1]) | (pos[:, 0] == pos[:, 2]) | (pos[:, 1] == pos[:, 2])
            if not dup.any():
                break
            pos[dup] = rng.integers(0, w.vocab, size=(int(dup.sum()), 3))
        amp = rng.uniform(8.0, 12.0, size=(rows, 3)).astype(np.float32)
    for b in range(n):
        blk = normals[b]
        if w.recipe == "spiked":
            r0 = b * rows_per_block
            for j in range(3):
                ridx = np.arange(rows_per_block)
                blk[ridx, pos[r0:r0 + rows_per_block, j]] += amp[r0:r0 + rows_per_block, j]
        elif w.recipe == "tempered":
            blk = (blk / np.float32(w.temperatures[tier])).astype(np.float32)
        if w.dtype == "f32":
            out[b] = blk
        else:
            out[b] = f32_to_bf16_bits_rne(blk)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_random_logits(rows: int, vocab: int, dtype: str, seed: int,
                       scale: float = 1.0) -> np.ndarray:
    """Plain N(0, scale^2) logits of shape [rows, vocab] for shape sweeps."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, vocab), dtype=np.float32) * np.float32(scale)).astype(np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits_rne(x)


def make_uniforms(num_blocks: int, slots: int, seed: int) -> np.ndarray:
    """The sampled commit's random draws, passed to both sides as input:
    float32 [N, B] uniform in [0, 1) from default_rng(seed).random."""
    return np.random.default_rng(seed).random((num_blocks, slots), dtype=np.float32)


def make_temperatures(num_blocks: int, seed: int, greedy_every: int = 4) -> np.ndarray:
    """Per-block sampling temperatures, float32 [N]: every greedy_every-th block
    (block 0 first) is a greedy row (T = 0); the others draw T uniformly from
    [0.5, 1.5) (the pages serve requests at their own temperature, T = 1
    in their measurement)."""
    rng = np.random.default_rng(seed)
    t = rng.uniform(0.5, 1.5, size=num_blocks).astype(np.float32)
    if greedy_every > 0:
        t[::greedy_every] = 0.0
    return t


def make_head_inputs(w: Workload, tier: int = 0, num_blocks: int | None = None):
    """Inputs of the paper's own head, as bfloat16 bit patterns:
    hidden [N, B, H_d] (the drafter's hidden state per slot) and target
    [N, H_t] (the target state behind the last committed token), both
    standard normal from default_rng(logits_seed(tier) + 500), hidden first;
    a prefix of blocks is the same at any N."""
    n = w.num_blocks if num_blocks is None else num_blocks
    rng = np.random.default_rng(w.logits_seed(tier) + 500)
    hidden = rng.standard_normal((w.num_blocks, w.slots, w.drafter_hidden), dtype=np.float32)
    target = rng.standard_normal((w.num_blocks, w.target_hidden), dtype=np.float32)
    return f32_to_bf16_bits_rne(hidden[:n]), f32_to_bf16_bits_rne(target[:n])
