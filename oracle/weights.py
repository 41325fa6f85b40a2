"""Synthetic encoder weights, generated from (dims, vocabulary, seed) alone.

The pages publish no checkpoint (SGLang PR "[Spec] Add LiLiCorr", Checkpoints
note), so the head's weights are seeded random. The generator is counter
based, so any single element can be produced on its own:

  k_t = splitmix64(seed XOR (t << 40))       one key per tensor id t
  r   = splitmix64(k_t + e)  (mod 2^64)      e = row-major element index
  u   = (r >> 40) * 2^-24                    uniform in [0, 1), 24 bits
  w   = fl32((2u - 1) * scale_t)             scale_t = fl32(1 / sqrt(fan_in))
  gamma tensors: fl32(1 + 0.25 * (2u - 1))

splitmix64(x) is the first output of a SplitMix64 generator whose state is x
(Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
OOPSLA 2014): add the golden-ratio increment, then the variant-13 mixer.
Matrices and tables are stored as bfloat16 (round to nearest even); vectors
(biases, norm gains, attention-bias tables) as float32. Every step is exact
or singly rounded, so any faithful implementation produces identical bits.

Parameter layout (LiLiCorr paper, Appendix A "Architecture"; attention in the
nn.MultiheadAttention layout named in the SGLang PR, design note 3): a fused
in-projection [3H, H] with q, k, v row blocks, each split into heads as
contiguous groups of H/heads rows.
"""
from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np

from .bf16 import round_bf16

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(x: np.ndarray) -> np.ndarray:
    """First SplitMix64 output for state x (uint64 array, wrapping arithmetic)."""
    with np.errstate(over="ignore"):
        z = np.asarray(x, dtype=np.uint64) + _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


@dataclass(frozen=True)
class Dims:
    hidden: int
    heads: int
    ffn: int
    d_e: int
    layers: int = 2
    # widths of the inputs of the paper's own head (0: the lattice head without
    # a drafter or a target, whose node embeds the token with E)
    target_hidden: int = 0      # H_t: target embedding and target-state width
    drafter_hidden: int = 0     # H_d: drafter hidden-state width

    @property
    def paper_head(self) -> bool:
        return self.target_hidden > 0


# Slot and rank tables are sized for the largest supported block (64 slots,
# 64 candidates), so the signed slot distance spans [-63, 63].
TABLE_ROWS = 64
DIST_SPAN = 127


def _scale(fan_in: int) -> float:
    return float(np.float32(1.0 / math.sqrt(float(fan_in))))


def weight_table(d: Dims, vocab: int):
    """List of (tensor id, name, shape, scale, kind) with kind in bf16/f32/gamma."""
    H, F, h, de = d.hidden, d.ffn, d.heads, d.d_e
    t = [] if d.paper_head else [(0, "E", (vocab, H), 1.0, "bf16")]
    t += [
        (1, "S", (TABLE_ROWS, H), 1.0, "bf16"),
        (2, "R", (TABLE_ROWS, H), 1.0, "bf16"),
        (3, "conf_w1", (H, 5), _scale(5), "bf16"),
        (4, "conf_b1", (H,), _scale(5), "f32"),
        (5, "conf_w2", (H, H), _scale(H), "bf16"),
        (6, "conf_b2", (H,), _scale(H), "f32"),
    ]
    for l in range(d.layers):
        b = 16 + 16 * l
        t += [
            (b + 0, f"l{l}.gamma1", (H,), 0.0, "gamma"),
            (b + 1, f"l{l}.wqkv", (3 * H, H), _scale(H), "bf16"),
            (b + 2, f"l{l}.bqkv", (3 * H,), _scale(H), "f32"),
            (b + 3, f"l{l}.wo", (H, H), _scale(H), "bf16"),
            (b + 4, f"l{l}.bo", (H,), _scale(H), "f32"),
            (b + 5, f"l{l}.gamma2", (H,), 0.0, "gamma"),
            (b + 6, f"l{l}.w1", (F, H), _scale(H), "bf16"),
            (b + 7, f"l{l}.b1", (F,), _scale(H), "f32"),
            (b + 8, f"l{l}.w2", (H, F), _scale(F), "bf16"),
            (b + 9, f"l{l}.b2", (H,), _scale(F), "f32"),
            (b + 10, f"l{l}.dist", (h, DIST_SPAN), 0.5, "f32"),
            (b + 11, f"l{l}.same", (h,), 0.5, "f32"),
        ]
    t += [
        (48, "gamma_f", (H,), 0.0, "gamma"),
        (49, "w_out", (de, H), _scale(H), "bf16"),
        (50, "b_out", (de,), _scale(H), "f32"),
        (51, "w_in", (de, H), _scale(H), "bf16"),
        (52, "b_in", (de,), _scale(H), "f32"),
    ]
    if d.paper_head:
        # LiLiCorr paper, Appendix A "Architecture": the target's frozen input
        # embedding projected down, the drafter hidden state projected down,
        # the target state normalised and projected, the concat fusion layer
        # and the anchor's out head.
        Ht, Hd = d.target_hidden, d.drafter_hidden
        t += [
            (56, "E_t", (vocab, Ht), 1.0, "bf16"),
            (57, "w_emb", (H, Ht), _scale(Ht), "bf16"),
            (58, "b_emb", (H,), _scale(Ht), "f32"),
            (59, "w_hid", (H, Hd), _scale(Hd), "bf16"),
            (60, "b_hid", (H,), _scale(Hd), "f32"),
            (61, "gamma_t", (Ht,), 0.0, "gamma"),
            (62, "w_tgt", (H, Ht), _scale(Ht), "bf16"),
            (63, "b_tgt", (H,), _scale(Ht), "f32"),
            (64, "w_fuse", (H, 3 * H), _scale(3 * H), "bf16"),
            (65, "b_fuse", (H,), _scale(3 * H), "f32"),
            (66, "w_anchor", (de, H), _scale(H), "bf16"),
            (67, "b_anchor", (de,), _scale(H), "f32"),
        ]
    return t


def _generate_chunk(key, scale: float, kind: str, elems: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        r = splitmix64(np.asarray(elems, dtype=np.uint64) + key)
    u = (r >> np.uint64(40)).astype(np.float64) * (2.0 ** -24)
    centred = 2.0 * u - 1.0                      # exact
    if kind == "gamma":
        return (1.0 + 0.25 * centred).astype(np.float32).astype(np.float64)
    w32 = (centred * scale).astype(np.float32)   # product exact in float64, one rounding
    if kind == "bf16":
        return round_bf16(w32.astype(np.float64))
    return w32.astype(np.float64)


def tensor_key(t: int, seed: int) -> np.uint64:
    return splitmix64(np.array([np.uint64(seed) ^ (np.uint64(t) << np.uint64(40))], dtype=np.uint64))[0]


def generate(t: int, scale: float, kind: str, seed: int, elems: np.ndarray) -> np.ndarray:
    """Values of tensor t at the given row-major element indices, as float64."""
    key = tensor_key(t, seed)
    elems = np.asarray(elems, dtype=np.uint64).reshape(-1)
    out = np.empty(elems.shape, dtype=np.float64)
    step = 1 << 16          # small temporaries stay in the allocator's heap
    for a in range(0, elems.size, step):
        out[a:a + step] = _generate_chunk(key, scale, kind, elems[a:a + step])
    return out


def generate_all(t: int, scale: float, kind: str, seed: int, n: int) -> np.ndarray:
    """All n elements of tensor t in row-major order, as float64."""
    key = tensor_key(t, seed)
    out = np.empty((n,), dtype=np.float64)
    step = 1 << 16
    for a in range(0, n, step):
        b = min(n, a + step)
        out[a:b] = _generate_chunk(key, scale, kind, np.arange(a, b, dtype=np.uint64))
    return out


class OracleWeights:
    """Lazily generated weights of one encoder; E is produced row by row."""

    def __init__(self, dims: Dims, vocab: int, seed: int = 42, overrides=None):
        self.dims = dims
        self.vocab = vocab
        self.seed = seed
        self._spec = {name: (t, shape, scale, kind) for t, name, shape, scale, kind in weight_table(dims, vocab)}
        self._cache = {}
        self._overrides = dict(overrides or {})

    def __getitem__(self, name: str) -> np.ndarray:
        if name in self._overrides:
            return np.asarray(self._overrides[name], dtype=np.float64)
        if name in ("E", "E_t"):
            raise KeyError("use embedding_rows() for the token embedding tables")
        if name not in self._cache:
            t, shape, scale, kind = self._spec[name]
            n = int(np.prod(shape))
            self._cache[name] = generate_all(t, scale, kind, self.seed, n).reshape(shape)
        return self._cache[name]

    def embedding_rows(self, tokens: np.ndarray, table: str = "E") -> np.ndarray:
        if table in self._overrides:
            return np.asarray(self._overrides[table], dtype=np.float64)[np.asarray(tokens)]
        t, shape, scale, kind = self._spec[table]
        H = shape[1]
        tok = np.asarray(tokens, dtype=np.uint64).reshape(-1, 1)
        elems = tok * np.uint64(H) + np.arange(H, dtype=np.uint64).reshape(1, -1)
        return generate(t, scale, kind, self.seed, elems.reshape(-1)).reshape(len(tokens), H)

    def tensor_elements(self, name: str, elems: np.ndarray) -> np.ndarray:
        """Generated values of selected row-major elements (no overrides)."""
        t, shape, scale, kind = self._spec[name]
        return generate(t, scale, kind, self.seed, np.asarray(elems, dtype=np.uint64))
