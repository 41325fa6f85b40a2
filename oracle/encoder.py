"""Candidate encoder: node build, two lattice-transformer layers, in/out heads.

Node (LiLiCorr paper, Section 3.2 and Appendix A "Architecture"): each
candidate's vector is a sum of equal-width terms. Without a drafter in this
path the hidden-state term is left out, leaving

  x0 = E[token] + S[slot] + R[rank] + (W2c . bf16(SiLU(W1c f + b1c)) + b2c)

where f holds the five confidence scalars of Appendix A: the log-probability,
the probability, the gap to the slot's top log-probability, the rank scaled to
[0, 1] (0 when K = 1) and the top-choice indicator. W1c f uses the
bfloat16-valued W1c and the unrounded features.

Layers (Appendix A: two bidirectional layers over the whole lattice, RMSNorm,
SiLU; per-head learned biases by signed slot distance and for same-slot
pairs added to the attention logits). Pre-norm, biases on every linear,
non-gated feed-forward:

  u  = bf16(RMSNorm(x; g1));  q, k, v = bf16(u Wqkv^T + bqkv)
  s_ij = q_i.k_j / sqrt(d_h) + Dist[slot_j - slot_i + 63] + Same * [slot_i == slot_j]
  p_ij = bf16(exp(s_ij - max_j s_ij)),  l_i = sum_j exp(s_ij - max_j s_ij)
  o_i  = (sum_j p_ij v_j) / l_i;      x += bf16(o) Wo^T + bo
  u2 = bf16(RMSNorm(x; g2));          x += bf16(SiLU(u2 W1^T + b1)) W2^T + b2

Heads (Section 3.2: an out and an in vector per node, each of width d_e and
normalised to unit norm):

  uf = bf16(RMSNorm(x; gf));  out = bf16(v / max(|v|, 1e-12)), v = uf Wout^T + bout
  (in likewise with Win, bin)

All accumulation is float64; the named bf16(.) points are the only roundings.
Attention never crosses blocks.
"""
from __future__ import annotations

import math

import numpy as np

from .bf16 import round_bf16
from .weights import OracleWeights

RMS_EPS = 1e-6
NORM_EPS = 1e-12


def rmsnorm(x: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + RMS_EPS) * gamma


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def confidence_features(logp_block: np.ndarray) -> np.ndarray:
    """Five scalars per candidate, [B, K, 5] float64, from float32 log-probs."""
    B, K = logp_block.shape
    lp = logp_block.astype(np.float64)
    f = np.empty((B, K, 5), dtype=np.float64)
    f[..., 0] = lp
    f[..., 1] = np.exp(lp)
    f[..., 2] = lp - lp[:, :1]
    f[..., 3] = (np.arange(K, dtype=np.float64) / (K - 1)) if K > 1 else 0.0
    f[..., 4] = (np.arange(K) == 0).astype(np.float64)
    return f


def node_build(idx_block: np.ndarray, logp_block: np.ndarray, w: OracleWeights) -> np.ndarray:
    B, K = idx_block.shape
    T = B * K
    slot = np.repeat(np.arange(B), K)
    rank = np.tile(np.arange(K), B)
    f = confidence_features(logp_block).reshape(T, 5)
    hid = round_bf16(silu(f @ w["conf_w1"].T + w["conf_b1"]))
    mlp = hid @ w["conf_w2"].T + w["conf_b2"]
    emb = w.embedding_rows(idx_block.reshape(T))
    return emb + w["S"][slot] + w["R"][rank] + mlp


def lattice_attention(qkv: np.ndarray, slot: np.ndarray, heads: int, dist: np.ndarray,
                      same: np.ndarray) -> np.ndarray:
    """Bidirectional attention over one block's T tokens; qkv holds bf16 values [T, 3H]."""
    T, H3 = qkv.shape
    H = H3 // 3
    dh = H // heads
    q, k, v = qkv[:, :H], qkv[:, H:2 * H], qkv[:, 2 * H:]
    delta = slot[None, :] - slot[:, None]            # slot_key - slot_query
    same_mask = (delta == 0).astype(np.float64)
    out = np.empty((T, H), dtype=np.float64)
    for h in range(heads):
        cols = slice(h * dh, (h + 1) * dh)
        s = (q[:, cols] @ k[:, cols].T) / math.sqrt(dh)
        s = s + dist[h][delta + 63] + same[h] * same_mask
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = round_bf16(e)
        out[:, cols] = (p @ v[:, cols]) / e.sum(axis=1, keepdims=True)
    return out


def encoder_layer(x: np.ndarray, slot: np.ndarray, w: OracleWeights, l: int, heads: int,
                  trace: dict | None = None) -> np.ndarray:
    u = round_bf16(rmsnorm(x, w[f"l{l}.gamma1"]))
    qkv = round_bf16(u @ w[f"l{l}.wqkv"].T + w[f"l{l}.bqkv"])
    o = lattice_attention(qkv, slot, heads, w[f"l{l}.dist"], w[f"l{l}.same"])
    x = x + (round_bf16(o) @ w[f"l{l}.wo"].T + w[f"l{l}.bo"])
    if trace is not None:
        trace[f"l{l}.qkv"] = qkv
        trace[f"l{l}.attn"] = o
        trace[f"l{l}.x_mid"] = x.copy()
    u2 = round_bf16(rmsnorm(x, w[f"l{l}.gamma2"]))
    hid = round_bf16(silu(u2 @ w[f"l{l}.w1"].T + w[f"l{l}.b1"]))
    return x + (hid @ w[f"l{l}.w2"].T + w[f"l{l}.b2"])


def unit_rows(v: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(v * v, axis=-1, keepdims=True))
    return v / np.maximum(n, NORM_EPS)


def encode_block(idx_block: np.ndarray, logp_block: np.ndarray, w: OracleWeights,
                 trace: dict | None = None):
    """Return (outv, inv) as float64 arrays of bf16 values, shape [B, K, d_e]."""
    B, K = idx_block.shape
    d = w.dims
    slot = np.repeat(np.arange(B), K)
    x = node_build(idx_block, logp_block, w)
    if trace is not None:
        trace["x0"] = x.copy()
    for l in range(d.layers):
        x = encoder_layer(x, slot, w, l, d.heads, trace)
        if trace is not None:
            trace[f"l{l}.x"] = x.copy()
    uf = round_bf16(rmsnorm(x, w["gamma_f"]))
    outv = round_bf16(unit_rows(uf @ w["w_out"].T + w["b_out"]))
    inv = round_bf16(unit_rows(uf @ w["w_in"].T + w["b_in"]))
    return outv.reshape(B, K, d.d_e), inv.reshape(B, K, d.d_e)
