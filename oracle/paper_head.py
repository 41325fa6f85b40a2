"""The paper's own head: drafter hidden state, target fusion, anchor out vector.
TEST INFRASTRUCTURE ONLY.

LiLiCorr paper, Section 3.2 and Appendix A "Architecture":
  * the lattice holds the B-1 drafted slots (1..B-1) x K candidates; the anchor
    (slot 0, the last committed token) has no candidates;
  * a node sums four equal-width terms: the target's frozen input embedding of
    the token projected down, the drafter's hidden state at the slot projected
    down (shared by the slot's K candidates), the confidence network over the
    five scalars, and the slot and rank tables:
        x0 = (E_t[tok] W_emb^T + b_emb) + (h_s W_hid^T + b_hid) + MLP(f) + S[s] + R[r]
  * the two lattice-transformer layers are those of oracle.encoder (slot ids
    1..B-1; only their differences enter the attention biases);
  * the target state (the target's hidden states behind the last verified
    token, collapsed across its captured layers -- an input here) is
    normalised and projected to the head width:
        t' = bf16(RMSNorm(t; gamma_t)) W_tgt^T + b_tgt
  * after the transformer each node is fused with t' by one linear layer over
    the concatenation [candidate state, t', their elementwise product],
    followed by SiLU; the out and in heads read the fused state:
        u = bf16(RMSNorm(x; gamma_f)),  tb = bf16(t')
        y = bf16(SiLU([u, tb, bf16(u * tb)] W_fuse^T + b_fuse))
        out = bf16(unit(y W_out^T + b_out)),  in = bf16(unit(y W_in^T + b_in))
  * a third head emits the anchor's single out vector from the target state:
        o_0 = bf16(unit(tb W_anchor^T + b_anchor))
  * the matching term of Eq. (1) couples the anchor to slot 1 through o_0
    (K_0 = 1) and slot s to slot s+1 through the candidates' out vectors.

Readings taken here (the pages fix the structure, not these details): the
candidate state fused with t' is the final RMS-normalised one (the same state
the lattice head's out/in heads read); bf16 rounding at every GEMM input as in
oracle.encoder (the hidden and target states and the embedding rows arrive as
bf16, t' and the elementwise product are rounded before the fusion layer);
every linear has a bias. In the [B, K, d_e] output layout slot 0 carries o_0
in every candidate row (its in vectors are zero and unused), so the pair
scores and commit rules of the lattice head apply unchanged, the walk starting
from slot 0's candidate 0.
"""
from __future__ import annotations

import numpy as np

from .bf16 import round_bf16
from .encoder import confidence_features, encoder_layer, rmsnorm, silu, unit_rows
from .weights import OracleWeights


def node_build_paper(idx_block, logp_block, hidden_block, w: OracleWeights) -> np.ndarray:
    """x0 for the (B-1) x K drafted candidates, [T', H] float64 (slot-major)."""
    B, K = idx_block.shape
    Tp = (B - 1) * K
    slot = np.repeat(np.arange(1, B), K)
    rank = np.tile(np.arange(K), B - 1)
    f = confidence_features(logp_block)[1:].reshape(Tp, 5)
    hid = round_bf16(silu(f @ w["conf_w1"].T + w["conf_b1"]))
    mlp = hid @ w["conf_w2"].T + w["conf_b2"]
    emb = w.embedding_rows(idx_block[1:].reshape(Tp), "E_t") @ w["w_emb"].T + w["b_emb"]
    hproj = np.asarray(hidden_block, dtype=np.float64)[1:] @ w["w_hid"].T + w["b_hid"]
    return emb + hproj[slot - 1] + mlp + w["S"][slot] + w["R"][rank]


def target_projection(target, w: OracleWeights) -> np.ndarray:
    """bf16(t'), [H] float64."""
    tn = round_bf16(rmsnorm(np.asarray(target, dtype=np.float64)[None, :], w["gamma_t"]))
    return round_bf16(tn @ w["w_tgt"].T + w["b_tgt"])[0]


def encode_block_paper(idx_block, logp_block, hidden_block, target, w: OracleWeights,
                       trace: dict | None = None):
    """Return (outv, inv) [B, K, d_e] float64 arrays of bf16 values; slot 0 rows carry o_0."""
    B, K = idx_block.shape
    d = w.dims
    slot = np.repeat(np.arange(1, B), K)
    x = node_build_paper(idx_block, logp_block, hidden_block, w)
    if trace is not None:
        trace["x0"] = x.copy()
    for l in range(d.layers):
        x = encoder_layer(x, slot, w, l, d.heads, trace)
    if trace is not None:
        trace["x_last"] = x.copy()
    u = round_bf16(rmsnorm(x, w["gamma_f"]))
    tb = target_projection(target, w)
    cat = np.concatenate([u, np.broadcast_to(tb, u.shape), round_bf16(u * tb)], axis=1)
    y = round_bf16(silu(cat @ w["w_fuse"].T + w["b_fuse"]))
    if trace is not None:
        trace["tb"], trace["y"] = tb, y
    out_l = round_bf16(unit_rows(y @ w["w_out"].T + w["b_out"]))
    in_l = round_bf16(unit_rows(y @ w["w_in"].T + w["b_in"]))
    o0 = round_bf16(unit_rows(tb[None, :] @ w["w_anchor"].T + w["b_anchor"]))[0]
    outv = np.zeros((B, K, d.d_e))
    inv = np.zeros((B, K, d.d_e))
    outv[0] = o0
    outv[1:] = out_l.reshape(B - 1, K, d.d_e)
    inv[1:] = in_l.reshape(B - 1, K, d.d_e)
    return outv, inv
