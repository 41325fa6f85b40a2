"""Pins for the oracle of the paper's own head (CPU only).

No trained head or worked example is published, so, as for the lattice head,
the pins are an independent float64 torch build from library routines
(F.rms_norm, F.linear, torch.cat, F.silu, F.normalize, scaled-dot-product
attention) with the bf16 rounding points switched off, and closed forms that a
dropped term, a swapped operand or a wrong slot index would break.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.encoder as enc
import oracle.paper_head as ph
from oracle.weights import Dims, OracleWeights
from oracle.scores import pair_scores
from oracle.walk import greedy_walk


def weights(H=16, heads=2, F_=24, de=8, V=60, Ht=32, Hd=24, overrides=None, seed=42):
    return OracleWeights(Dims(H, heads, F_, de, target_hidden=Ht, drafter_hidden=Hd), V, seed=seed,
                         overrides=overrides)


def inputs(rng, B, K, V, Ht, Hd):
    idx = np.stack([rng.permutation(V)[:K] for _ in range(B)])
    lp = -np.sort(np.abs(rng.standard_normal((B, K))).astype(np.float32) * 3, axis=1)
    from oracle.bf16 import round_bf16
    hidden = round_bf16(rng.standard_normal((B, Hd)))
    target = round_bf16(rng.standard_normal(Ht))
    return idx, lp, hidden, target


def _torch_paper(idx, lp, hidden, target, w):
    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    d = w.dims
    B, K = idx.shape
    H, heads = d.hidden, d.heads
    dh = H // heads
    Tp = (B - 1) * K
    slot = torch.arange(1, B).repeat_interleave(K)
    rank = torch.arange(K).repeat(B - 1)
    lpt = t(lp)[1:]
    feats = torch.stack([lpt, lpt.exp(), lpt - t(lp)[1:, :1],
                         (rank.view(B - 1, K).double() / (K - 1)) if K > 1 else torch.zeros(B - 1, K, dtype=torch.float64),
                         (rank.view(B - 1, K) == 0).double()], dim=-1).reshape(Tp, 5)
    mlp = F.linear(F.silu(F.linear(feats, t(w["conf_w1"]), t(w["conf_b1"]))), t(w["conf_w2"]), t(w["conf_b2"]))
    emb = F.linear(t(w.embedding_rows(idx[1:].reshape(-1), "E_t")), t(w["w_emb"]), t(w["b_emb"]))
    hp = F.linear(t(hidden)[1:], t(w["w_hid"]), t(w["b_hid"]))[slot - 1]
    x = emb + hp + mlp + t(w["S"])[slot] + t(w["R"])[rank]
    delta = slot[None, :] - slot[:, None]
    for l in range(d.layers):
        u = F.rms_norm(x, (H,), t(w[f"l{l}.gamma1"]), eps=1e-6)
        q, k, v = F.linear(u, t(w[f"l{l}.wqkv"]), t(w[f"l{l}.bqkv"])).split(H, dim=-1)
        q, k, v = (a.view(Tp, heads, dh).transpose(0, 1) for a in (q, k, v))
        bias = t(w[f"l{l}.dist"])[:, delta + 63] + t(w[f"l{l}.same"])[:, None, None] * (delta == 0)
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=bias).transpose(0, 1).reshape(Tp, H)
        x = x + F.linear(o, t(w[f"l{l}.wo"]), t(w[f"l{l}.bo"]))
        u2 = F.rms_norm(x, (H,), t(w[f"l{l}.gamma2"]), eps=1e-6)
        x = x + F.linear(F.silu(F.linear(u2, t(w[f"l{l}.w1"]), t(w[f"l{l}.b1"]))), t(w[f"l{l}.w2"]), t(w[f"l{l}.b2"]))
    u = F.rms_norm(x, (H,), t(w["gamma_f"]), eps=1e-6)
    tp = F.linear(F.rms_norm(t(target), (d.target_hidden,), t(w["gamma_t"]), eps=1e-6), t(w["w_tgt"]), t(w["b_tgt"]))
    tpb = tp.expand(Tp, H)
    y = F.silu(F.linear(torch.cat([u, tpb, u * tpb], dim=1), t(w["w_fuse"]), t(w["b_fuse"])))
    out = F.normalize(F.linear(y, t(w["w_out"]), t(w["b_out"])), dim=-1, eps=1e-12)
    inn = F.normalize(F.linear(y, t(w["w_in"]), t(w["b_in"])), dim=-1, eps=1e-12)
    o0 = F.normalize(F.linear(tp, t(w["w_anchor"]), t(w["b_anchor"])), dim=-1, eps=1e-12)
    return out.numpy().reshape(B - 1, K, -1), inn.numpy().reshape(B - 1, K, -1), o0.numpy()


@pytest.mark.parametrize("B,K,H,heads,F_,de,Ht,Hd", [(16, 4, 64, 2, 128, 32, 128, 96), (5, 3, 48, 3, 40, 16, 32, 24),
                                                    (2, 1, 16, 1, 8, 8, 16, 16)])
def test_matches_independent_torch_build_without_rounding(monkeypatch, B, K, H, heads, F_, de, Ht, Hd):
    ident = lambda a: np.asarray(a, dtype=np.float64)
    monkeypatch.setattr(enc, "round_bf16", ident)
    monkeypatch.setattr(ph, "round_bf16", ident)
    w = weights(H, heads, F_, de, 300, Ht, Hd, seed=7)
    rng = np.random.default_rng(B * K + H)
    idx, lp, hidden, target = inputs(rng, B, K, 300, Ht, Hd)
    outv, inv = ph.encode_block_paper(idx, lp, hidden, target, w)
    to, ti, o0 = _torch_paper(idx, lp, hidden, target, w)
    assert np.allclose(outv[1:], to, rtol=0, atol=1e-12)
    assert np.allclose(inv[1:], ti, rtol=0, atol=1e-12)
    assert np.allclose(outv[0], np.broadcast_to(o0, outv[0].shape), rtol=0, atol=1e-12)
    assert np.all(inv[0] == 0)


def test_rounding_points_change_result_only_slightly():
    w = weights(64, 2, 128, 32, 300, 128, 96)
    rng = np.random.default_rng(11)
    idx, lp, hidden, target = inputs(rng, 16, 4, 300, 128, 96)
    outv, _ = ph.encode_block_paper(idx, lp, hidden, target, w)
    to, _, _ = _torch_paper(idx, lp, hidden, target, w)
    err = np.abs(outv[1:] - to).max()
    assert 0 < err < 0.05


def test_constant_fusion_output_makes_every_pair_score_equal():
    H, de = 16, 8
    w = weights(H=H, de=de, overrides={"w_fuse": np.zeros((H, 3 * H)), "b_fuse": np.linspace(-1, 1, H)})
    rng = np.random.default_rng(12)
    idx, lp, hidden, target = inputs(rng, 6, 4, 60, 32, 24)
    outv, inv = ph.encode_block_paper(idx, lp, hidden, target, w)
    assert np.all(outv[1:] == outv[1, 0]) and np.all(inv[1:] == inv[1, 0])
    cos = pair_scores(outv, inv)
    for s in range(1, 5):
        assert np.all(cos[s] == cos[s][0, 0])
    # sigma * cos rule: every step ties, the lowest index wins
    r = greedy_walk(idx, lp, cos, 8.0, use_logp=False)
    assert r.choice.tolist() == [0] * 6


def test_zero_target_projection_reduces_fusion_to_a_plain_layer():
    H = 16
    w0 = weights(H=H)
    wf = w0["w_fuse"]
    w = weights(H=H, overrides={"w_tgt": np.zeros((H, 32)), "b_tgt": np.zeros(H)})
    rng = np.random.default_rng(13)
    idx, lp, hidden, target = inputs(rng, 4, 3, 60, 32, 24)
    tr = {}
    ph.encode_block_paper(idx, lp, hidden, target, w, tr)
    assert np.all(tr["tb"] == 0)
    from oracle.bf16 import round_bf16
    # recompute from the layer output recorded by the trace
    xl = tr["x_last"]
    u = round_bf16(enc.rmsnorm(xl, w["gamma_f"]))
    expect = round_bf16(enc.silu(u @ wf[:, :H].T + w["b_fuse"]))
    assert np.array_equal(tr["y"], expect)


def test_anchor_vector_hand_example():
    H, de = 16, 8
    b = np.zeros(de)
    b[0], b[1] = 3.0, 4.0
    w = weights(H=H, de=de, overrides={"w_anchor": np.zeros((de, H)), "b_anchor": b})
    rng = np.random.default_rng(14)
    idx, lp, hidden, target = inputs(rng, 3, 2, 60, 32, 24)
    outv, inv = ph.encode_block_paper(idx, lp, hidden, target, w)
    # 0.6 and 0.8 rounded to bf16 by hand: 0.6015625 and 0.80078125
    assert outv[0, :, :2].tolist() == [[0.6015625, 0.80078125]] * 2
    assert np.all(outv[0, :, 2:] == 0)


def test_anchor_slot_candidates_do_not_enter_the_lattice():
    w = weights()
    rng = np.random.default_rng(15)
    idx, lp, hidden, target = inputs(rng, 5, 3, 60, 32, 24)
    a = ph.encode_block_paper(idx, lp, hidden, target, w)
    idx2, lp2, hidden2 = idx.copy(), lp.copy(), hidden.copy()
    idx2[0] = [59, 58, 57]
    lp2[0] = [-0.1, -0.2, -9.0]
    hidden2[0] = 7.0
    b = ph.encode_block_paper(idx2, lp2, hidden2, target, w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # while a drafted slot's hidden state reaches every node of the block
    hidden2 = hidden.copy()
    hidden2[2] += 1.0
    c = ph.encode_block_paper(idx, lp, hidden2, target, w)
    assert not np.array_equal(a[0][4], c[0][4])


def test_node_terms():
    H, Ht, Hd, V = 16, 32, 24, 60
    w = weights(H=H, Ht=Ht, Hd=Hd, V=V, overrides={"conf_w2": np.zeros((H, H)), "conf_b2": np.zeros(H)})
    rng = np.random.default_rng(16)
    idx, lp, hidden, target = inputs(rng, 3, 2, V, Ht, Hd)
    x0 = ph.node_build_paper(idx, lp, hidden, w)
    E_t = w.embedding_rows(np.arange(V), "E_t")
    for t_, (s, r) in enumerate([(1, 0), (1, 1), (2, 0), (2, 1)]):
        expect = (E_t[idx[s, r]] @ w["w_emb"].T + w["b_emb"] + hidden[s] @ w["w_hid"].T + w["b_hid"]
                  + w["S"][s] + w["R"][r])
        assert np.allclose(x0[t_], expect, rtol=0, atol=1e-12)


# --- where the paper's head rounds to bfloat16 -------------------------------
# The lattice head's nine points plus the target branch and the fusion: the
# normalised target state, t', the elementwise product u*t', the fused state y
# and the anchor vector. A float64 torch build places them with torch's own
# bfloat16 conversion; the oracle must agree exactly, and dropping any one
# point from the torch build must break the agreement.
PAPER_ROUND_POINTS = ("conf_hidden", "u1", "qkv", "probs", "attn_out", "u2", "ffn_hidden", "uf",
                      "t_norm", "t_proj", "prod", "fused", "heads", "anchor")


def _bf16(a, name, skip):
    return a if name in skip else a.to(torch.bfloat16).to(torch.float64)


def _torch_paper_rounded(idx, lp, hidden, target, w, skip=()):
    import math
    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    d = w.dims
    B, K = idx.shape
    H, heads = d.hidden, d.heads
    dh = H // heads
    Tp = (B - 1) * K
    slot = torch.arange(1, B).repeat_interleave(K)
    rank = torch.arange(K).repeat(B - 1)
    lpt = t(lp)[1:]
    feats = torch.stack([lpt, lpt.exp(), lpt - t(lp)[1:, :1],
                         (rank.view(B - 1, K).double() / (K - 1)) if K > 1 else torch.zeros(B - 1, K, dtype=torch.float64),
                         (rank.view(B - 1, K) == 0).double()], dim=-1).reshape(Tp, 5)
    hid = _bf16(F.silu(F.linear(feats, t(w["conf_w1"]), t(w["conf_b1"]))), "conf_hidden", skip)
    mlp = F.linear(hid, t(w["conf_w2"]), t(w["conf_b2"]))
    emb = F.linear(t(w.embedding_rows(idx[1:].reshape(-1), "E_t")), t(w["w_emb"]), t(w["b_emb"]))
    hp = F.linear(t(hidden)[1:], t(w["w_hid"]), t(w["b_hid"]))[slot - 1]
    x = emb + hp + mlp + t(w["S"])[slot] + t(w["R"])[rank]
    delta = slot[None, :] - slot[:, None]
    for l in range(d.layers):
        u = _bf16(F.rms_norm(x, (H,), t(w[f"l{l}.gamma1"]), eps=1e-6), "u1", skip)
        qkv = _bf16(F.linear(u, t(w[f"l{l}.wqkv"]), t(w[f"l{l}.bqkv"])), "qkv", skip)
        q, k, v = (a.reshape(Tp, heads, dh).transpose(0, 1) for a in qkv.split(H, dim=-1))
        bias = t(w[f"l{l}.dist"])[:, delta + 63] + t(w[f"l{l}.same"])[:, None, None] * (delta == 0)
        s = torch.matmul(q, k.transpose(1, 2).contiguous()) / math.sqrt(dh) + bias
        e = torch.exp(s - s.amax(dim=-1, keepdim=True))
        o = torch.matmul(_bf16(e, "probs", skip), v) / e.sum(dim=-1, keepdim=True)
        o = _bf16(o.transpose(0, 1).reshape(Tp, H), "attn_out", skip)
        x = x + F.linear(o, t(w[f"l{l}.wo"]), t(w[f"l{l}.bo"]))
        u2 = _bf16(F.rms_norm(x, (H,), t(w[f"l{l}.gamma2"]), eps=1e-6), "u2", skip)
        hd = _bf16(F.silu(F.linear(u2, t(w[f"l{l}.w1"]), t(w[f"l{l}.b1"]))), "ffn_hidden", skip)
        x = x + F.linear(hd, t(w[f"l{l}.w2"]), t(w[f"l{l}.b2"]))
    u = _bf16(F.rms_norm(x, (H,), t(w["gamma_f"]), eps=1e-6), "uf", skip)
    tn = _bf16(F.rms_norm(t(target), (d.target_hidden,), t(w["gamma_t"]), eps=1e-6), "t_norm", skip)
    tp = _bf16(F.linear(tn, t(w["w_tgt"]), t(w["b_tgt"])), "t_proj", skip)
    tpb = tp.expand(Tp, H)
    cat = torch.cat([u, tpb, _bf16(u * tpb, "prod", skip)], dim=1)
    y = _bf16(F.silu(F.linear(cat, t(w["w_fuse"]), t(w["b_fuse"]))), "fused", skip)
    out = _bf16(F.normalize(F.linear(y, t(w["w_out"]), t(w["b_out"])), dim=-1, eps=1e-12), "heads", skip)
    inn = _bf16(F.normalize(F.linear(y, t(w["w_in"]), t(w["b_in"])), dim=-1, eps=1e-12), "heads", skip)
    o0 = _bf16(F.normalize(F.linear(tp, t(w["w_anchor"]), t(w["b_anchor"])), dim=-1, eps=1e-12), "anchor", skip)
    return out.numpy().reshape(B - 1, K, -1), inn.numpy().reshape(B - 1, K, -1), o0.numpy()


def _paper_rounded_case(B=16, K=4, H=64, heads=2, F_=128, de=32, Ht=128, Hd=96, seed=21):
    w = weights(H, heads, F_, de, 300, Ht, Hd, seed=seed)
    idx, lp, hidden, target = inputs(np.random.default_rng(seed), B, K, 300, Ht, Hd)
    return w, idx, lp, hidden, target


@pytest.mark.parametrize("B,K,H,heads,F_,de,Ht,Hd", [(16, 4, 64, 2, 128, 32, 128, 96), (6, 5, 48, 3, 40, 16, 32, 24)])
def test_rounding_points_match_torch_bfloat16_build(B, K, H, heads, F_, de, Ht, Hd):
    w, idx, lp, hidden, target = _paper_rounded_case(B, K, H, heads, F_, de, Ht, Hd)
    outv, inv = ph.encode_block_paper(idx, lp, hidden, target, w)
    to, ti, o0 = _torch_paper_rounded(idx, lp, hidden, target, w)
    assert np.array_equal(outv[1:], to) and np.array_equal(inv[1:], ti)
    assert np.array_equal(outv[0], np.broadcast_to(o0, outv[0].shape))


@pytest.mark.parametrize("point", PAPER_ROUND_POINTS)
def test_each_rounding_point_is_load_bearing(point):
    w, idx, lp, hidden, target = _paper_rounded_case()
    outv, inv = ph.encode_block_paper(idx, lp, hidden, target, w)
    to, ti, o0 = _torch_paper_rounded(idx, lp, hidden, target, w, skip=(point,))
    diff = max(np.abs(outv[1:] - to).max(), np.abs(inv[1:] - ti).max(), np.abs(outv[0, 0] - o0).max())
    assert diff > 1e-4
