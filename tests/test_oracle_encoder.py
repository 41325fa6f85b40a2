"""Pins for the oracle's candidate encoder (CPU only).

The pages print no worked example of the head and publish no checkpoint, so
the encoder is pinned by closed forms and special cases that a dropped term,
a wrong sign or index, or a transposed operand would break, and by an
independent float64 torch build from library routines (F.rms_norm,
F.scaled_dot_product_attention with an additive mask, F.silu, F.normalize)
with the bf16 rounding points switched off.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.encoder as enc
from oracle.bf16 import round_bf16
from oracle.weights import Dims, OracleWeights

B13 = 0.333984375          # bf16(1/3), worked by hand: 1.0101010|1010.. x 2^-2 rounds up


def small_weights(H=16, heads=2, F_=24, de=8, V=50, overrides=None):
    return OracleWeights(Dims(H, heads, F_, de), V, seed=42, overrides=overrides)


def test_rmsnorm_closed_form():
    H = 64
    for c in (0.5, -3.0, 1e-3):
        y = enc.rmsnorm(np.full((1, H), c), np.full(H, 2.0))
        assert np.allclose(y, 2.0 * c / math.sqrt(c * c + enc.RMS_EPS), rtol=1e-15)


def test_rmsnorm_scale_invariance():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 128)) * 10
    g = rng.uniform(0.5, 1.5, 128)
    # equal up to the eps term: eps / mean(x^2) ~ 1e-8 here
    assert np.allclose(enc.rmsnorm(x, g), enc.rmsnorm(7.0 * x, g), rtol=1e-7)


def test_silu_values():
    assert enc.silu(np.array([1.0]))[0] == pytest.approx(0.7310585786300049, abs=1e-15)
    assert enc.silu(np.array([0.0]))[0] == 0.0
    assert abs(enc.silu(np.array([-40.0]))[0]) < 1e-15


def test_features_hand_example():
    lp = np.array([[-0.5, -1.5, -2.5]], dtype=np.float32)
    f = enc.confidence_features(lp)
    assert f[0, :, 0].tolist() == [-0.5, -1.5, -2.5]
    assert np.allclose(f[0, :, 1], np.exp([-0.5, -1.5, -2.5]), rtol=1e-15)
    assert f[0, :, 2].tolist() == [0.0, -1.0, -2.0]
    assert f[0, :, 3].tolist() == [0.0, 0.5, 1.0]
    assert f[0, :, 4].tolist() == [1.0, 0.0, 0.0]
    f1 = enc.confidence_features(np.array([[-0.25]], dtype=np.float32))
    assert f1[0, 0].tolist() == [-0.25, math.exp(-0.25), 0.0, 0.0, 1.0]


def test_node_build_is_sum_of_tables_when_mlp_is_zero():
    H = 16
    E = np.arange(50 * H, dtype=np.float64).reshape(50, H)
    S = 1000.0 * np.arange(64)[:, None] * np.ones((1, H))
    R = 0.5 * np.arange(64)[:, None] * np.ones((1, H))
    w = small_weights(H=H, overrides={"E": E, "S": S, "R": R, "conf_w2": np.zeros((H, H)),
                                      "conf_b2": np.zeros(H)})
    idx = np.array([[7, 3], [11, 40]])
    lp = np.array([[-1, -2], [-1, -3]], dtype=np.float32)
    x0 = enc.node_build(idx, lp, w)
    for t, (s, j) in enumerate([(0, 0), (0, 1), (1, 0), (1, 1)]):
        assert np.array_equal(x0[t], E[idx[s, j]] + S[s] + R[j])


def test_zero_output_projections_leave_residual_unchanged():
    H, F_ = 16, 24
    ov = {}
    for l in range(2):
        ov.update({f"l{l}.wo": np.zeros((H, H)), f"l{l}.bo": np.zeros(H),
                   f"l{l}.w2": np.zeros((H, F_)), f"l{l}.b2": np.zeros(H)})
    w = small_weights(H=H, F_=F_, overrides=ov)
    rng = np.random.default_rng(1)
    idx = rng.integers(0, 50, (3, 4))
    lp = -np.sort(np.abs(rng.standard_normal((3, 4))).astype(np.float32), axis=1)
    tr = {}
    enc.encode_block(idx, lp, w, tr)
    assert np.array_equal(tr["l0.x"], tr["x0"]) and np.array_equal(tr["l1.x"], tr["x0"])


def test_single_token_attention_returns_v():
    w = small_weights()
    tr = {}
    enc.encode_block(np.array([[5]]), np.array([[-0.5]], dtype=np.float32), w, tr)
    H = 16
    assert np.array_equal(tr["l0.attn"], tr["l0.qkv"][:, 2 * H:])


def test_uniform_attention_is_mean_of_v():
    rng = np.random.default_rng(2)
    T, H, heads = 12, 8, 2
    qkv = np.zeros((T, 3 * H))
    qkv[:, 2 * H:] = round_bf16(rng.standard_normal((T, H)))
    slot = np.repeat(np.arange(4), 3)
    o = enc.lattice_attention(qkv, slot, heads, np.zeros((heads, 127)), np.zeros(heads))
    assert np.allclose(o, qkv[:, 2 * H:].mean(0, keepdims=True), rtol=0, atol=1e-15)


def test_distance_bias_sign_and_rounding_points():
    # 3 slots x 1 candidate, 2 heads of width 3, q = k = 0, v_j = e_j per head.
    H, heads = 6, 2
    qkv = np.zeros((3, 3 * H))
    for j in range(3):
        qkv[j, 2 * H + j] = 1.0
        qkv[j, 2 * H + 3 + j] = 1.0
    dist = np.zeros((heads, 127))
    dist[0, 63 + 1] = math.log(3.0)      # head 0 favours the key one slot AFTER the query
    dist[1, 63 - 1] = math.log(3.0)      # head 1 favours the key one slot BEFORE the query
    o = enc.lattice_attention(qkv, np.arange(3), heads, dist, np.zeros(heads))
    hi, lo = 0.6, B13 * 0.6             # p = [bf16(1/3), 1, bf16(1/3)], l = 5/3 unrounded
    third = 1.0 / 3.0
    expect0 = np.array([[lo, hi, lo], [lo, lo, hi], [third, third, third]])
    expect1 = np.array([[third, third, third], [hi, lo, lo], [lo, hi, lo]])
    assert np.allclose(o[:, :3], expect0, atol=1e-15)
    assert np.allclose(o[:, 3:], expect1, atol=1e-15)


def test_same_slot_bias():
    H = 4
    qkv = np.zeros((4, 3 * H))
    qkv[:, 2 * H:] = np.eye(4)
    slot = np.array([0, 0, 1, 1])
    o = enc.lattice_attention(qkv, slot, 1, np.zeros((1, 127)), np.array([math.log(3.0)]))
    # query 0: s = [ln3, ln3, 0, 0] -> p = [1, 1, b, b], l = 8/3
    assert np.allclose(o[0], [3 / 8, 3 / 8, 3 * B13 / 8, 3 * B13 / 8], atol=1e-15)
    assert np.allclose(o[3], [3 * B13 / 8, 3 * B13 / 8, 3 / 8, 3 / 8], atol=1e-15)


def test_query_key_orientation_and_scale():
    H = 4
    qkv = np.zeros((2, 3 * H))
    qkv[0, 0] = 1.0                      # q_0 = e_0
    qkv[1, H] = 2.0                      # k_1 = 2 e_0  -> q_0.k_1 / sqrt(4) = 1
    qkv[:, 2 * H:2 * H + 2] = np.eye(2)
    o = enc.lattice_attention(qkv, np.array([0, 1]), 1, np.zeros((1, 127)), np.zeros(1))
    e1 = math.exp(-1.0)
    assert np.allclose(o[0, :2], [round_bf16(np.array([e1]))[0] / (1 + e1), 1 / (1 + e1)], atol=1e-15)
    assert np.allclose(o[1, :2], [0.5, 0.5], atol=1e-15)   # q_1 = 0: uniform


def test_head_outputs_normalised_and_rounded():
    H, de = 16, 8
    b = np.zeros(de)
    b[0], b[1] = 3.0, 4.0
    w = small_weights(H=H, de=de, overrides={"w_out": np.zeros((de, H)), "b_out": b})
    outv, inv = enc.encode_block(np.array([[1, 2]]), np.array([[-1, -2]], dtype=np.float32), w)
    # 0.6 and 0.8 rounded to bf16 by hand: 0.6015625 and 0.80078125
    assert outv[0, 0, :2].tolist() == [0.6015625, 0.80078125]
    assert np.all(outv[0, :, 2:] == 0)
    n = np.linalg.norm(inv, axis=-1)
    assert np.all(np.abs(n - 1) < 2 ** -7)


def test_encoder_layer_permutation_equivariance():
    # Position enters only through slot ids: permuting tokens together with
    # their slot ids permutes the layer's output.
    w = small_weights()
    rng = np.random.default_rng(3)
    x = rng.standard_normal((12, 16))
    slot = np.repeat(np.arange(4), 3)
    perm = rng.permutation(12)
    y = enc.encoder_layer(x, slot, w, 0, 2)
    yp = enc.encoder_layer(x[perm], slot[perm], w, 0, 2)
    assert np.allclose(yp, y[perm], rtol=0, atol=1e-12)


def _torch_encoder(idx, lp, w, heads):
    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    B, K = idx.shape
    T = B * K
    d = w.dims
    H, dh = d.hidden, d.hidden // heads
    slot = torch.arange(B).repeat_interleave(K)
    rank = torch.arange(K).repeat(B)
    lpt = t(lp)
    feats = torch.stack([lpt, lpt.exp(), lpt - lpt[:, :1],
                         (rank.view(B, K).double() / (K - 1)) if K > 1 else torch.zeros(B, K, dtype=torch.float64),
                         (rank.view(B, K) == 0).double()], dim=-1).reshape(T, 5)
    x = (t(w.embedding_rows(idx.reshape(-1))) + t(w["S"])[slot] + t(w["R"])[rank]
         + F.linear(F.silu(F.linear(feats, t(w["conf_w1"]), t(w["conf_b1"]))), t(w["conf_w2"]), t(w["conf_b2"])))
    delta = slot[None, :] - slot[:, None]
    for l in range(d.layers):
        u = F.rms_norm(x, (H,), t(w[f"l{l}.gamma1"]), eps=1e-6)
        q, k, v = F.linear(u, t(w[f"l{l}.wqkv"]), t(w[f"l{l}.bqkv"])).split(H, dim=-1)
        q, k, v = (a.view(T, heads, dh).transpose(0, 1) for a in (q, k, v))
        bias = t(w[f"l{l}.dist"])[:, delta + 63] + t(w[f"l{l}.same"])[:, None, None] * (delta == 0)
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=bias).transpose(0, 1).reshape(T, H)
        x = x + F.linear(o, t(w[f"l{l}.wo"]), t(w[f"l{l}.bo"]))
        u2 = F.rms_norm(x, (H,), t(w[f"l{l}.gamma2"]), eps=1e-6)
        x = x + F.linear(F.silu(F.linear(u2, t(w[f"l{l}.w1"]), t(w[f"l{l}.b1"]))), t(w[f"l{l}.w2"]), t(w[f"l{l}.b2"]))
    uf = F.rms_norm(x, (H,), t(w["gamma_f"]), eps=1e-6)
    out = F.normalize(F.linear(uf, t(w["w_out"]), t(w["b_out"])), dim=-1, eps=1e-12)
    inn = F.normalize(F.linear(uf, t(w["w_in"]), t(w["b_in"])), dim=-1, eps=1e-12)
    return out.numpy().reshape(B, K, -1), inn.numpy().reshape(B, K, -1)


@pytest.mark.parametrize("B,K,H,heads,F_,de", [(16, 4, 64, 2, 256, 32), (5, 3, 48, 3, 40, 16), (2, 1, 16, 1, 8, 8)])
def test_matches_independent_torch_build_without_rounding(monkeypatch, B, K, H, heads, F_, de):
    monkeypatch.setattr(enc, "round_bf16", lambda a: np.asarray(a, dtype=np.float64))
    w = OracleWeights(Dims(H, heads, F_, de), 300, seed=7)
    rng = np.random.default_rng(B * K)
    idx = rng.integers(0, 300, (B, K))
    lp = -np.sort(np.abs(rng.standard_normal((B, K))).astype(np.float32) * 3, axis=1)
    outv, inv = enc.encode_block(idx, lp, w)
    to, ti = _torch_encoder(idx, lp, w, heads)
    assert np.allclose(outv, to, rtol=0, atol=1e-12)
    assert np.allclose(inv, ti, rtol=0, atol=1e-12)


def test_rounding_points_change_result_only_slightly():
    w = small_weights(H=64, heads=2, F_=256, de=32, V=1000)
    rng = np.random.default_rng(4)
    idx = rng.integers(0, 1000, (16, 4))
    lp = -np.sort(np.abs(rng.standard_normal((16, 4))).astype(np.float32) * 3, axis=1)
    outv, _ = enc.encode_block(idx, lp, w)
    to, _ = _torch_encoder(idx, lp, w, 2)
    err = np.abs(outv - to).max()
    assert 0 < err < 0.05


# --- where the encoder rounds to bfloat16 ----------------------------------
# The pages fix no rounding; the reading taken (bf16 at every GEMM input and at
# the attention probabilities, float32 residual stream, norms and softmax sums)
# names nine points. A second float64 torch build places them with torch's own
# bfloat16 conversion (float64 -> float32 -> bfloat16, round to nearest even at
# each step, the way a float32 producer stores bfloat16). The oracle must agree
# with it to float64 round-off, and dropping any single point from the torch
# build must break that agreement, so a missing or an extra rounding in the
# oracle cannot pass.
ROUND_POINTS = ("conf_hidden", "u1", "qkv", "probs", "attn_out", "u2", "ffn_hidden", "uf", "heads")


def _bf16(a, name, skip):
    return a if name in skip else a.to(torch.bfloat16).to(torch.float64)


def _torch_encoder_rounded(idx, lp, w, heads, skip=()):
    t = lambda a: torch.tensor(np.asarray(a), dtype=torch.float64)
    B, K = idx.shape
    T = B * K
    d = w.dims
    H, dh = d.hidden, d.hidden // heads
    slot = torch.arange(B).repeat_interleave(K)
    rank = torch.arange(K).repeat(B)
    lpt = t(lp)
    feats = torch.stack([lpt, lpt.exp(), lpt - lpt[:, :1],
                         (rank.view(B, K).double() / (K - 1)) if K > 1 else torch.zeros(B, K, dtype=torch.float64),
                         (rank.view(B, K) == 0).double()], dim=-1).reshape(T, 5)
    hid = _bf16(F.silu(F.linear(feats, t(w["conf_w1"]), t(w["conf_b1"]))), "conf_hidden", skip)
    x = t(w.embedding_rows(idx.reshape(-1))) + t(w["S"])[slot] + t(w["R"])[rank] \
        + F.linear(hid, t(w["conf_w2"]), t(w["conf_b2"]))
    delta = slot[None, :] - slot[:, None]
    for l in range(d.layers):
        u = _bf16(F.rms_norm(x, (H,), t(w[f"l{l}.gamma1"]), eps=1e-6), "u1", skip)
        qkv = _bf16(F.linear(u, t(w[f"l{l}.wqkv"]), t(w[f"l{l}.bqkv"])), "qkv", skip)
        q, k, v = (a.reshape(T, heads, dh).transpose(0, 1) for a in qkv.split(H, dim=-1))
        bias = t(w[f"l{l}.dist"])[:, delta + 63] + t(w[f"l{l}.same"])[:, None, None] * (delta == 0)
        s = torch.matmul(q, k.transpose(1, 2).contiguous()) / math.sqrt(dh) + bias
        e = torch.exp(s - s.amax(dim=-1, keepdim=True))
        o = torch.matmul(_bf16(e, "probs", skip), v) / e.sum(dim=-1, keepdim=True)
        o = _bf16(o.transpose(0, 1).reshape(T, H), "attn_out", skip)
        x = x + F.linear(o, t(w[f"l{l}.wo"]), t(w[f"l{l}.bo"]))
        u2 = _bf16(F.rms_norm(x, (H,), t(w[f"l{l}.gamma2"]), eps=1e-6), "u2", skip)
        hd = _bf16(F.silu(F.linear(u2, t(w[f"l{l}.w1"]), t(w[f"l{l}.b1"]))), "ffn_hidden", skip)
        x = x + F.linear(hd, t(w[f"l{l}.w2"]), t(w[f"l{l}.b2"]))
    uf = _bf16(F.rms_norm(x, (H,), t(w["gamma_f"]), eps=1e-6), "uf", skip)
    out = _bf16(F.normalize(F.linear(uf, t(w["w_out"]), t(w["b_out"])), dim=-1, eps=1e-12), "heads", skip)
    inn = _bf16(F.normalize(F.linear(uf, t(w["w_in"]), t(w["b_in"])), dim=-1, eps=1e-12), "heads", skip)
    return out.numpy().reshape(B, K, -1), inn.numpy().reshape(B, K, -1)


def _rounded_case(B=16, K=4, H=64, heads=2, F_=256, de=32, V=1000, seed=5):
    w = OracleWeights(Dims(H, heads, F_, de), V, seed=seed)
    rng = np.random.default_rng(seed)
    idx = rng.integers(0, V, (B, K))
    lp = -np.sort(np.abs(rng.standard_normal((B, K))).astype(np.float32) * 3, axis=1)
    return w, idx, lp


@pytest.mark.parametrize("B,K,H,heads,F_,de", [(16, 4, 64, 2, 256, 32), (7, 5, 96, 3, 160, 24)])
def test_rounding_points_match_torch_bfloat16_build(B, K, H, heads, F_, de):
    w, idx, lp = _rounded_case(B, K, H, heads, F_, de)
    outv, inv = enc.encode_block(idx, lp, w)
    to, ti = _torch_encoder_rounded(idx, lp, w, heads)
    # every stored output is a bf16 value on both sides; they agree exactly
    # unless a float64 summation-order difference straddles a rounding
    # boundary (probability ~1e-9 per value), which these cases do not hit
    assert np.array_equal(outv, to) and np.array_equal(inv, ti)


@pytest.mark.parametrize("point", ROUND_POINTS)
def test_each_rounding_point_is_load_bearing(point):
    # the agreement above is not vacuous: the torch build without any one of
    # the nine roundings moves the outputs far beyond float64 round-off
    w, idx, lp = _rounded_case()
    outv, inv = enc.encode_block(idx, lp, w)
    to, ti = _torch_encoder_rounded(idx, lp, w, 2, skip=(point,))
    assert max(np.abs(outv - to).max(), np.abs(inv - ti).max()) > 1e-4
