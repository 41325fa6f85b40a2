"""Why the pair-cosine tolerance is statistical plus a bf16 bound (CPU only).

The encoder rounds its activations to bfloat16 at every GEMM input and at the
attention probabilities. Two implementations of those same rounding points
that differ only in accumulation precision (float32 here, float64 in the
oracle) round a few values differently; each such flip perturbs the next
layer's inputs, which flips more roundings, and the cosines drift by up to
about 1e-3. This test builds the encoder independently in float32 numpy and
shows that drift: it reaches the order of the 1e-3 bar on its own, while
staying inside the bf16 bound 2^-7 that the GPU parity tests use as a hard
ceiling.
"""
import math

import numpy as np

import synth
import oracle
from oracle.bf16 import round_bf16
from oracle.scores import pair_scores
from helpers import COS_HARD


def _f32(a):
    return np.asarray(a, np.float32).astype(np.float64)


def _mm(a, b):
    return (np.asarray(a, np.float32) @ np.asarray(b, np.float32)).astype(np.float64)


def _rms(x, g):
    x = np.asarray(x, np.float32)
    ms = (x * x).sum(-1, keepdims=True, dtype=np.float32) / np.float32(x.shape[-1])
    return ((x * (np.float32(1) / np.sqrt(ms + np.float32(1e-6)))) * np.asarray(g, np.float32)).astype(np.float64)


def _silu(z):
    z = np.asarray(z, np.float32)
    return (z / (np.float32(1) + np.exp(-z))).astype(np.float64)


def encoder_float32(idx, logp, w, K):
    B = idx.shape[0]
    T, d = B * K, w.dims
    H, heads = d.hidden, d.heads
    dh = H // heads
    slot, rank = np.repeat(np.arange(B), K), np.tile(np.arange(K), B)
    lp = logp.astype(np.float32)
    f = np.stack([lp, np.exp(lp), lp - lp[:, :1], np.tile(np.arange(K, dtype=np.float32) / max(K - 1, 1), (B, 1)),
                  np.tile((np.arange(K) == 0).astype(np.float32), (B, 1))], -1).reshape(T, 5)
    hid = round_bf16(_silu(_mm(f, w["conf_w1"].T) + w["conf_b1"]))
    x = _f32(_f32(w.embedding_rows(idx.reshape(T)) + w["S"][slot]) + w["R"][rank])
    x = _f32(x + _f32(_mm(hid, w["conf_w2"].T) + w["conf_b2"]))
    delta = slot[None, :] - slot[:, None]
    for l in range(d.layers):
        u = round_bf16(_rms(x, w[f"l{l}.gamma1"]))
        qkv = round_bf16(_mm(u, w[f"l{l}.wqkv"].T) + w[f"l{l}.bqkv"])
        o = np.empty((T, H))
        for h in range(heads):
            c = slice(h * dh, (h + 1) * dh)
            s = _f32(_mm(qkv[:, c], qkv[:, H:2 * H][:, c].T) * np.float32(1 / math.sqrt(dh)))
            s = _f32(s + w[f"l{l}.dist"][h][delta + 63] + w[f"l{l}.same"][h] * (delta == 0))
            e = _f32(np.exp(np.asarray(s - s.max(1, keepdims=True), np.float32)))
            o[:, c] = _f32(_mm(round_bf16(e), qkv[:, 2 * H:][:, c]) / e.sum(1, keepdims=True))
        x = _f32(x + _f32(_mm(round_bf16(o), w[f"l{l}.wo"].T) + w[f"l{l}.bo"]))
        u2 = round_bf16(_rms(x, w[f"l{l}.gamma2"]))
        hd = round_bf16(_silu(_mm(u2, w[f"l{l}.w1"].T) + w[f"l{l}.b1"]))
        x = _f32(x + _f32(_mm(hd, w[f"l{l}.w2"].T) + w[f"l{l}.b2"]))
    uf = round_bf16(_rms(x, w["gamma_f"]))
    heads_out = []
    for wn, bn in (("w_out", "b_out"), ("w_in", "b_in")):
        v = _f32(_mm(uf, w[wn].T) + w[bn])
        heads_out.append(round_bf16(v / np.maximum(np.sqrt((v * v).sum(-1, keepdims=True)), 1e-12)).reshape(B, K, -1))
    return heads_out


def test_float32_build_drifts_to_the_bar_but_not_past_the_bound():
    V, K = 2048, 8
    w = synth.Workload("drift", 2, 16, V, K, 128, 1, 512, 64, "bf16", "spiked")
    synth.WORKLOADS_ORDER.append("drift")
    try:
        host = synth.make_logits(w)
    finally:
        synth.WORKLOADS_ORDER.remove("drift")
    ow = oracle.OracleWeights(oracle.Dims(128, 1, 512, 64), V, synth.WEIGHTS_SEED)
    worst = 0.0
    for b in range(2):
        r = oracle.rerank_block(host[b], K, ow, 1.0)
        o32, i32 = encoder_float32(r.idx, r.logp, ow, K)
        d = np.abs(pair_scores(o32, i32).astype(np.float64) - r.cos)
        worst = max(worst, d.max())
        assert np.mean(o32 != r.outv) > 0.05      # the cascade reaches the stored vectors
    assert 5e-4 < worst < COS_HARD


def test_float32_drift_rate_of_the_wide_odd_shape():
    """The wide odd shape (H = 2560, 15 slots, K = 7) drifts more: the float32
    build misses 1e-3 on more than 0.1 % of its cosines (the bar of the main
    workloads), still inside the bf16 bound; its GPU case uses fraction 0.995."""
    w = synth.WORKLOADS["odd_h2560"]
    host = synth.make_logits(w)
    ow = oracle.OracleWeights(oracle.Dims(w.hidden, w.heads, w.ffn, w.d_e), w.vocab, synth.WEIGHTS_SEED)
    bad = total = 0
    worst = 0.0
    for b in (0, 1):
        r = oracle.rerank_block(host[b], w.topk, ow, 1.0)
        o32, i32 = encoder_float32(r.idx, r.logp, ow, w.topk)
        d = np.abs(pair_scores(o32, i32).astype(np.float64) - r.cos)
        bad += int((d > 1e-3 * np.maximum(1.0, np.abs(r.cos))).sum())
        total += d.size
        worst = max(worst, d.max())
    assert 0.001 < bad / total < 0.005
    assert worst < COS_HARD
