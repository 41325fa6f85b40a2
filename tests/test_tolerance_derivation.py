"""Where the parity bars on cosines and in/out vectors come from (CPU only).

The encoder rounds its activations to bfloat16 at every GEMM input and at the
attention probabilities. Two implementations of those same rounding points
that differ only in accumulation precision (float32 here, float64 in the
oracle) round a few values differently; each flip perturbs the next layer's
inputs, which flips more roundings. This module builds the encoder
independently in float32 numpy and measures that drift at the workloads' real
shapes (H = 1024 with K = 8 and K = 16, H = 2048 with K = 32). It asserts
that
  * the drift is real: some cosine misses 1e-3 and ~8 % of the stored vector
    components differ by more than one bf16 ulp, so neither an elementwise
    1e-3 bar on every cosine nor bit-equal vectors is a bar any float32
    implementation meets;
  * the bars the GPU tests use (tests/helpers.py) hold the float32 build with
    a margin of about two: COS_MAX, COS_FRACTION, VEC_MAX, VEC_MEAN and
    VEC_ULP_FRACTION;
  * the float32 build commits the oracle's tokens, or differs only at slots
    whose oracle score gap is within 1e-3 (the token excuse of the GPU tests).
"""
import math

import numpy as np

import synth
import oracle
from oracle.bf16 import round_bf16
from oracle.scores import pair_scores
from helpers import (TOL, COS_MAX, COS_FRACTION, VEC_MAX, VEC_MEAN, VEC_ULP_FRACTION,
                     bf16_ulp, compare_walk)
from oracle.walk import greedy_walk


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


def _drift(name, tier, blocks):
    """float32-build statistics against the oracle over the given blocks."""
    w = synth.WORKLOADS[name]
    host = synth.make_logits(w, tier, num_blocks=max(blocks) + 1)
    ow = oracle.OracleWeights(oracle.Dims(w.hidden, w.heads, w.ffn, w.d_e), w.vocab, synth.WEIGHTS_SEED)
    cos_rel, vec_d, vec_ulp, excused, slots = [], [], [], [], 0
    for b in blocks:
        r = oracle.rerank_block(host[b], w.topk, ow, 1.0)
        o32, i32 = encoder_float32(r.idx, r.logp, ow, w.topk)
        c32 = pair_scores(o32, i32)
        cos_rel.append((np.abs(c32.astype(np.float64) - r.cos) / np.maximum(1.0, np.abs(r.cos))).ravel())
        for g, o in ((o32, r.outv), (i32, r.inv)):
            d = np.abs(g - o).ravel()
            vec_d.append(d)
            vec_ulp.append(d <= np.maximum(bf16_ulp(o), bf16_ulp(g)).ravel() * (1 + 1e-9))
        walk = greedy_walk(r.idx, r.logp, c32, 1.0, True)
        excused += compare_walk(r.logp, r.cos, walk.choice, 1.0)     # raises beyond TOL
        slots += w.slots - 1
    rel, d, ulp = np.concatenate(cos_rel), np.concatenate(vec_d), np.concatenate(vec_ulp)
    return {"cos_max": rel.max(), "cos_over": np.mean(rel > TOL), "vec_max": d.max(), "vec_mean": d.mean(),
            "vec_within_ulp": ulp.mean(), "excused": excused, "slots": slots}


# (workload, tier, blocks): one or two blocks of each real encoder shape
REAL_SHAPES = [("c32", 0, [0, 1]), ("c256_k16", 0, [0, 1]), ("entropy_k32", 0, [0])]


def test_float32_drift_at_real_shapes_needs_and_fits_the_bars():
    stats = {f"{n}/{t}": _drift(n, t, b) for n, t, b in REAL_SHAPES}
    for k, st in stats.items():
        # the derived bars hold the float32 build with a margin of about two
        assert st["cos_max"] <= COS_MAX / 1.5, (k, st)
        assert st["cos_over"] <= (1 - COS_FRACTION) / 2, (k, st)
        assert st["vec_max"] <= VEC_MAX / 2, (k, st)
        assert st["vec_mean"] <= VEC_MEAN / 2, (k, st)
        assert st["vec_within_ulp"] >= VEC_ULP_FRACTION + 0.05, (k, st)
        # bit-equal-or-one-ulp vectors are out of reach for any float32 build
        assert st["vec_within_ulp"] < 0.95, (k, st)
        assert len(st["excused"]) <= max(1, st["slots"] // 100), (k, st)
    # and an elementwise 1e-3 bar on every cosine fails at a real shape
    assert max(st["cos_max"] for st in stats.values()) > TOL, stats


def test_float32_drift_rate_of_the_wide_odd_shape():
    """The wide odd shape (H = 2560, 15 slots, K = 7) drifts more: the float32
    build misses 1e-3 on more than 0.1 % of its cosines (the bar of the main
    workloads), still inside COS_MAX; its GPU case uses fraction 0.995."""
    st = _drift("odd_h2560", 0, [0, 1])
    assert 0.001 < st["cos_over"] < 0.005, st
    assert st["cos_max"] <= COS_MAX / 1.5, st
    assert st["vec_max"] <= VEC_MAX / 2 and st["vec_mean"] <= VEC_MEAN / 2, st
