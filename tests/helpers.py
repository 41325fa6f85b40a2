"""Shared helpers of the GPU parity tests: tolerances, conversions, the
walk comparison with documented score-gap excuses, and cached weights."""
from __future__ import annotations

import numpy as np

import synth
from oracle.bf16 import bf16_bits_to_f64
from oracle.weights import Dims, OracleWeights
from oracle.walk import step_scores

# Relative tolerance on float32 scores: |gpu - oracle| <= TOL * max(1, |oracle|).
# The log-partition and log-probabilities meet it for every element.
TOL = 1e-3
# Pair cosines and committed step scores come out of two bf16 transformer
# layers. Against a float64 oracle, any float32-accumulating implementation of
# the same rounding points drifts by a bf16 rounding cascade (reproduced on the
# CPU by tests/test_tolerance_derivation.py), so for them TOL is required of
# at least COS_FRACTION of the elements, and every element must stay within
# COS_HARD: both operands are unit vectors stored in bf16; if every component
# of each disagrees by one rounding (at most 2^-8 relative), the dot product
# moves by at most 2 * 2^-8 * sum|o_d||i_d| <= 2^-7.
COS_FRACTION = 0.999
COS_HARD = 2.0 ** -7


def within(g, o, tol=TOL):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    return np.abs(g - o) <= tol * np.maximum(1.0, np.abs(o))


def assert_within(g, o, tol=TOL, what=""):
    ok = within(g, o, tol)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        g = np.asarray(g)
        o = np.asarray(o)
        raise AssertionError(f"{what}: {(~ok).sum()} outside tol {tol}; first {bad.tolist()}: "
                             f"gpu {[float(g[tuple(b)]) for b in bad]} oracle {[float(o[tuple(b)]) for b in bad]}")


def assert_scores(g, o, what="", alpha=1.0, fraction=COS_FRACTION, step=False):
    """Cosines / step scores: a fraction (COS_FRACTION unless a case states its
    own, derived from the float32 drift of its shape) within TOL, all within the
    bf16 bound. A step score fl32(logp + fl32(alpha * cos)) carries |alpha| times
    its cosine's error, so for step=True the TOL part is scaled by max(1, |alpha|)."""
    g = np.asarray(g, dtype=np.float64).ravel()
    o = np.asarray(o, dtype=np.float64).ravel()
    err = np.abs(g - o)
    tol = TOL * (max(1.0, abs(alpha)) if step else 1.0)
    hard = tol * np.maximum(1.0, np.abs(o)) + abs(alpha) * COS_HARD
    assert np.all(err <= hard), f"{what}: max error {err.max()} beyond the bf16 bound"
    n_bad = int((~within(g, o, tol)).sum())
    allowed = max(1, int((1.0 - fraction) * err.size))
    assert n_bad <= allowed, f"{what}: {n_bad} of {err.size} outside {TOL} (allowed {allowed})"
    return {"n": int(err.size), "over_tol": n_bad, "max": float(err.max()),
            "p999": float(np.percentile(err, 99.9)) if err.size else 0.0}


def bf16_to_f64(t) -> np.ndarray:
    """torch bfloat16 tensor -> float64 numpy of the same values."""
    import torch
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return bf16_bits_to_f64(bits)


def to_device(arr: np.ndarray, device="cuda"):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def f64_to_bf16_device(x: np.ndarray, device="cuda"):
    from oracle.bf16 import f64_to_bf16_bits
    return to_device(f64_to_bf16_bits(x), device)


def oracle_step_scores(logp, cos, choice, alpha, use_logp=True):
    """Oracle scores of the committed candidates along a given path (slots 1..B-1)."""
    return np.array([step_scores(logp[s], cos[s - 1][choice[s - 1]], alpha, use_logp)[choice[s]]
                     for s in range(1, logp.shape[0])], dtype=np.float64)


def compare_walk(logp, cos, gpu_choice, alpha, use_logp=True, tol=TOL):
    """Check a GPU path against the oracle's scores slot by slot.

    A GPU pick that differs from the oracle's argmax is excused only when the
    oracle's score of the GPU pick is within the score tolerance of the best
    score (tol * max(1, |best|) + |alpha| * COS_HARD, the bound the step scores
    are held to); the oracle walk then follows the GPU's pick. Returns the list
    of excused (slot, gap) pairs; raises on a real mismatch.
    """
    B, K = logp.shape
    excused = []
    assert gpu_choice[0] == 0
    for s in range(1, B):
        z = step_scores(logp[s], cos[s - 1][gpu_choice[s - 1]], alpha, use_logp).astype(np.float64)
        best = z.max()
        pick = int(gpu_choice[s])
        if pick != int(np.argmax(z)):
            gap = best - z[pick]
            if gap > tol * max(1.0, abs(best)) + abs(alpha) * COS_HARD:
                raise AssertionError(f"slot {s}: gpu picked {pick} (z={z[pick]}), oracle best "
                                     f"{int(np.argmax(z))} (z={best}), gap {gap}")
            excused.append((s, float(gap)))
    return excused


_WEIGHTS = {}


def oracle_weights(w: synth.Workload) -> OracleWeights:
    key = (w.hidden, w.heads, w.ffn, w.d_e, w.vocab, w.target_hidden, w.drafter_hidden)
    if key not in _WEIGHTS:
        _WEIGHTS[key] = OracleWeights(Dims(w.hidden, w.heads, w.ffn, w.d_e, target_hidden=w.target_hidden,
                                           drafter_hidden=w.drafter_hidden), w.vocab, synth.WEIGHTS_SEED)
    return _WEIGHTS[key]


_DEV_WEIGHTS = {}


def device_weights(w: synth.Workload):
    import draft_block_candidate_amd as L
    key = (w.hidden, w.heads, w.ffn, w.d_e, w.vocab, w.target_hidden, w.drafter_hidden)
    if key not in _DEV_WEIGHTS:
        _DEV_WEIGHTS.clear()   # keep one blob resident at a time
        _DEV_WEIGHTS[key] = L.Weights(L.EncoderDims(w.hidden, w.heads, w.ffn, w.d_e,
                                                    target_hidden=w.target_hidden,
                                                    drafter_hidden=w.drafter_hidden), w.vocab,
                                      synth.WEIGHTS_SEED)
    return _DEV_WEIGHTS[key]
