"""Parity of the exact best path and the sampled commit against the oracle (GPU).

Stand-alone entry points (lilicorr_best_path, lilicorr_sample_path) run the
rerank path's fused commit kernel on seeded scores that both sides receive:
  * exact path: tokens and per-slot scores bit-exact (same float32 operations,
    same tie rule), also on coarse inputs full of exact ties;
  * sampled commit: greedy rows (T <= 0) bit-exact with the greedy walk and
    one-hot proposals; drawn rows follow the oracle's inverse-CDF draw, except
    where the input uniform lies within 1e-5 of a cumulative boundary (float32
    exponentials and sums against float64; each excused slot is reported), and
    proposals within 1e-5 absolute.
Through lilicorr_rerank (rule = exact / sample) the GPU's cosines differ from
the oracle's by the bf16 cascade measured in test_gpu_rerank.py, so:
  * exact path: the oracle's total of the GPU's path must be within
    2 * sum_s |alpha| * max|cos_gpu - cos_oracle| (+ float32 slack) of the
    oracle's best total (any two paths' totals move by at most half of that);
    otherwise the paths must be identical;
  * sampled commit: along the GPU's path, each proposal row within the bound
    that the same cosine difference puts on softmax(z / T), and each draw the
    oracle's unless u lies within that bound of a cumulative boundary.
"""
import numpy as np
import pytest

from helpers import to_device, oracle_weights, device_weights, assert_within
import synth
import oracle
from oracle.paths import best_path as o_best_path, sample_path as o_sample_path, path_total, softmax_t
from oracle.walk import greedy_walk as o_greedy_walk, step_scores

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import torch
    import draft_block_candidate_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.lib()
    return lib


def _sync():
    import torch
    torch.cuda.synchronize()


def _lattice(rng, N, B, K, coarse):
    if coarse:
        logp = rng.choice([-1.0, -0.5, 0.0], size=(N, B, K)).astype(np.float32)
        cos = rng.choice([-0.5, 0.0, 0.5], size=(N, max(B - 1, 1), K, K)).astype(np.float32)
    else:
        logp = -np.abs(rng.standard_normal((N, B, K))).astype(np.float32)
        cos = rng.uniform(-1, 1, size=(N, max(B - 1, 1), K, K)).astype(np.float32)
    # distinct ids within a slot, so a token names its candidate
    idx = (rng.integers(0, 151936 - 64, size=(N, B, 1)) + np.arange(K)).astype(np.int32)
    return idx, logp, cos


SHAPES = [(1, 4), (2, 1), (2, 5), (16, 3), (16, 8), (16, 32), (8, 64), (64, 8), (5, 16), (15, 7)]


@pytest.mark.parametrize("B,K", SHAPES)
@pytest.mark.parametrize("alpha,use_logp", [(1.0, True), (0.5, True), (0.7, True), (8.0, False)])
@pytest.mark.parametrize("coarse", [False, True])
def test_best_path_bit_exact(L, B, K, alpha, use_logp, coarse):
    rng = np.random.default_rng(B * 977 + K * 13 + int(alpha * 10) + coarse)
    N = 5
    idx, logp, cos = _lattice(rng, N, B, K, coarse)
    print(f"[case] best_path B {B} K {K} alpha {alpha} use_logp {use_logp} coarse {coarse}", flush=True)
    tok, score = L.best_path(to_device(idx), to_device(logp), to_device(cos), alpha, use_logp)
    _sync()
    for n in range(N):
        r = o_best_path(idx[n], logp[n], cos[n], alpha, use_logp)
        assert np.array_equal(tok[n].cpu().numpy(), r.tokens.astype(np.int32)), f"block {n}"
        assert np.array_equal(score[n].cpu().numpy(), r.score), f"block {n}"


def _check_sample_block(gidx_choice, gprop, r_logp, r_cos, idx, T, u, alpha, use_logp, zbound=None):
    """Walk the GPU's path; at each slot compare the proposal row and the draw
    with the oracle's for the same previous candidate. zbound[s] bounds the
    score difference of slot s (None: identical scores). Returns excused slots."""
    B, K = r_logp.shape
    excused = []
    choice = gidx_choice
    assert choice[0] == 0
    assert np.array_equal(gprop[0], np.eye(K)[0])
    for s in range(1, B):
        z = step_scores(r_logp[s], r_cos[s - 1][choice[s - 1]], alpha, use_logp)
        q = softmax_t(z, T)
        c = np.cumsum(q)
        if zbound is None:
            qb = np.full(K, 1e-5)
        else:
            qb = 2.0 * zbound[s] / T * q + 1e-5      # |d q_j| <= q_j * 2 max|dz| / T
        assert np.all(np.abs(gprop[s] - q) <= qb), f"slot {s}: proposal {gprop[s]} vs {q}"
        expect = min(int(np.sum(c <= float(u[s]))), K - 1)
        if choice[s] != expect:
            edge = np.min(np.abs(c - float(u[s])))
            band = 1e-5 if zbound is None else float(qb.sum())
            assert edge <= band, f"slot {s}: drew {choice[s]}, oracle {expect}, u {u[s]} cdf {c}"
            excused.append((s, float(edge)))
    return excused


@pytest.mark.parametrize("B,K", SHAPES)
@pytest.mark.parametrize("alpha,use_logp", [(1.0, True), (1.3, True), (8.0, False)])
@pytest.mark.parametrize("coarse", [False, True])
def test_sample_path(L, B, K, alpha, use_logp, coarse):
    rng = np.random.default_rng(B * 1009 + K * 17 + int(alpha) + coarse)
    N = 8
    idx, logp, cos = _lattice(rng, N, B, K, coarse)
    temps = synth.make_temperatures(N, seed=B * 31 + K)
    u = synth.make_uniforms(N, B, seed=B * 37 + K)
    print(f"[case] sample_path B {B} K {K} alpha {alpha} coarse {coarse}", flush=True)
    tok, prop, score = L.sample_path(to_device(idx), to_device(logp), to_device(cos), to_device(temps),
                                     to_device(u), alpha, use_logp)
    gtok, gsc, _ = L.greedy_walk(to_device(idx), to_device(logp), to_device(cos), alpha, use_logp)
    _sync()
    tok, prop, score = tok.cpu().numpy(), prop.cpu().numpy(), score.cpu().numpy()
    gtok, gsc = gtok.cpu().numpy(), gsc.cpu().numpy()
    excused = []
    for n in range(N):
        if temps[n] <= 0:
            r = o_greedy_walk(idx[n], logp[n], cos[n], alpha, use_logp)
            assert np.array_equal(tok[n], r.tokens.astype(np.int32)), f"greedy row {n}"
            assert np.array_equal(tok[n], gtok[n]) and np.array_equal(score[n], gsc[n]), f"greedy row {n}"
            assert np.array_equal(prop[n], np.eye(K, dtype=np.float32)[r.choice])
            continue
        choice = (tok[n] - idx[n][:, 0]).astype(np.int64)
        ex = _check_sample_block(choice, prop[n], logp[n], cos[n], idx[n], float(temps[n]), u[n],
                                 alpha, use_logp)
        excused += [(n,) + e for e in ex]
        z_path = [step_scores(logp[n][s], cos[n][s - 1][choice[s - 1]], alpha, use_logp)[choice[s]]
                  for s in range(1, B)]
        assert np.array_equal(score[n][1:], np.array(z_path, dtype=np.float32)), f"block {n} scores"
        if not ex:
            r = o_sample_path(idx[n], logp[n], cos[n], float(temps[n]), u[n], alpha, use_logp)
            assert np.array_equal(tok[n], r.tokens.astype(np.int32)), f"block {n} tokens"
    if excused:
        print(f"[excused] sample_path B {B} K {K}: {excused}", flush=True)


# ------------------------------------------------------------ through rerank

PIPE = [("tiny", 0, None), ("c1_qwen3_8b", 0, None), ("c32", 0, [0, 5, 31]), ("c256_k16", 0, [7]),
        ("entropy_k32", 1, [3])]


def _pipeline(L, name, tier, rule, **kw):
    w = synth.WORKLOADS[name]
    host = synth.make_logits(w, tier)
    print(f"[case] rerank rule {rule} {name} tier {tier}", flush=True)
    dev = to_device(host)
    tokens, dbg = L.rerank(dev, w.topk, device_weights(w), w.alpha, debug=True, rule=rule, **kw)
    _sync()
    return w, host, tokens.cpu().numpy(), {k: v.cpu() for k, v in dbg.items()}


@pytest.mark.parametrize("name,tier,sample", PIPE)
def test_rerank_exact_rule(L, name, tier, sample):
    w, host, tokens, dbg = _pipeline(L, name, tier, "exact")
    ow = oracle_weights(w)
    for b in (range(w.num_blocks) if sample is None else sample):
        r = oracle.rerank_block(host[b], w.topk, ow, w.alpha, rule="exact")
        gidx = dbg["topk_idx"][b].numpy()
        assert np.array_equal(gidx, r.idx), f"block {b}: top-K ids"
        choice = np.array([int(np.nonzero(gidx[s] == tokens[b][s])[0][0]) for s in range(w.slots)])
        g_cos = dbg["cos"][b].numpy().astype(np.float64)
        dz = abs(w.alpha) * np.abs(g_cos - r.cos).reshape(w.slots - 1, -1).max(axis=1)
        bound = 2.0 * float(dz.sum()) + w.slots * 2.0 ** -20 * max(1.0, abs(float(r.exact.total)))
        g_total = float(path_total(r.logp, r.cos, choice, w.alpha))
        gap = float(r.exact.total) - g_total
        assert gap <= bound, f"block {b}: GPU path total {g_total} vs best {r.exact.total} (bound {bound})"
        if not np.array_equal(tokens[b], r.exact.tokens.astype(np.int32)):
            print(f"[excused] exact {name} block {b}: total gap {gap:.3g} <= {bound:.3g}", flush=True)


@pytest.mark.parametrize("name,tier,sample", PIPE)
def test_rerank_sample_rule(L, name, tier, sample):
    import torch
    w = synth.WORKLOADS[name]
    temps = synth.make_temperatures(w.num_blocks, seed=w.logits_seed(tier) + 7)
    u = synth.make_uniforms(w.num_blocks, w.slots, seed=w.logits_seed(tier) + 11)
    prop = torch.empty((w.num_blocks, w.slots, w.topk), dtype=torch.float32, device="cuda")
    w, host, tokens, dbg = _pipeline(L, name, tier, "sample", temperature=to_device(temps),
                                     uniforms=to_device(u), proposal=prop)
    prop = prop.cpu().numpy()
    ow = oracle_weights(w)
    blocks = list(range(w.num_blocks) if sample is None else sample)
    if w.num_blocks > 1 and 1 not in blocks:
        blocks.append(1)          # block 0 is a greedy row; block 1 draws
    excused = []
    for b in blocks:
        r = oracle.rerank_block(host[b], w.topk, ow, w.alpha, rule="sample", temperature=float(temps[b]),
                                uniforms=u[b])
        gidx = dbg["topk_idx"][b].numpy()
        assert np.array_equal(gidx, r.idx), f"block {b}: top-K ids"
        choice = np.array([int(np.nonzero(gidx[s] == tokens[b][s])[0][0]) for s in range(w.slots)])
        g_cos = dbg["cos"][b].numpy().astype(np.float64)
        dz = np.concatenate([[0.0], abs(w.alpha) * np.abs(g_cos - r.cos).reshape(w.slots - 1, -1).max(axis=1)
                             + 2.0 ** -20])
        if temps[b] <= 0:
            from helpers import compare_walk
            ex = compare_walk(r.logp, r.cos, choice, w.alpha)
            assert np.array_equal(prop[b], np.eye(w.topk, dtype=np.float32)[choice])
        else:
            ex = _check_sample_block(choice, prop[b], r.logp, r.cos, gidx, float(temps[b]), u[b], w.alpha,
                                     True, zbound=dz)
        excused += [(b,) + tuple(e) for e in ex]
        if not ex:
            assert np.array_equal(tokens[b], r.tokens.astype(np.int32)), f"block {b}: tokens"
    if excused:
        print(f"[excused] sample {name}: {excused}", flush=True)
