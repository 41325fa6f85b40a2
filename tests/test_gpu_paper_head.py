"""Parity of the paper's own head against the oracle (GPU).

The head (LiLiCorr paper, Section 3.2 and Appendix A) takes the drafter's hidden
state per slot and the target state per block besides the logits; the
paper's configuration (Table 4: width 1024, 8 heads, FFN 2048, d_e 1024, the
sigma * cos rule with sigma = 8) runs at its full size with Qwen3-8B widths
(4096) for the drafter and target states, and on a small twin the oracle
checks block by block (every block of the 32-block case). The bars are those
of the lattice head (tests/helpers.py, tests/test_gpu_rerank.py): top-K ids
exactly; lse and logp within 1e-3; cosines within 1e-3 on 99.9 % of the
elements and all within 2e-3 (step scores sigma times that); in/out vectors
within 2^-8 per component; committed tokens exactly unless the oracle's score
gap of the GPU's pick is within the step tolerance, on at most 1 % of slots.
Weights: every tensor of the head, sampled elements bit-exact against the
oracle's generator.
"""
import numpy as np
import pytest

from helpers import (assert_within, assert_scores, assert_vectors, assert_excuse_cap, record, bf16_to_f64,
                     to_device, oracle_weights, device_weights, compare_walk, oracle_step_scores, COS_FRACTION)
import synth
import oracle
from oracle.weights import Dims, weight_table

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import torch
    import draft_block_candidate_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.lib()
    return lib


@pytest.mark.parametrize("name", ["paper_tiny", "paper_qwen3_8b"])
def test_paper_weights_bit_exact(L, name):
    import torch
    w = synth.WORKLOADS[name]
    dw = device_weights(w)
    ow = oracle_weights(w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    d = Dims(w.hidden, w.heads, w.ffn, w.d_e, target_hidden=w.target_hidden, drafter_hidden=w.drafter_hidden)
    for t, tname, shape, scale, kind in weight_table(d, w.vocab):
        n = int(np.prod(shape))
        elems = np.arange(n) if n <= 70000 else np.unique(rng.integers(0, n, 20000))
        dev = dw.tensor(t)[torch.from_numpy(elems).cuda()]
        got = bf16_to_f64(dev) if dev.dtype == torch.bfloat16 else dev.double().cpu().numpy()
        assert np.array_equal(got, ow.tensor_elements(tname, elems.astype(np.uint64))), tname


CASES = [("paper_tiny", None, "greedy"), ("paper_qwen3_8b", None, "greedy"),
         ("paper_c32", None, "greedy"), ("paper_tiny", None, "exact")]


@pytest.mark.parametrize("name,sample,rule", CASES)
def test_paper_head_matches_oracle(L, name, sample, rule):
    import torch
    w = synth.WORKLOADS[name]
    host = synth.make_logits(w)
    hid_bits, tgt_bits = synth.make_head_inputs(w)
    print(f"[case] paper head {name} rule {rule} blocks {w.num_blocks}", flush=True)
    tokens, dbg = L.rerank(to_device(host), w.topk, device_weights(w), w.alpha, w.use_logp, debug=True,
                           rule=rule, hidden=to_device(hid_bits), target=to_device(tgt_bits))
    torch.cuda.synchronize()
    ow = oracle_weights(w)
    hidden = synth.bf16_bits_to_f32(hid_bits).astype(np.float64)
    target = synth.bf16_bits_to_f32(tgt_bits).astype(np.float64)
    g_cos, o_cos, g_z, o_z, excused, g_vec, o_vec = [], [], [], [], [], [], []
    blocks = list(range(w.num_blocks) if sample is None else sample)
    for b in blocks:
        r = oracle.rerank_block(host[b], w.topk, ow, w.alpha, w.use_logp, rule=rule, hidden=hidden[b],
                                target=target[b])
        gidx = dbg["topk_idx"][b].cpu().numpy()
        assert np.array_equal(gidx, r.idx), f"block {b}: top-K ids"
        assert_within(dbg["lse"][b].cpu().numpy(), r.lse, what=f"block {b} lse")
        assert_within(dbg["topk_logp"][b].cpu().numpy(), r.logp, what=f"block {b} logp")
        go, gi = bf16_to_f64(dbg["outv"][b]), bf16_to_f64(dbg["inv"][b])
        g_vec += [go.ravel(), gi.ravel()]
        o_vec += [r.outv.ravel(), r.inv.ravel()]
        assert np.all(gi[0] == 0) and np.all(go[0] == go[0][0]), "anchor rows"
        gtok = tokens[b].cpu().numpy()
        choice = np.array([int(np.nonzero(gidx[s] == gtok[s])[0][0]) for s in range(w.slots)])
        g_cos.append(dbg["cos"][b].cpu().numpy())
        o_cos.append(r.cos)
        g_z.append(dbg["score"][b].cpu().numpy()[1:])
        o_z.append(oracle_step_scores(r.logp, r.cos, choice, w.alpha, w.use_logp))
        if rule == "greedy":
            ex = compare_walk(r.logp, r.cos, choice, w.alpha, w.use_logp)
            excused += [(b,) + e for e in ex]
            if not ex:
                assert np.array_equal(gtok, r.tokens.astype(np.int32)), f"block {b}: tokens"
        else:
            from oracle.paths import path_total
            dz = abs(w.alpha) * np.abs(g_cos[-1].astype(np.float64) - r.cos).reshape(w.slots - 1, -1).max(axis=1)
            bound = 2.0 * float(dz.sum()) + w.slots * 2.0 ** -20 * max(1.0, abs(float(r.exact.total)))
            gap = float(r.exact.total) - float(path_total(r.logp, r.cos, choice, w.alpha, w.use_logp))
            assert gap <= bound, f"block {b}: exact path total gap {gap} > {bound}"
    sc = assert_scores(np.concatenate([c.ravel() for c in g_cos]), np.concatenate([c.ravel() for c in o_cos]),
                       f"{name} cos", 1.0, COS_FRACTION)
    sz = assert_scores(np.concatenate(g_z), np.concatenate(o_z), f"{name} step scores", w.alpha, COS_FRACTION, step=True)
    vec = assert_vectors(np.concatenate(g_vec), np.concatenate(o_vec), f"{name} in/out vectors")
    n_slots = len(blocks) * (w.slots - 1)
    record(f"paper/{name}/{rule}", blocks=len(blocks), slots=n_slots, excused=excused, cos=sc, step=sz, vectors=vec)
    assert_excuse_cap(excused, n_slots, name)


def test_paper_head_errors_without_inputs(L):
    w = synth.WORKLOADS["paper_tiny"]
    host = synth.make_logits(w)
    with pytest.raises(L.LilicorrError) as e:
        L.rerank(to_device(host), w.topk, device_weights(w), w.alpha, w.use_logp)
    assert e.value.code == L.EINVAL


@pytest.mark.parametrize("B,K,N,de", [(2, 1, 3, 64), (2, 5, 2, 64), (3, 7, 4, 64), (17, 3, 2, 64),
                                      (5, 3, 2, 544)])
def test_paper_head_degenerate_and_ragged(L, B, K, N, de):
    # one drafted slot (B = 2), one candidate (K = 1), odd lattices, a ragged
    # slot count, and wide vectors in ragged 256-wide slices (d_e = 544)
    import torch
    w = synth.Workload(f"paper_edge_{B}_{K}_{N}_{de}", N, B, 4096, K, 128, 2, 128, de, "f32", "normal",
                       alpha=8.0, use_logp=False, target_hidden=192, drafter_hidden=128)
    rng = np.random.default_rng(B * 100 + K * 10 + N)
    host = rng.standard_normal((N, B, w.vocab), dtype=np.float32)
    hid_bits = synth.f32_to_bf16_bits_rne(rng.standard_normal((N, B, 128), dtype=np.float32))
    tgt_bits = synth.f32_to_bf16_bits_rne(rng.standard_normal((N, 192), dtype=np.float32))
    print(f"[case] paper head edge B {B} K {K} N {N} d_e {de}", flush=True)
    tokens, dbg = L.rerank(to_device(host), K, device_weights(w), w.alpha, w.use_logp, debug=True,
                           hidden=to_device(hid_bits), target=to_device(tgt_bits))
    torch.cuda.synchronize()
    ow = oracle_weights(w)
    hidden = synth.bf16_bits_to_f32(hid_bits).astype(np.float64)
    target = synth.bf16_bits_to_f32(tgt_bits).astype(np.float64)
    excused, g_vec, o_vec = [], [], []
    for b in range(N):
        r = oracle.rerank_block(host[b], K, ow, w.alpha, w.use_logp, hidden=hidden[b], target=target[b])
        gidx = dbg["topk_idx"][b].cpu().numpy()
        assert np.array_equal(gidx, r.idx), f"block {b}: top-K ids"
        g_vec += [bf16_to_f64(dbg["outv"][b]).ravel(), bf16_to_f64(dbg["inv"][b]).ravel()]
        o_vec += [r.outv.ravel(), r.inv.ravel()]
        assert_scores(dbg["cos"][b].cpu().numpy(), r.cos, f"edge block {b} cos", 1.0, COS_FRACTION)
        gtok = tokens[b].cpu().numpy()
        choice = np.array([int(np.nonzero(gidx[s] == gtok[s])[0][0]) for s in range(B)])
        ex = compare_walk(r.logp, r.cos, choice, w.alpha, w.use_logp)
        excused += [(b,) + e for e in ex]
        if not ex:
            assert np.array_equal(gtok, r.tokens.astype(np.int32)), f"block {b}: tokens"
    vec = assert_vectors(np.concatenate(g_vec), np.concatenate(o_vec), f"edge {B}x{K} in/out vectors")
    record(f"paper/edge/B{B}/K{K}/N{N}/de{de}", blocks=N, slots=N * (B - 1), excused=excused, vectors=vec)
    assert_excuse_cap(excused, N * (B - 1), f"edge {B}x{K}")
