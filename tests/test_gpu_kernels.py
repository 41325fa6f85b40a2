"""Per-kernel parity of the HIP library against the oracle (GPU).

Every call goes through the C ABI (the ctypes binding). Inputs are seeded;
expected values come from the oracle only.
"""
import numpy as np
import pytest

from helpers import (assert_within, bf16_to_f64, to_device, f64_to_bf16_device, oracle_weights,
                     device_weights, TOL)
import synth
from oracle.bf16 import round_bf16
from oracle.topk_lse import topk_lse as oracle_topk
from oracle.weights import Dims, OracleWeights, weight_table
from oracle import encoder as oenc
from oracle.scores import pair_scores as oracle_pair_scores
from oracle.walk import greedy_walk as oracle_walk

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


# ---------------------------------------------------------------- weights

@pytest.mark.parametrize("name", ["tiny", "c1_qwen3_8b"])
def test_weights_bit_exact(L, name):
    import torch
    w = synth.WORKLOADS[name]
    dw = device_weights(w)
    ow = oracle_weights(w)
    _sync()
    rng = np.random.default_rng(0)
    for t, tname, shape, scale, kind in weight_table(Dims(w.hidden, w.heads, w.ffn, w.d_e), w.vocab):
        n = int(np.prod(shape))
        elems = np.arange(n) if n <= 70000 else np.unique(rng.integers(0, n, 20000))
        dev = dw.tensor(t)
        got = dev.double().cpu().numpy()[elems] if dev.dtype != torch.bfloat16 else bf16_to_f64(dev)[elems]
        expect = ow.tensor_elements(tname, elems.astype(np.uint64))
        assert np.array_equal(got, expect), tname


# ---------------------------------------------------------------- top-K + lse

def _check_topk(L, host, K):
    rows = host.reshape(-1, host.shape[-1])
    idx, logp, lse = L.topk_lse(to_device(rows), K)
    _sync()
    oi, ol, olse = oracle_topk(rows, K)
    assert np.array_equal(idx.cpu().numpy(), oi), "top-K ids differ"
    assert_within(lse.cpu().numpy(), olse, what="lse")
    assert_within(logp.cpu().numpy(), ol, what="logp")


@pytest.mark.parametrize("V", [4, 7, 8, 9, 63, 1023, 1024, 1025, 4095, 4096, 4097, 8193, 151936, 151937])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_topk_shape_zoo(L, V, dtype):
    for K in (1, 4, 8, 16, 32, 64):
        if K > V:
            continue
        rows = 5 if V > 100000 else 24
        host = synth.make_random_logits(rows, V, dtype, seed=V * 7 + K, scale=0.5 if dtype == "bf16" else 1.0)
        _check_topk(L, host, K)


@pytest.mark.parametrize("rows", [1, 3, 64, 700])
def test_topk_row_counts_change_chunking(L, rows):
    host = synth.make_random_logits(rows, 151936, "bf16", seed=rows)
    _check_topk(L, host, 16)


@pytest.mark.parametrize("V", [5000, 40000])     # one chunk per row, several chunks per row
def test_topk_crafted_rows(L, V):
    rows = []
    rows.append(np.full(V, 0.75, dtype=np.float32))                       # constant
    z = np.zeros(V, dtype=np.float32)
    z[::2] = -0.0                                                           # +-0 mixed
    rows.append(z)
    rows.append(np.arange(V, dtype=np.float32) / V)                         # ascending: every element a new max
    rows.append(-np.arange(V, dtype=np.float32) / V)                        # descending
    r = np.random.default_rng(1).integers(-2, 3, V).astype(np.float32)     # heavy ties
    rows.append(r)
    last = np.zeros(V, dtype=np.float32)
    last[-1] = 5.0
    rows.append(last)
    big = np.random.default_rng(2).standard_normal(V).astype(np.float32) * 40 + 300  # large magnitudes
    rows.append(big)
    host = np.stack(rows)
    for K in (1, 8, 33, 64):
        _check_topk(L, host, K)
        _check_topk(L, synth.f32_to_bf16_bits_rne(host), K)


def test_topk_entropy_tiers(L):
    w = synth.WORKLOADS["entropy_k32"]
    for tier in range(3):
        host = synth.make_logits(w, tier, num_blocks=2)
        _check_topk(L, host, 32)


# ---------------------------------------------------------------- linear

def _rand_bf16(rng, shape, scale=1.0):
    return round_bf16(rng.standard_normal(shape) * scale)


@pytest.mark.parametrize("M,Kd,N", [(64, 64, 32), (100, 256, 96), (128, 1024, 3072), (300, 1024, 1024),
                                    (100, 1024, 2100), (128, 2048, 2048),
                                    (2100, 512, 200), (4096, 1024, 4096), (128, 4096, 1024),
                                    (8192, 1024, 4096), (33000, 256, 1000), (6000, 192, 640),
                                    (64, 1024, 256), (50, 512, 1000), (128, 768, 4096), (7, 256, 48), (1, 4096, 1024), (1, 1024, 1024), (16, 4096, 1024),
                                    (4096, 512, 3072), (5000, 256, 2500), (4096, 4096, 1024), (3840, 3072, 1024),
                                    (100, 1024, 3000), (65, 2048, 2080), (120, 1024, 4096)])
@pytest.mark.parametrize("epi", [0, 1, 2, 3])
def test_linear(L, M, Kd, N, epi):
    import torch
    rng = np.random.default_rng(M + Kd + N + epi)
    A = _rand_bf16(rng, (M, Kd))
    W = _rand_bf16(rng, (N, Kd), 1 / np.sqrt(Kd))
    b = rng.standard_normal(N).astype(np.float32).astype(np.float64) * 0.1
    y = A @ W.T + b
    resid = rng.standard_normal((M, N)).astype(np.float32)
    res_dev = to_device(resid) if epi == 3 else None
    out = L.linear(f64_to_bf16_device(A), f64_to_bf16_device(W), to_device(b.astype(np.float32)), epi, res_dev)
    _sync()
    if epi == 0:
        assert_within(out.cpu().numpy(), y, what="linear f32")
    elif epi == 3:
        assert_within(out.cpu().numpy(), resid.astype(np.float64) + y, what="linear resid")
    else:
        ref = y if epi == 1 else oenc.silu(y)
        got = bf16_to_f64(out)
        # one bf16 rounding of a value that agrees to ~1e-6: equal or one ulp apart
        ulp = np.maximum(np.abs(ref), 1e-30) * 2.0 ** -7
        assert np.all(np.abs(got - ref) <= ulp + 1e-6)
        assert np.mean(got == round_bf16(ref)) > 0.99


# ---------------------------------------------------------------- rmsnorm

@pytest.mark.parametrize("M,H", [(1, 64), (5, 1024), (100, 2048), (33, 192)])
def test_rmsnorm(L, M, H):
    rng = np.random.default_rng(M * H)
    x = (rng.standard_normal((M, H)) * 3).astype(np.float32)
    g = rng.uniform(0.75, 1.25, H).astype(np.float32)
    out = L.rmsnorm(to_device(x), to_device(g), 1e-6)
    _sync()
    ref = oenc.rmsnorm(x.astype(np.float64), g.astype(np.float64))
    got = bf16_to_f64(out)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-6)
    assert np.mean(got == round_bf16(ref)) > 0.99


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("N,B,K,heads,dh", [(1, 16, 4, 2, 32), (2, 16, 8, 8, 128), (1, 16, 16, 8, 128),
                                            (1, 16, 32, 16, 128), (3, 5, 3, 2, 64), (1, 1, 1, 1, 32),
                                            (2, 7, 9, 4, 32), (1, 64, 8, 2, 64), (2, 25, 8, 4, 64),
                                            (3, 10, 13, 2, 128), (2, 20, 15, 2, 32), (1, 17, 16, 4, 128),
                                            (2, 33, 9, 2, 64),
                                            # K a multiple of 16 (wave-uniform slots) at each d_h, both
                                            # kernels; two-pass with a part-full second round
                                            (1, 8, 16, 2, 64), (1, 12, 16, 4, 32), (1, 12, 8, 2, 64),
                                            (1, 9, 32, 4, 64), (2, 24, 16, 2, 32),
                                            # 129-256 tokens at d_h = 128: two workgroups per
                                            # (head, block) with K and V in turn; part-full tile
                                            # rounds, K a multiple of 4 but not 16, and a
                                            # (head, block) count that leaves the last group of
                                            # eight pairs part-full
                                            (3, 12, 16, 3, 128), (2, 20, 12, 2, 128), (2, 9, 16, 2, 128),
                                            (1, 11, 20, 5, 128)])
def test_lattice_attention(L, N, B, K, heads, dh):
    rng = np.random.default_rng(N * 1000 + B * 10 + K)
    H = heads * dh
    T = B * K
    qkv = _rand_bf16(rng, (N * T, 3 * H))
    dist = (rng.uniform(-0.5, 0.5, (heads, 127))).astype(np.float32)
    same = rng.uniform(-0.5, 0.5, heads).astype(np.float32)
    out = L.lattice_attention(f64_to_bf16_device(qkv), N, B, K, H, heads, to_device(dist), to_device(same))
    _sync()
    got = bf16_to_f64(out)
    slot = np.repeat(np.arange(B), K)
    for n in range(N):
        ref = oenc.lattice_attention(qkv[n * T:(n + 1) * T], slot, heads, dist.astype(np.float64),
                                     same.astype(np.float64))
        g = got[n * T:(n + 1) * T]
        # p and o are bf16-rounded; fp32 vs fp64 scores may flip a rounding
        assert np.all(np.abs(g - ref) <= 2.0 ** -6 * np.abs(ref) + 2e-3), (n, np.abs(g - ref).max())


# ---------------------------------------------------------------- pair scores

def _unit_bf16(rng, shape):
    v = rng.standard_normal(shape)
    return round_bf16(v / np.linalg.norm(v, axis=-1, keepdims=True))


@pytest.mark.parametrize("N,B,K,de", [(1, 16, 4, 32), (2, 16, 8, 128), (1, 16, 16, 128), (1, 16, 32, 256),
                                      (2, 3, 5, 64), (1, 2, 64, 32), (3, 64, 8, 96)])
def test_pair_scores(L, N, B, K, de):
    rng = np.random.default_rng(N + B + K + de)
    outv = _unit_bf16(rng, (N, B, K, de))
    inv = _unit_bf16(rng, (N, B, K, de))
    cos = L.pair_scores(f64_to_bf16_device(outv), f64_to_bf16_device(inv))
    _sync()
    got = cos.cpu().numpy()
    for n in range(N):
        assert_within(got[n], oracle_pair_scores(outv[n], inv[n]), tol=1e-5, what="cos")


# ---------------------------------------------------------------- greedy walk

@pytest.mark.parametrize("B,K", [(1, 4), (2, 1), (16, 3), (16, 8), (16, 32), (8, 64), (15, 7), (16, 33), (64, 64), (5, 16)])
# alpha = 0.7 is not a power of two: alpha * cos is rounded before the sum
# (an FMA would round once and change the scores)
@pytest.mark.parametrize("alpha,use_logp", [(1.0, True), (0.0, True), (0.5, True), (0.7, True), (8.0, False)])
@pytest.mark.parametrize("coarse", [False, True])
def test_greedy_walk_bit_exact(L, B, K, alpha, use_logp, coarse):
    import torch
    rng = np.random.default_rng(B * 131 + K + int(alpha * 10) + coarse)
    N = 6
    if coarse:
        logp = rng.choice([-1.0, -0.5, 0.0], size=(N, B, K)).astype(np.float32)
        cos = rng.choice([-0.5, 0.0, 0.5], size=(N, max(B - 1, 1), K, K)).astype(np.float32)
    else:
        logp = -np.abs(rng.standard_normal((N, B, K))).astype(np.float32)
        cos = rng.uniform(-1, 1, size=(N, max(B - 1, 1), K, K)).astype(np.float32)
    idx = rng.integers(0, 151936, size=(N, B, K)).astype(np.int32)
    tok, score, gap = L.greedy_walk(to_device(idx), to_device(logp), to_device(cos), alpha, use_logp)
    _sync()
    for n in range(N):
        r = oracle_walk(idx[n], logp[n], cos[n], alpha, use_logp)
        assert np.array_equal(tok[n].cpu().numpy(), r.tokens.astype(np.int32))
        assert np.array_equal(score[n].cpu().numpy(), r.score)
        assert np.array_equal(gap[n].cpu().numpy(), r.gap)


@pytest.mark.parametrize("M,Kd,N", [(128, 1024, 3072), (128, 4096, 1024), (64, 256, 512)])
def test_linear_split_k_is_bit_reproducible(L, M, Kd, N):
    import torch
    rng = np.random.default_rng(M * 7 + N)
    A = f64_to_bf16_device(_rand_bf16(rng, (M, Kd)))
    W = f64_to_bf16_device(_rand_bf16(rng, (N, Kd), 1 / np.sqrt(Kd)))
    b = to_device(rng.standard_normal(N).astype(np.float32))
    outs = [L.linear(A, W, b, L.EPI_F32) for _ in range(3)]
    _sync()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
