"""Vocabulary-sharded top-K + log-partition on one GPU (simulated shards).

Each shard's slice is copied to its own contiguous [rows, V_shard] buffer, as a
tensor-parallel LM head leaves it on its GPU; lilicorr_topk_shard reduces it
and lilicorr_topk_merge combines the stacked shard outputs. Against the oracle
(the unsplit definition, pinned to the sharded decomposition on the CPU):
top-K ids exactly, lse and logp within 1e-3 * max(1, |oracle|). Ids must also
equal the unsharded kernel's for every row.
"""
import numpy as np
import pytest

from helpers import to_device, assert_within
import synth
from oracle.sharded import shard_bounds
from oracle.topk_lse import topk_lse_row

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import torch
    import draft_block_candidate_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.lib()
    return lib


def sharded(L, dev, K, G):
    import torch
    rows, V = dev.shape
    val = torch.empty((G, rows, K), dtype=torch.float32, device=dev.device)
    idx = torch.empty((G, rows, K), dtype=torch.int32, device=dev.device)
    ms = torch.empty((G, rows, 2), dtype=torch.float32, device=dev.device)
    slices = []
    for g, (lo, hi) in enumerate(shard_bounds(V, G)):
        sl = dev[:, lo:hi].contiguous()
        slices.append(sl)
        L.topk_shard(sl, K, lo, out=(val[g], idx[g], ms[g]))
    return L.topk_merge(val, idx, ms)


def _check(L, host, K, G, sample_rows=None):
    import torch
    dev = to_device(host)
    print(f"[case] shards rows {host.shape[0]} V {host.shape[1]} K {K} G {G}", flush=True)
    gi, gl, gs = sharded(L, dev, K, G)
    ui, ul, us = L.topk_lse(dev, K)
    torch.cuda.synchronize()
    gi, gl, gs = gi.cpu().numpy(), gl.cpu().numpy(), gs.cpu().numpy()
    assert np.array_equal(gi, ui.cpu().numpy()), "ids differ from the unsharded kernel"
    rows = range(host.shape[0]) if sample_rows is None else sample_rows
    for r in rows:
        idx, logp, lse = topk_lse_row(host[r], K)
        assert np.array_equal(gi[r], idx), f"row {r}: ids"
        assert_within(gl[r], logp, what=f"row {r} logp")
        assert_within(gs[r], lse, what=f"row {r} lse")


@pytest.mark.parametrize("G", [1, 2, 7, 8, 64])
def test_shards_c1_rows(L, G):
    w = synth.WORKLOADS["c1_qwen3_8b"]
    host = synth.make_logits(w).reshape(-1, w.vocab)
    _check(L, host, w.topk, G)


@pytest.mark.parametrize("tier", [0, 2])
def test_shards_entropy_rows(L, tier):
    w = synth.WORKLOADS["entropy_k32"]
    host = synth.make_logits(w, tier, num_blocks=4).reshape(-1, w.vocab)
    _check(L, host, w.topk, 8, sample_rows=[0, 17, 63])


@pytest.mark.parametrize("rows,V,K,G", [(33, 4099, 16, 7), (5, 1000, 64, 3), (512, 2048, 8, 4), (3, 640, 4, 64)])
@pytest.mark.parametrize("kind", ["f32", "bf16", "ties"])
def test_shards_shape_zoo(L, rows, V, K, G, kind):
    rng = np.random.default_rng(rows + V + K + G)
    if kind == "ties":      # few distinct values: ties straddle every shard boundary
        host = rng.integers(-3, 3, size=(rows, V)).astype(np.float32)
    else:
        host = rng.standard_normal((rows, V)).astype(np.float32)
        if kind == "bf16":
            host = synth.f32_to_bf16_bits_rne(host)
    _check(L, host, K, G, sample_rows=range(min(rows, 12)))


def test_shards_full_256_block_rows(L):
    # the 256-block workload at an 8-way split: each shard is [4096, 18992]
    w = synth.WORKLOADS["c256_k16"]
    host = synth.make_logits(w).reshape(-1, w.vocab)
    _check(L, host, w.topk, 8, sample_rows=[0, 1, 2047, 4095])


def test_shard_argument_errors(L):
    import torch
    x = torch.zeros((4, 100), dtype=torch.float32, device="cuda")
    with pytest.raises(L.LilicorrError):
        L.topk_shard(x, 101, 0)                 # K > V_shard
    with pytest.raises(L.LilicorrError):
        L.topk_shard(x, 8, -1)                  # negative id offset
    with pytest.raises(L.LilicorrError):
        L.topk_shard(x, 8, 2 ** 31 - 50)        # ids past int32
    v = torch.zeros((65, 4, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(L.LilicorrError):
        L.topk_merge(v, v.int(), torch.zeros((65, 4, 2), device="cuda"))   # G > 64
