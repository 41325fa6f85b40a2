"""lilicorr_rerank_noalloc against lilicorr_rerank (GPU).

The allocation-free entry point runs the same launch sequence on the
library's fixed device scratch instead of a caller's workspace, so its outputs
must equal lilicorr_rerank's bit for bit. Two calls in a row, the second
smaller than the first (the scratch keeps the first call's contents), and a
problem above the scratch is refused on the host with ETOOLARGE.
"""
import numpy as np
import pytest

from helpers import to_device, device_weights
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import torch
    import draft_block_candidate_amd as lib
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib.lib()
    return lib


def _same(a, b):
    import torch
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    return torch.equal(a, b)


def _compare(L, logits, w, weights, **kw):
    import torch
    ref_tok, ref_dbg = L.rerank(logits, w.topk, weights, w.alpha, w.use_logp, debug=True, **kw)
    torch.cuda.synchronize()
    tok, dbg = L.rerank(logits, w.topk, weights, w.alpha, w.use_logp, debug=True, noalloc=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(tok, ref_tok)
    for k in ref_dbg:
        assert _same(dbg[k], ref_dbg[k]), k


def test_noalloc_matches_rerank_on_two_calls_second_smaller(L):
    w = synth.WORKLOADS["c32"]
    weights = device_weights(w)
    host = synth.make_logits(w, num_blocks=4)
    print("[case] noalloc c32-shaped blocks: 4 blocks, then 1 block", flush=True)
    _compare(L, to_device(host[:4]), w, weights)
    _compare(L, to_device(host[1:2]), w, weights)


def test_noalloc_paper_head_and_tiny(L):
    for name in ("paper_qwen3_8b", "tiny"):
        w = synth.WORKLOADS[name]
        print(f"[case] noalloc {name}", flush=True)
        kw = {}
        if w.target_hidden:
            hid, tgt = synth.make_head_inputs(w)
            kw = {"hidden": to_device(hid), "target": to_device(tgt)}
        _compare(L, to_device(synth.make_logits(w)), w, device_weights(w), **kw)


def test_noalloc_refuses_problems_above_its_scratch(L):
    import torch
    w = synth.WORKLOADS["c32"]           # 32 blocks need ~94 MiB of workspace
    weights = device_weights(w)
    assert L.workspace_bytes(32, w.slots, w.vocab, w.topk, weights.dims) > L.NOALLOC_SCRATCH_BYTES
    logits = torch.zeros((32, w.slots, w.vocab), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(L.LilicorrError) as e:
        L.rerank(logits, w.topk, weights, noalloc=True)
    assert e.value.code == L.ETOOLARGE
