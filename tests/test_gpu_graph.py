"""The rerank call captured in a HIP graph (GPU).

The library enqueues only kernels (no memset nodes, no host synchronisation),
so a captured call must replay identically. Each replay is checked bit for
bit against the eager result, with other eager work and synchronisations
between replays.
"""
import ctypes

import numpy as np
import pytest

from helpers import to_device, device_weights
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "c1_qwen3_8b", "c32", "paper_qwen3_8b"])
def test_graph_replays_match_eager(name):
    import torch
    import draft_block_candidate_amd as L
    w = synth.WORKLOADS[name]
    host = synth.make_logits(w)
    dev = to_device(host)
    other = to_device(synth.make_logits(w, 0)[:, ::-1].copy())   # different logits, same shape
    weights = device_weights(w)
    dims = weights.dims
    head = {}
    if w.target_hidden > 0:     # the paper's head: its drafter and target states
        hid, tgt = synth.make_head_inputs(w)
        head = {"hidden": to_device(hid), "target": to_device(tgt)}
    ws = L.Workspace(w.num_blocks, w.slots, w.vocab, w.topk, dims)
    ws_eager = L.Workspace(w.num_blocks, w.slots, w.vocab, w.topk, dims)
    eager = L.rerank(dev, w.topk, weights, w.alpha, w.use_logp, workspace=ws_eager, **head)
    torch.cuda.synchronize()

    out = torch.empty((w.num_blocks, w.slots), dtype=torch.int32, device="cuda")
    ldt = L.BF16 if w.dtype == "bf16" else L.F32
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        p = L.make_params(w.num_blocks, ldt, weights, ws, w.alpha, w.use_logp,
                          stream=ctypes.c_void_p(side.cuda_stream), **head)
        rc = L.lib().lilicorr_rerank(ctypes.c_void_p(dev.data_ptr()), w.slots, w.vocab, w.topk,
                                     ctypes.byref(p), ctypes.c_void_p(out.data_ptr()))
        assert rc == 0
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(-1)
        # unrelated eager work on the same workspace-free path between replays
        other_tok = L.rerank(other, w.topk, weights, w.alpha, w.use_logp, workspace=ws_eager, **head)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from eager"
        assert other_tok.shape == eager.shape
