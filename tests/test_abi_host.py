"""Host-side checks of the C ABI (no GPU needed).

The library must load without a GPU, export every entry point the header
declares, and reject bad arguments in its host-only validation with the
documented status codes, without launching anything.
"""
import ctypes
import os
import re
import subprocess

import pytest

import draft_block_candidate_amd as L
from oracle.weights import weight_table, Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lilicorr.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="library not built")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LILICORR_API\s+[^;(]*?\b(lilicorr_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("lilicorr_rerank", "lilicorr_validate", "lilicorr_workspace_bytes",
                 "lilicorr_weights_bytes", "lilicorr_weights_init", "lilicorr_strerror",
                 "lilicorr_topk_lse", "lilicorr_greedy_walk", "lilicorr_pair_scores",
                 "lilicorr_best_path", "lilicorr_sample_path", "lilicorr_topk_shard",
                 "lilicorr_topk_merge"):
        assert must in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s+(lilicorr_\w+)", out))
    assert set(declared_functions()) <= exported
    # internal helpers stay hidden
    assert not any(s.startswith("_ZN2ll") for s in re.findall(r"\s[TW]\s+(\S+)", out))
    lib = L.lib()
    for name in declared_functions():
        assert getattr(lib, name) is not None


def test_bindings_cover_the_header():
    assert set(declared_functions()) == set(L._SIGNATURES)


def test_clock_probe_rejects_bad_arguments():
    """The diagnostic clock probe checks its arguments before touching a device."""
    lib = L.lib()
    fake = ctypes.c_void_p(4096)
    assert lib.lilicorr_clock_probe(None, 100, None) == L.EINVAL
    assert lib.lilicorr_clock_probe(ctypes.c_void_p(4097), 100, None) == L.EINVAL   # misaligned
    assert lib.lilicorr_clock_probe(fake, 0, None) == L.EINVAL
    assert lib.lilicorr_clock_probe(fake, 1000001, None) == L.EINVAL


def test_strerror_codes():
    assert L.strerror(0) == "ok"
    assert "workspace" in L.strerror(L.EWORKSPACE)
    assert L.strerror(12345) == "unknown status"


DIMS = L.EncoderDims(64, 2, 256, 32)
PAPER_DIMS = L.EncoderDims(64, 2, 128, 32, target_hidden=128, drafter_hidden=192)


def _good(**over):
    args = dict(logits_ptr=1 << 20, N=1, B=16, V=1024, K=4, logits_dtype=L.F32, vocab=1024,
                dims=over.get("dims", DIMS), wptr=1 << 24, wbytes=None, ws=1 << 28, wsbytes=None, out=1 << 12,
                abi=L.ABI_VERSION, use_logp=1, weights=True, timing=None, rule=L.RULE_GREEDY,
                temp=0, unif=0)
    args.update(over)
    wb = args["wbytes"] if args["wbytes"] is not None else L.weights_bytes(args["dims"], args["vocab"])
    desc = L.WeightsDesc(args["dims"].c(), args["vocab"], 42, ctypes.c_void_p(args["wptr"]), wb) if args["weights"] else None
    wsb = args["wsbytes"]
    if wsb is None:
        wsb = L.workspace_bytes(args["N"], args["B"], args["V"], args["K"], args["dims"]) or (1 << 30)
    return L.validate(args["logits_ptr"], args["N"], args["B"], args["V"], args["K"], args["logits_dtype"],
                      desc, args["ws"], wsb, args["out"], args["abi"], args["use_logp"], args["timing"],
                      args["rule"], args["temp"], args["unif"], args.get("hid", 0), args.get("tgt", 0))


@pytest.mark.parametrize("over,code", [
    ({}, L.OK),
    ({"logits_ptr": 0}, L.EINVAL),
    ({"out": 0}, L.EINVAL),
    ({"abi": 1}, L.EINVAL),                                        # layout before the commit rules
    ({"N": 0}, L.EINVAL),
    ({"B": 0}, L.EINVAL),
    ({"B": 65}, L.EINVAL),
    ({"K": 0}, L.EINVAL),
    ({"K": 65}, L.EINVAL),
    ({"V": 3, "vocab": 3, "wsbytes": 1 << 30}, L.EINVAL),          # K > V
    ({"B": 64, "K": 16, "wsbytes": 1 << 30}, L.EINVAL),            # B*K > 512
    ({"logits_dtype": 2}, L.EUNSUPPORTED),
    ({"logits_ptr": (1 << 20) + 8}, L.EINVAL),                     # 16-byte alignment
    ({"use_logp": 2}, L.EINVAL),
    ({"weights": False}, L.EINVAL),
    ({"dims": L.EncoderDims(64, 3, 256, 32)}, L.EUNSUPPORTED),     # heads do not divide hidden
    ({"dims": L.EncoderDims(96, 2, 256, 32)}, L.EUNSUPPORTED),     # hidden % 64
    ({"dims": L.EncoderDims(64, 2, 256, 48)}, L.EUNSUPPORTED),     # d_e % 32
    ({"vocab": 2048}, L.EWEIGHTS),
    ({"wbytes": 1024}, L.EWEIGHTS),
    ({"wptr": 0}, L.EWEIGHTS),
    ({"wptr": (1 << 24) + 16}, L.EWEIGHTS),
    ({"ws": 0}, L.EWORKSPACE),
    ({"wsbytes": 100}, L.EWORKSPACE),
    ({"ws": (1 << 28) + 64}, L.EWORKSPACE),
    ({"timing": (L.STAGE_FFN2, 0x1000, 0x2000)}, L.OK),             # stage timing events
    ({"timing": (L.STAGE_SCORES_WALK, 0x1000, 0x2000)}, L.OK),
    ({"timing": (L.STAGE_COUNT, 0x1000, 0x2000)}, L.EINVAL),       # no such stage
    ({"timing": (-1, 0x1000, 0x2000)}, L.EINVAL),
    ({"timing": (L.STAGE_TOPK, 0x1000, 0)}, L.EINVAL),             # one event only
    ({"timing": (99, 0, 0)}, L.OK),                                # no events: stage ignored
    ({"rule": L.RULE_EXACT}, L.OK),
    ({"rule": L.RULE_EXACT, "temp": 0x3000}, L.OK),                # sampling inputs ignored
    ({"rule": 3}, L.EINVAL),
    ({"rule": -1}, L.EINVAL),
    ({"rule": L.RULE_SAMPLE, "temp": 0x3000, "unif": 0x4000}, L.OK),
    ({"rule": L.RULE_SAMPLE}, L.EINVAL),                           # temperatures and uniforms required
    ({"rule": L.RULE_SAMPLE, "temp": 0x3000}, L.EINVAL),
    ({"rule": L.RULE_SAMPLE, "unif": 0x4000}, L.EINVAL),
    ({"dims": PAPER_DIMS, "hid": 0x5000, "tgt": 0x6000}, L.OK),    # the paper's head
    ({"dims": PAPER_DIMS}, L.EINVAL),                               # its inputs are required
    ({"dims": PAPER_DIMS, "hid": 0x5000}, L.EINVAL),
    ({"dims": PAPER_DIMS, "hid": 0x5008, "tgt": 0x6000}, L.EINVAL),  # 16-byte alignment
    ({"dims": PAPER_DIMS, "hid": 0x5000, "tgt": 0x6000, "B": 1, "wsbytes": 1 << 30}, L.EINVAL),  # no drafted slot
    ({"dims": L.EncoderDims(64, 2, 128, 32, target_hidden=96, drafter_hidden=128)}, L.EUNSUPPORTED),
    ({"dims": L.EncoderDims(64, 2, 128, 32, drafter_hidden=128)}, L.EUNSUPPORTED),
    ({"dims": L.EncoderDims(64, 2, 128, 1056)}, L.EUNSUPPORTED),   # d_e <= 1024
])
def test_validate_status_codes(over, code):
    assert _good(**over) == code


def test_sizes_for_the_workloads():
    import synth
    for name in synth.WORKLOADS_ORDER:
        w = synth.WORKLOADS[name]
        d = L.EncoderDims(w.hidden, w.heads, w.ffn, w.d_e, target_hidden=w.target_hidden,
                          drafter_hidden=w.drafter_hidden)
        assert L.weights_bytes(d, w.vocab) > 0
        ws = L.workspace_bytes(w.num_blocks, w.slots, w.vocab, w.topk, d)
        M = w.num_blocks * w.slots * w.topk
        assert ws >= M * w.hidden * 4 + M * w.ffn * 2
    assert L.workspace_bytes(1, 16, 1024, 65, DIMS) == 0
    assert L.weights_bytes(L.EncoderDims(64, 2, 256, 32, layers=3), 10) == 0


@pytest.mark.parametrize("paper", [False, True])
def test_weight_layout_matches_the_generator_table(paper):
    DIMS_ = PAPER_DIMS if paper else DIMS
    d = Dims(64, 2, 128, 32, target_hidden=128, drafter_hidden=192) if paper else Dims(64, 2, 256, 32)
    spans = []
    for t, name, shape, scale, kind in weight_table(d, 1024):
        off, n, dt = L.weights_tensor_info(DIMS_, 1024, t)
        assert n == (shape[0] * (shape[1] if len(shape) > 1 else 1))
        assert dt == (L.BF16 if kind == "bf16" else L.F32)
        spans.append((off, off + n * (2 if dt == L.BF16 else 4), name))
    spans.sort()
    for (a0, a1, _), (b0, b1, _) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= L.weights_bytes(DIMS_, 1024)
    wo, wi = L.weights_tensor_info(DIMS_, 1024, 49), L.weights_tensor_info(DIMS_, 1024, 51)
    assert wi[0] == wo[0] + wo[1] * 2      # one GEMM with N = 2 d_e covers both heads
    bo, bi = L.weights_tensor_info(DIMS_, 1024, 50), L.weights_tensor_info(DIMS_, 1024, 52)
    assert bi[0] == bo[0] + bo[1] * 4
    with pytest.raises(L.LilicorrError):
        L.weights_tensor_info(DIMS_, 1024, 7)
    if paper:       # the paper's head embeds with E_t only
        with pytest.raises(L.LilicorrError):
            L.weights_tensor_info(DIMS_, 1024, 0)
    else:
        with pytest.raises(L.LilicorrError):
            L.weights_tensor_info(DIMS_, 1024, 56)


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", "/nonexistent/liblilicorr.so")
    with pytest.raises(L.LilicorrUnavailable):
        L.lib()


def _parse_audit(lines):
    steps = []
    for ln in lines:
        parts = ln.split()
        reads = set() if parts[3] == "-" else set(parts[3].split(","))
        writes = set() if parts[5] == "-" else set(parts[5].split(","))
        steps.append((parts[1], reads, writes))
    return steps


AUDIT_SHAPES = [("tiny", 1), ("c1_qwen3_8b", 1), ("c32", 32), ("c256_k16", 256), ("entropy_k32", 64),
                ("odd_h2560", 41), ("paper_tiny", 1), ("paper_qwen3_8b", 1), ("paper_c32", 32)]


@pytest.mark.parametrize("name,N", AUDIT_SHAPES)
def test_rerank_reads_no_workspace_region_before_writing_it(name, N):
    # lilicorr_rerank never clears its workspace: every region a launch reads
    # must have been written by an earlier launch of the same call
    import synth
    w = synth.WORKLOADS[name]
    dims = L.EncoderDims(w.hidden, w.heads, w.ffn, w.d_e, target_hidden=w.target_hidden,
                         drafter_hidden=w.drafter_hidden)
    st, lines = L.rerank_audit(N, w.slots, w.vocab, w.topk, dims)
    assert st == L.OK, lines
    steps = _parse_audit(lines)
    assert steps[0][0] in ("topk_lse", "topk_chunks") and steps[-1][0] == "scores_walk"
    # two layers; few-row lattices of 65..128 tokens at d_h = 128 fuse the
    # output projection's per-head K slices into the attention launch
    assert sum(s[0] in ("lattice_attention", "lattice_attention_o") for s in steps) == 2
    # the audit is not vacuous: leaving out a launch whose outputs are new
    # (not all written by an earlier launch) must be caught
    for i, (nm, _, writes) in enumerate(steps):
        before = set().union(*[s[2] for s in steps[:i]]) if i else set()
        # scratch regions are written and read within one launch, unless a
        # later launch reads them (the few-row node build merges the top-K's
        # chunk outputs)
        later_reads = set().union(*[s[1] for s in steps[i + 1:]]) if i + 1 < len(steps) else set()
        scratch = {"gemm_part", "topk_part"} - later_reads
        st_drop, drop_lines = L.rerank_audit(N, w.slots, w.vocab, w.topk, dims, i)
        if writes - before - scratch:
            assert st_drop == L.EINVAL and any("UNWRITTEN" in ln for ln in drop_lines), (i, nm)
        else:
            assert st_drop == L.OK, (i, nm)


def test_rerank_audit_wide_vectors_and_bad_sizes():
    # d_e >= 512 adds the sliced pair products, whose partial sums the walk reads
    dims = L.EncoderDims(128, 2, 256, 544)
    st, lines = L.rerank_audit(2, 7, 4096, 7, dims)
    assert st == L.OK
    names = [s[0] for s in _parse_audit(lines)]
    assert names[-2:] == ["pair_slices", "scores_walk"]
    assert L.rerank_audit(0, 16, 4096, 4, dims)[0] == L.EINVAL
    assert L.rerank_audit(1, 16, 4096, 65, dims)[0] == L.EINVAL
    assert L.rerank_audit(1, 16, 4096, 4, L.EncoderDims(100, 2, 256, 32))[0] == L.EUNSUPPORTED


def test_binding_rejects_host_tensors_before_the_library():
    # a host tensor never reaches the library as a device pointer
    import torch
    w = L.EncoderDims(64, 2, 256, 32)
    with pytest.raises(L.LilicorrArgumentError) as e:
        L.rerank(torch.zeros((1, 16, 1024)), 4, None)
    assert e.value.code == L.EINVAL
    with pytest.raises(L.LilicorrArgumentError):
        L.greedy_walk(torch.zeros((1, 4, 2), dtype=torch.int32), torch.zeros((1, 4, 2)), torch.zeros((1, 3, 2, 2)))
    with pytest.raises(L.LilicorrArgumentError):
        L.topk_lse(torch.zeros((4, 100)), 4)
    del w


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define LILICORR_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == L.NOALLOC_SCRATCH_BYTES
    assert L.strerror(L.ETOOLARGE).startswith("problem needs more")
