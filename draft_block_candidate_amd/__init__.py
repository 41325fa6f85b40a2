"""Python binding of liblilicorr.so, the gfx950 LiLiCorr reranking library.

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch provides device memory and the current stream. The entry
points and their contracts are those of include/lilicorr.h. Importing this
module does not need a GPU; calling a compute entry point without the built
library raises ``LilicorrUnavailable``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblilicorr.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EWEIGHTS, EHIP, ETOOLARGE = 0, -1, -2, -3, -4, -5, -6
NOALLOC_SCRATCH_BYTES = 48 << 20
F32, BF16 = 0, 1
EPI_F32, EPI_BF16, EPI_SILU_BF16, EPI_RESID_F32 = 0, 1, 2, 3
# lilicorr_stage values (per-layer stages of layer l: base + 5*l)
STAGE_TOPK, STAGE_NODE, STAGE_CONF_LINEAR = 0, 1, 2
STAGE_QKV, STAGE_ATTENTION, STAGE_O, STAGE_FFN1, STAGE_FFN2 = 3, 4, 5, 6, 7
STAGE_HEADS, STAGE_SCORES_WALK, STAGE_COUNT = 13, 14, 15
ABI_VERSION = 3
# commit rules (lilicorr_rule)
RULE_GREEDY, RULE_EXACT, RULE_SAMPLE = 0, 1, 2
_RULES = {"greedy": RULE_GREEDY, "exact": RULE_EXACT, "sample": RULE_SAMPLE}
MAX_SLOTS, MAX_TOPK, MAX_LATTICE = 64, 64, 512


class LilicorrUnavailable(RuntimeError):
    pass


class LilicorrError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} ({code})")


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("heads", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("d_e", ctypes.c_int32), ("layers", ctypes.c_int32),
                ("target_hidden", ctypes.c_int32), ("drafter_hidden", ctypes.c_int32)]


class WeightsDesc(ctypes.Structure):
    _fields_ = [("dims", Dims), ("vocab", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("dev", ctypes.c_void_p), ("bytes", ctypes.c_size_t)]


class Params(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("num_blocks", ctypes.c_int32),
                ("logits_dtype", ctypes.c_int32), ("alpha", ctypes.c_float),
                ("use_logp", ctypes.c_int32), ("weights", ctypes.POINTER(WeightsDesc)),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("stream", ctypes.c_void_p),
                ("dbg_topk_idx", ctypes.c_void_p), ("dbg_topk_logp", ctypes.c_void_p),
                ("dbg_lse", ctypes.c_void_p), ("dbg_outv", ctypes.c_void_p),
                ("dbg_inv", ctypes.c_void_p), ("dbg_cos", ctypes.c_void_p),
                ("dbg_score", ctypes.c_void_p), ("dbg_gap", ctypes.c_void_p),
                ("timing_stage", ctypes.c_int32), ("timing_begin", ctypes.c_void_p),
                ("timing_end", ctypes.c_void_p),
                ("rule", ctypes.c_int32), ("temperature", ctypes.c_void_p),
                ("uniforms", ctypes.c_void_p), ("proposal", ctypes.c_void_p),
                ("hidden", ctypes.c_void_p), ("target", ctypes.c_void_p)]


_c_int, _c_size, _vp, _f = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_SIGNATURES = {
    "lilicorr_rerank": (_c_int, [_vp, _c_int, _c_int, _c_int, ctypes.POINTER(Params), _vp]),
    "lilicorr_validate": (_c_int, [_vp, _c_int, _c_int, _c_int, ctypes.POINTER(Params), _vp]),
    "lilicorr_rerank_noalloc": (_c_int, [_vp, _c_int, _c_int, _c_int, ctypes.POINTER(Params), _vp]),
    "lilicorr_rerank_audit": (_c_int, [_c_int, _c_int, _c_int, _c_int, ctypes.POINTER(Dims), _c_int,
                                       ctypes.c_char_p, _c_size]),
    "lilicorr_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, ctypes.POINTER(Dims)]),
    "lilicorr_weights_bytes": (_c_size, [ctypes.POINTER(Dims), _c_int]),
    "lilicorr_weights_init": (_c_int, [ctypes.POINTER(WeightsDesc), _vp]),
    "lilicorr_weights_tensor": (_c_int, [ctypes.POINTER(Dims), _c_int, _c_int, ctypes.POINTER(_c_size),
                                         ctypes.POINTER(_c_size), ctypes.POINTER(_c_int)]),
    "lilicorr_strerror": (ctypes.c_char_p, [_c_int]),
    "lilicorr_topk_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "lilicorr_topk_lse": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _vp, _c_size, _vp, _vp, _vp, _vp]),
    "lilicorr_topk_shard_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "lilicorr_topk_shard": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _c_size, _vp, _vp, _vp,
                                     _vp]),
    "lilicorr_topk_merge": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp]),
    "lilicorr_pair_scores": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp]),
    "lilicorr_greedy_walk": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _f, _c_int, _vp, _vp, _vp, _vp]),
    "lilicorr_best_path": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _f, _c_int, _vp, _vp, _vp]),
    "lilicorr_sample_path": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _f, _c_int, _vp, _vp, _vp, _vp,
                                      _vp, _vp]),
    "lilicorr_linear_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "lilicorr_linear": (_c_int, [_vp, _c_int, _c_int, _vp, _c_int, _vp, _c_int, _vp, _vp, _vp, _c_size, _vp]),
    "lilicorr_rmsnorm": (_c_int, [_vp, _c_int, _c_int, _vp, _f, _vp, _vp]),
    "lilicorr_lattice_attention": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp]),
    "lilicorr_clock_probe": (_c_int, [_vp, ctypes.c_int64, _vp]),
}

_lib = None


def lib():
    """Load liblilicorr.so (built in-tree by draft_block_candidate_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LilicorrUnavailable(
                f"{LIB_PATH} is missing: build it with `python -m draft_block_candidate_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def strerror(code: int) -> str:
    return lib().lilicorr_strerror(code).decode()


def _check(code: int, where: str):
    if code != OK:
        raise LilicorrError(code, where)


def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


class LilicorrArgumentError(LilicorrError):
    """A tensor handed to the binding has the wrong device, layout, dtype or shape
    (status EINVAL; raised before anything is passed to the library)."""

    def __init__(self, where: str, why: str):
        self.code = EINVAL
        RuntimeError.__init__(self, f"{where}: {why}")


def _require_cuda(t, name):
    if not t.is_cuda:
        raise LilicorrArgumentError(name, "must be a device tensor")
    if not t.is_contiguous():
        raise LilicorrArgumentError(name, "must be contiguous")


def _require(t, name, dtype, shape, device=None):
    """Check a tensor the library will read or write through a raw pointer:
    on the device (the same one as the call's other tensors), contiguous, of
    the dtype and the exact shape the C ABI documents for it."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise LilicorrArgumentError(name, "must be a torch tensor")
    _require_cuda(t, name)
    if device is not None and t.device != device:
        raise LilicorrArgumentError(name, f"is on {t.device}, the call's other tensors on {device}")
    if t.dtype != dtype:
        raise LilicorrArgumentError(name, f"must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise LilicorrArgumentError(name, f"must have shape {tuple(shape)}, got {tuple(t.shape)}")


@dataclass(frozen=True)
class EncoderDims:
    hidden: int
    heads: int
    ffn: int
    d_e: int
    layers: int = 2
    target_hidden: int = 0      # > 0: the paper's head (with drafter_hidden)
    drafter_hidden: int = 0

    def c(self) -> Dims:
        return Dims(self.hidden, self.heads, self.ffn, self.d_e, self.layers, self.target_hidden,
                    self.drafter_hidden)


def weights_bytes(dims: EncoderDims, vocab: int) -> int:
    d = dims.c()
    return int(lib().lilicorr_weights_bytes(ctypes.byref(d), vocab))


def workspace_bytes(N: int, B: int, V: int, K: int, dims: EncoderDims) -> int:
    d = dims.c()
    return int(lib().lilicorr_workspace_bytes(N, B, V, K, ctypes.byref(d)))


def weights_tensor_info(dims: EncoderDims, vocab: int, tensor_id: int):
    d = dims.c()
    off, n, dt = _c_size(), _c_size(), _c_int()
    _check(lib().lilicorr_weights_tensor(ctypes.byref(d), vocab, tensor_id, ctypes.byref(off),
                                         ctypes.byref(n), ctypes.byref(dt)), "weights_tensor")
    return int(off.value), int(n.value), int(dt.value)


class Weights:
    """Device blob of synthetic encoder weights, filled by lilicorr_weights_init."""

    def __init__(self, dims: EncoderDims, vocab: int, seed: int = 42, device="cuda"):
        torch = _torch()
        self.dims, self.vocab, self.seed = dims, vocab, seed
        nbytes = weights_bytes(dims, vocab)
        if nbytes == 0:
            raise LilicorrError(EUNSUPPORTED, "weights_bytes")
        self.blob = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.desc = WeightsDesc(dims.c(), vocab, seed, ctypes.c_void_p(self.blob.data_ptr()), nbytes)
        _check(lib().lilicorr_weights_init(ctypes.byref(self.desc), _stream()), "weights_init")

    def tensor(self, tensor_id: int):
        """View of one stored tensor (bf16 as torch.bfloat16, else float32), flat."""
        torch = _torch()
        off, n, dt = weights_tensor_info(self.dims, self.vocab, tensor_id)
        size = 2 if dt == BF16 else 4
        raw = self.blob[off:off + n * size]
        return raw.view(torch.bfloat16) if dt == BF16 else raw.view(torch.float32)


def _logits_dtype(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError("logits must be bfloat16 or float32")


class Workspace:
    """Reusable device scratch for rerank calls of one shape."""

    def __init__(self, N, B, V, K, dims: EncoderDims, device="cuda"):
        torch = _torch()
        self.nbytes = workspace_bytes(N, B, V, K, dims)
        if self.nbytes == 0:
            raise LilicorrError(EINVAL, "workspace_bytes")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)


def make_params(N, logits_dtype, weights: Weights, workspace: Workspace | None, alpha=1.0, use_logp=True,
                stream=None, dbg=None, rule: str = "greedy", temperature=None, uniforms=None,
                proposal=None, hidden=None, target=None) -> Params:
    p = Params()
    p.hidden = _ptr(hidden)
    p.target = _ptr(target)
    p.rule = _RULES[rule]
    p.temperature = _ptr(temperature)
    p.uniforms = _ptr(uniforms)
    p.proposal = _ptr(proposal)
    p.abi_version = ABI_VERSION
    p.num_blocks = N
    p.logits_dtype = logits_dtype
    p.alpha = alpha
    p.use_logp = 1 if use_logp else 0
    p.weights = ctypes.pointer(weights.desc)
    p.workspace = ctypes.c_void_p(workspace.buf.data_ptr() if workspace is not None else 0)
    p.workspace_bytes = workspace.nbytes if workspace is not None else 0
    p.stream = stream if stream is not None else _stream()
    for k, v in (dbg or {}).items():
        setattr(p, "dbg_" + k, ctypes.c_void_p(v.data_ptr()))
    return p


def rerank(logits, K: int, weights: Weights, alpha: float = 1.0, use_logp: bool = True,
           workspace: Workspace | None = None, debug: bool = False, out=None, rule: str = "greedy",
           temperature=None, uniforms=None, proposal=None, hidden=None, target=None,
           noalloc: bool = False):
    """Rerank [N, B, V] device logits; returns int32 tokens [N, B] (and debug tensors).

    noalloc=True calls lilicorr_rerank_noalloc, whose workspace is the library's
    fixed device scratch (no workspace is allocated or passed).

    rule: "greedy", "exact" or "sample" (then temperature [N] and uniforms [N, B]
    float32 device tensors are required; proposal [N, B, K] float32 is optional).
    With the paper's head (weights.dims.target_hidden > 0) hidden [N, B, H_d] and
    target [N, H_t] bfloat16 device tensors are required."""
    torch = _torch()
    _require_cuda(logits, "logits")
    if logits.dim() != 3:
        raise LilicorrArgumentError("logits", f"must be [N, B, V], got shape {tuple(logits.shape)}")
    N, B, V = logits.shape
    dev = logits.device
    d = weights.dims
    if weights.blob.device != dev:
        raise LilicorrArgumentError("weights", f"are on {weights.blob.device}, the logits on {dev}")
    if noalloc:
        workspace = None
    elif workspace is None:
        workspace = Workspace(N, B, V, K, weights.dims, device=dev)
    elif workspace.buf.device != dev:
        raise LilicorrArgumentError("workspace", f"is on {workspace.buf.device}, the logits on {dev}")
    if out is None:
        out = torch.empty((N, B), dtype=torch.int32, device=dev)
    _require(out, "out", torch.int32, (N, B), dev)
    if temperature is not None:
        _require(temperature, "temperature", torch.float32, (N,), dev)
    if uniforms is not None:
        _require(uniforms, "uniforms", torch.float32, (N, B), dev)
    if proposal is not None:
        _require(proposal, "proposal", torch.float32, (N, B, K), dev)
    if hidden is not None:
        _require(hidden, "hidden", torch.bfloat16, (N, B, d.drafter_hidden), dev)
    if target is not None:
        _require(target, "target", torch.bfloat16, (N, d.target_hidden), dev)
    dbg = None
    if debug:
        de = weights.dims.d_e
        dbg = {
            "topk_idx": torch.empty((N, B, K), dtype=torch.int32, device=dev),
            "topk_logp": torch.empty((N, B, K), dtype=torch.float32, device=dev),
            "lse": torch.empty((N, B), dtype=torch.float32, device=dev),
            "outv": torch.empty((N, B, K, de), dtype=torch.bfloat16, device=dev),
            "inv": torch.empty((N, B, K, de), dtype=torch.bfloat16, device=dev),
            "cos": torch.empty((N, max(B - 1, 1), K, K), dtype=torch.float32, device=dev),
            "score": torch.empty((N, B), dtype=torch.float32, device=dev),
            "gap": torch.empty((N, B), dtype=torch.float32, device=dev),
        }
    p = make_params(N, _logits_dtype(logits), weights, workspace, alpha, use_logp, dbg=dbg, rule=rule,
                    temperature=temperature, uniforms=uniforms, proposal=proposal, hidden=hidden,
                    target=target)
    if noalloc:
        _check(lib().lilicorr_rerank_noalloc(_ptr(logits), B, V, K, ctypes.byref(p), _ptr(out)), "rerank_noalloc")
    else:
        _check(lib().lilicorr_rerank(_ptr(logits), B, V, K, ctypes.byref(p), _ptr(out)), "rerank")
    return (out, dbg) if debug else out


def validate(logits_ptr: int, N: int, B: int, V: int, K: int, logits_dtype: int,
             weights_desc: WeightsDesc | None, workspace_ptr: int, workspace_nbytes: int,
             out_ptr: int, abi_version: int = ABI_VERSION, use_logp: int = 1,
             timing: tuple[int, int, int] | None = None, rule: int = RULE_GREEDY,
             temperature_ptr: int = 0, uniforms_ptr: int = 0, hidden_ptr: int = 0,
             target_ptr: int = 0) -> int:
    """Host-only argument check of rerank (no GPU needed); returns the status code.

    timing = (stage, begin_event, end_event) as plain integers (handles are
    only checked for presence here)."""
    p = Params()
    p.abi_version = abi_version
    p.num_blocks = N
    p.logits_dtype = logits_dtype
    p.alpha = 1.0
    p.use_logp = use_logp
    p.weights = ctypes.pointer(weights_desc) if weights_desc is not None else None
    p.workspace = ctypes.c_void_p(workspace_ptr)
    p.workspace_bytes = workspace_nbytes
    p.rule = rule
    p.temperature = ctypes.c_void_p(temperature_ptr)
    p.uniforms = ctypes.c_void_p(uniforms_ptr)
    p.hidden = ctypes.c_void_p(hidden_ptr)
    p.target = ctypes.c_void_p(target_ptr)
    if timing is not None:
        p.timing_stage, p.timing_begin, p.timing_end = timing[0], timing[1] or None, timing[2] or None
    return int(lib().lilicorr_validate(ctypes.c_void_p(logits_ptr), B, V, K, ctypes.byref(p),
                                       ctypes.c_void_p(out_ptr)))


def rerank_audit(N: int, B: int, V: int, K: int, dims: EncoderDims, drop_step: int = -1):
    """Host-only audit of the rerank launch sequence; returns (status, report lines)."""
    d = dims.c()
    buf = ctypes.create_string_buffer(1 << 16)
    st = int(lib().lilicorr_rerank_audit(N, B, V, K, ctypes.byref(d), drop_step, buf, len(buf)))
    return st, buf.value.decode().splitlines()


def topk_lse(logits2d, K: int):
    """Fused log-partition + exact top-K of [rows, V] device logits."""
    torch = _torch()
    _require_cuda(logits2d, "logits")
    if logits2d.dim() != 2:
        raise LilicorrArgumentError("logits", "must be [rows, V]")
    rows, V = logits2d.shape
    nbytes = int(lib().lilicorr_topk_workspace_bytes(rows, V, K))
    if nbytes == 0:
        raise LilicorrError(EINVAL, "topk_workspace_bytes")
    ws = torch.empty(nbytes, dtype=torch.uint8, device=logits2d.device)
    idx = torch.empty((rows, K), dtype=torch.int32, device=logits2d.device)
    logp = torch.empty((rows, K), dtype=torch.float32, device=logits2d.device)
    lse = torch.empty((rows,), dtype=torch.float32, device=logits2d.device)
    _check(lib().lilicorr_topk_lse(_ptr(logits2d), rows, V, K, _logits_dtype(logits2d), _ptr(ws), nbytes,
                                   _ptr(idx), _ptr(logp), _ptr(lse), _stream()), "topk_lse")
    return idx, logp, lse


def topk_shard(logits2d, K: int, id_offset: int, out=None, workspace=None):
    """One shard of a split vocabulary: [rows, V_shard] device logits holding ids
    id_offset.. -> (values f32 [rows, K], global ids i32 [rows, K], (m, s) f32 [rows, 2]).
    out: optional (values, ids, ms) views to write into (e.g. slices of stacked buffers)."""
    torch = _torch()
    _require_cuda(logits2d, "logits")
    if logits2d.dim() != 2:
        raise LilicorrArgumentError("logits", "must be [rows, V_shard]")
    rows, V = logits2d.shape
    dev = logits2d.device
    nbytes = int(lib().lilicorr_topk_shard_workspace_bytes(rows, V, K))
    if nbytes == 0:
        raise LilicorrError(EINVAL, "topk_shard_workspace_bytes")
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if out is None:
        out = (torch.empty((rows, K), dtype=torch.float32, device=dev),
               torch.empty((rows, K), dtype=torch.int32, device=dev),
               torch.empty((rows, 2), dtype=torch.float32, device=dev))
    val, idx, ms = out
    _require(val, "values", torch.float32, (rows, K), dev)
    _require(idx, "ids", torch.int32, (rows, K), dev)
    _require(ms, "ms", torch.float32, (rows, 2), dev)
    _require(workspace, "workspace", torch.uint8, (workspace.numel(),), dev)
    _check(lib().lilicorr_topk_shard(_ptr(logits2d), rows, V, K, _logits_dtype(logits2d), id_offset,
                                     _ptr(workspace), workspace.numel(), _ptr(val), _ptr(idx), _ptr(ms),
                                     _stream()), "topk_shard")
    return val, idx, ms


def topk_merge(val, idx, ms):
    """Merge stacked shard outputs [G, rows, K] / [G, rows, 2] -> (ids, logp, lse)."""
    torch = _torch()
    _require_cuda(val, "values")
    if val.dim() != 3:
        raise LilicorrArgumentError("values", "must be [G, rows, K]")
    G, rows, K = val.shape
    dev = val.device
    _require(val, "values", torch.float32, (G, rows, K), dev)
    _require(idx, "ids", torch.int32, (G, rows, K), dev)
    _require(ms, "ms", torch.float32, (G, rows, 2), dev)
    tidx = torch.empty((rows, K), dtype=torch.int32, device=dev)
    logp = torch.empty((rows, K), dtype=torch.float32, device=dev)
    lse = torch.empty((rows,), dtype=torch.float32, device=dev)
    _check(lib().lilicorr_topk_merge(_ptr(val), _ptr(idx), _ptr(ms), G, rows, K, _ptr(tidx), _ptr(logp),
                                     _ptr(lse), _stream()), "topk_merge")
    return tidx, logp, lse


def pair_scores(outv, inv):
    """outv, inv: [N, B, K, d_e] bf16 device tensors -> cos [N, B-1, K, K] float32."""
    torch = _torch()
    _require_cuda(outv, "outv")
    if outv.dim() != 4:
        raise LilicorrArgumentError("outv", "must be [N, B, K, d_e]")
    N, B, K, de = outv.shape
    _require(outv, "outv", torch.bfloat16, (N, B, K, de))
    _require(inv, "inv", torch.bfloat16, (N, B, K, de), outv.device)
    cos = torch.empty((N, B - 1, K, K), dtype=torch.float32, device=outv.device)
    _check(lib().lilicorr_pair_scores(_ptr(outv), _ptr(inv), N, B, K, de, _ptr(cos), _stream()),
           "pair_scores")
    return cos


def greedy_walk(topk_idx, topk_logp, cos, alpha: float = 1.0, use_logp: bool = True):
    """Greedy commit; returns (tokens int32 [N,B], score, gap float32 [N,B])."""
    torch = _torch()
    _require_cuda(topk_idx, "topk_idx")
    if topk_idx.dim() != 3:
        raise LilicorrArgumentError("topk_idx", "must be [N, B, K]")
    N, B, K = topk_idx.shape
    dev = topk_idx.device
    _require(topk_idx, "topk_idx", torch.int32, (N, B, K), dev)
    _require(topk_logp, "topk_logp", torch.float32, (N, B, K), dev)
    if B > 1 or cos is not None:
        _require(cos, "cos", torch.float32, (N, max(B - 1, 1), K, K), dev)
    out = torch.empty((N, B), dtype=torch.int32, device=dev)
    score = torch.empty((N, B), dtype=torch.float32, device=dev)
    gap = torch.empty((N, B), dtype=torch.float32, device=dev)
    _check(lib().lilicorr_greedy_walk(_ptr(topk_idx), _ptr(topk_logp), _ptr(cos), N, B, K, alpha,
                                      1 if use_logp else 0, _ptr(out), _ptr(score), _ptr(gap), _stream()),
           "greedy_walk")
    return out, score, gap


def best_path(topk_idx, topk_logp, cos, alpha: float = 1.0, use_logp: bool = True):
    """Exact best path over given scores; returns (tokens int32 [N,B], score float32 [N,B])."""
    torch = _torch()
    _require_cuda(topk_idx, "topk_idx")
    if topk_idx.dim() != 3:
        raise LilicorrArgumentError("topk_idx", "must be [N, B, K]")
    N, B, K = topk_idx.shape
    dev = topk_idx.device
    _require(topk_idx, "topk_idx", torch.int32, (N, B, K), dev)
    _require(topk_logp, "topk_logp", torch.float32, (N, B, K), dev)
    if B > 1 or cos is not None:
        _require(cos, "cos", torch.float32, (N, max(B - 1, 1), K, K), dev)
    out = torch.empty((N, B), dtype=torch.int32, device=dev)
    score = torch.empty((N, B), dtype=torch.float32, device=dev)
    _check(lib().lilicorr_best_path(_ptr(topk_idx), _ptr(topk_logp), _ptr(cos), N, B, K, alpha,
                                    1 if use_logp else 0, _ptr(out), _ptr(score), _stream()), "best_path")
    return out, score


def sample_path(topk_idx, topk_logp, cos, temperature, uniforms, alpha: float = 1.0,
                use_logp: bool = True):
    """Sampled commit over given scores; returns (tokens int32 [N,B],
    proposal float32 [N,B,K], score float32 [N,B])."""
    torch = _torch()
    _require_cuda(topk_idx, "topk_idx")
    if topk_idx.dim() != 3:
        raise LilicorrArgumentError("topk_idx", "must be [N, B, K]")
    N, B, K = topk_idx.shape
    dev = topk_idx.device
    _require(topk_idx, "topk_idx", torch.int32, (N, B, K), dev)
    _require(topk_logp, "topk_logp", torch.float32, (N, B, K), dev)
    if B > 1 or cos is not None:
        _require(cos, "cos", torch.float32, (N, max(B - 1, 1), K, K), dev)
    _require(temperature, "temperature", torch.float32, (N,), dev)
    _require(uniforms, "uniforms", torch.float32, (N, B), dev)
    out = torch.empty((N, B), dtype=torch.int32, device=dev)
    prop = torch.empty((N, B, K), dtype=torch.float32, device=dev)
    score = torch.empty((N, B), dtype=torch.float32, device=dev)
    _check(lib().lilicorr_sample_path(_ptr(topk_idx), _ptr(topk_logp), _ptr(cos), N, B, K, alpha,
                                      1 if use_logp else 0, _ptr(temperature), _ptr(uniforms), _ptr(out),
                                      _ptr(prop), _ptr(score), _stream()), "sample_path")
    return out, prop, score


def linear(A, W, bias=None, epilogue: int = EPI_F32, resid=None, workspace=None):
    """Y = A W^T + bias on MFMA with the given epilogue; A [M, Kd], W [N, Kd] bf16."""
    torch = _torch()
    _require_cuda(A, "A")
    if A.dim() != 2 or W.dim() != 2:
        raise LilicorrArgumentError("linear", "A and W must be 2-D")
    M, Kd = A.shape
    N = W.shape[0]
    dev = A.device
    _require(A, "A", torch.bfloat16, (M, Kd), dev)
    _require(W, "W", torch.bfloat16, (N, Kd), dev)
    if bias is not None:
        _require(bias, "bias", torch.float32, (N,), dev)
    if resid is not None:
        _require(resid, "resid", torch.float32, (M, N), dev)
    if epilogue in (EPI_F32, EPI_RESID_F32):
        out = resid if (epilogue == EPI_RESID_F32 and resid is not None) else torch.empty((M, N), dtype=torch.float32, device=A.device)
    else:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    nbytes = int(lib().lilicorr_linear_workspace_bytes(M, Kd, N))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=A.device)
    _check(lib().lilicorr_linear(_ptr(A), M, Kd, _ptr(W), N, _ptr(bias), epilogue, _ptr(resid), _ptr(out),
                                 _ptr(workspace), workspace.numel(), _stream()), "linear")
    return out


def rmsnorm(x, gamma, eps: float = 1e-6):
    torch = _torch()
    _require_cuda(x, "x")
    if x.dim() != 2:
        raise LilicorrArgumentError("x", "must be [M, H]")
    M, H = x.shape
    _require(x, "x", torch.float32, (M, H), x.device)
    _require(gamma, "gamma", torch.float32, (H,), x.device)
    out = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    _check(lib().lilicorr_rmsnorm(_ptr(x), M, H, _ptr(gamma), eps, _ptr(out), _stream()), "rmsnorm")
    return out


def clock_probe(out, window_us: int, stream=None):
    """Diagnostic (not part of the path): launch the shader-clock probe on
    `stream` (default: the current one). `out` is a device int64 tensor [2];
    once the probe has run, 0.1 * out[1] / out[0] is the shader clock in GHz
    over its window (see lilicorr_clock_probe)."""
    torch = _torch()
    _require(out, "out", torch.int64, (2,))
    s = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
    _check(lib().lilicorr_clock_probe(_ptr(out), int(window_us), ctypes.c_void_p(s)), "clock_probe")


def lattice_attention(qkv, N: int, B: int, K: int, hidden: int, heads: int, dist, same):
    torch = _torch()
    _require(qkv, "qkv", torch.bfloat16, (N * B * K, 3 * hidden))
    _require(dist, "dist", torch.float32, (heads, 127), qkv.device)
    _require(same, "same", torch.float32, (heads,), qkv.device)
    out = torch.empty((N * B * K, hidden), dtype=torch.bfloat16, device=qkv.device)
    _check(lib().lilicorr_lattice_attention(_ptr(qkv), N, B, K, hidden, heads, _ptr(dist), _ptr(same),
                                            _ptr(out), _stream()), "lattice_attention")
    return out
