"""Python binding of libkvpop.so, the MI355X (gfx950) library for the KVpop
future-attention target and fixed-budget sparse attention.

The binding only marshals arguments: every step of the computation runs in
the HIP kernels behind the C ABI declared in include/kvpop.h.  PyTorch is used
for device memory and streams.  There is no fallback: if the library is not
built, or no GPU is present, the calls raise.

Entry points (same names as the C ABI, without the ``kvpop_`` prefix):
    attn_fwd_lse(q, k, v, ...)            -> (o, lse)
    future_target(q, k, lse, window, ...) -> target
    budget_mask_fwd(q, k, v, scores, sinks, window, topk, ...) -> (o, lse, rank, cutoff)
    teacher_labels(target, sinks, window, topk, ...) -> (label, boundary)
    boundary_loss(pred, label, boundary, sinks, window, topk, tau, ...) -> (loss, grad)
    DecodeCache(...).step(q, k, v, score) -> (o, lse)   (decode_state_size / decode_init / decode_step)
    workspace_size(which, ...)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Union

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvpop.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
BF16, F32 = 0, 1
AGG_SUM, AGG_MAX, AGG_NONE = 0, 1, 2
CALL_FWD_LSE, CALL_FUTURE_TARGET, CALL_BUDGET_MASK_FWD = 0, 1, 2
CUTOFF_ALL = 2 ** 31 - 1
CUTOFF_NONE = -1
EXPORTS = ("kvpop_attn_fwd_lse", "kvpop_future_target", "kvpop_budget_mask_fwd",
           "kvpop_workspace_size", "kvpop_status_str", "kvpop_last_error",
           "kvpop_teacher_labels", "kvpop_teacher_workspace_size",
           "kvpop_boundary_loss", "kvpop_boundary_loss_workspace_size",
           "kvpop_decode_state_size", "kvpop_decode_init", "kvpop_decode_step",
           "kvpop_budget_lists_layout", "kvpop_future_target_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20

_AGG_NAMES = {"sum": AGG_SUM, "max": AGG_MAX, "none": AGG_NONE}


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("cu_seqlens", ctypes.c_void_p),
                ("cu_seqlens_host", ctypes.c_void_p), ("n_docs", ctypes.c_int32)]


class DecodeShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("sinks", ctypes.c_int32), ("window", ctypes.c_int32), ("topk", ctypes.c_int32)]


class ListsLayout(ctypes.Structure):
    _fields_ = [("lists_offset", ctypes.c_size_t), ("spans_offset", ctypes.c_size_t),
                ("lens_offset", ctypes.c_size_t),
                ("lens_full_offset", ctypes.c_size_t), ("status_offset", ctypes.c_size_t),
                ("n_query_blocks", ctypes.c_int32), ("query_block", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("tile_keys", ctypes.c_int32)]


class KvpopError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def load():
    """Load libkvpop.so (built in place by attention_target_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m attention_target_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    SP = ctypes.POINTER(Shape)
    lib.kvpop_attn_fwd_lse.argtypes = [SP, P, P, P, P, P, P]
    lib.kvpop_attn_fwd_lse.restype = I
    lib.kvpop_future_target.argtypes = [SP, P, P, P, I, I, I, F, P, P, Z, P]
    lib.kvpop_future_target.restype = I
    lib.kvpop_budget_mask_fwd.argtypes = [SP, P, P, P, P, I, I, I, P, P, P, P, P, Z, P]
    lib.kvpop_budget_mask_fwd.restype = I
    lib.kvpop_workspace_size.argtypes = [I, SP, I, I, I]
    lib.kvpop_workspace_size.restype = Z
    lib.kvpop_status_str.argtypes = [I]
    lib.kvpop_status_str.restype = ctypes.c_char_p
    lib.kvpop_last_error.argtypes = []
    lib.kvpop_last_error.restype = ctypes.c_char_p
    lib.kvpop_teacher_labels.argtypes = [I, I, I, P, P, I, I, I, I, P, P, P, P, P, Z, P]
    lib.kvpop_teacher_labels.restype = I
    lib.kvpop_teacher_workspace_size.argtypes = [I, I, I]
    lib.kvpop_teacher_workspace_size.restype = Z
    lib.kvpop_boundary_loss.argtypes = [I, I, I, P, P, P, I, I, I, F, P, P, P, P, Z, P]
    lib.kvpop_boundary_loss.restype = I
    lib.kvpop_boundary_loss_workspace_size.argtypes = [I, I, I]
    lib.kvpop_boundary_loss_workspace_size.restype = Z
    DP = ctypes.POINTER(DecodeShape)
    lib.kvpop_decode_state_size.argtypes = [DP]
    lib.kvpop_decode_state_size.restype = Z
    lib.kvpop_decode_init.argtypes = [DP, P, Z, P]
    lib.kvpop_decode_init.restype = I
    lib.kvpop_decode_step.argtypes = [DP, P, Z, I, P, P, P, P, P, P, P]
    lib.kvpop_decode_step.restype = I
    lib.kvpop_future_target_noalloc.argtypes = [SP, P, P, P, I, I, I, F, P, P]
    lib.kvpop_future_target_noalloc.restype = I
    lib.kvpop_budget_lists_layout.argtypes = [SP, I, I, I, ctypes.POINTER(ListsLayout)]
    lib.kvpop_budget_lists_layout.restype = I
    _lib = lib
    return lib


def status_str(st: int) -> str:
    return load().kvpop_status_str(st).decode()


def last_error() -> str:
    return load().kvpop_last_error().decode()


def _check(st: int):
    if st != OK:
        raise KvpopError(st, f"kvpop: {status_str(st)}: {last_error()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


class DocOffsets:
    """Host and device copies of packed document offsets (cu_seqlens).

    Every call that takes `cu_seqlens` accepts a list, a CPU tensor or a
    DocOffsets; a DocOffsets made once and passed to repeated calls saves the
    per-call device copy (the calls then allocate nothing for it)."""

    def __init__(self, cu_seqlens, device):
        if cu_seqlens is None:
            self.host = self.dev = None
            self.n_docs = 1
            return
        host = torch.as_tensor(cu_seqlens, dtype=torch.int32).detach().to("cpu").contiguous()
        self.host = host
        self.dev = host.to(device)
        self.n_docs = int(host.numel()) - 1

    def tolist(self):
        return self.host.tolist()


def _Packed(cu_seqlens, device):
    if isinstance(cu_seqlens, DocOffsets):
        return cu_seqlens
    return DocOffsets(cu_seqlens, device)


def make_shape(q: torch.Tensor, k: torch.Tensor, packed: DocOffsets, scale: float) -> Shape:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, S, D]")
    B, Hq, S, D = q.shape
    sh = Shape()
    sh.batch, sh.seqlen, sh.n_q_heads, sh.n_kv_heads, sh.head_dim = B, S, Hq, k.shape[1], D
    sh.dtype = _dtype_code(q)
    sh.softmax_scale = float(scale)
    sh.cu_seqlens = None if packed.dev is None else packed.dev.data_ptr()
    sh.cu_seqlens_host = None if packed.host is None else packed.host.data_ptr()
    sh.n_docs = packed.n_docs
    return sh


def _dev(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _require(name: str, t: torch.Tensor, dtype=None, shape=None, device=None, placed=True):
    """Shape and dtype, then contiguity, then (unless `placed` is False)
    placement: a GPU tensor, on `device` when given."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if placed:
        _placed(device, (name, t))


def _placed(device, *named):
    """Every given tensor is a GPU tensor, on `device` (or on the first one's
    device).  Called after the shape checks, so that a shape mismatch is
    reported as such whatever the device."""
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA (HIP) tensor")
        if device is None:
            device = t.device
        elif t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def _require_qkv(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor] = None):
    """q [B, Hq, S, D]; k (and v) [B, Hkv, S, D] with the same B, S, D and
    dtype, Hq a multiple of Hkv, all on q's device.  The kernels take B, S and
    D from q and read K and V with them, so any other K/V shape would be read
    out of bounds."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B, Hq, S, D]")
    if not isinstance(k, torch.Tensor) or k.dim() != 4:
        raise ValueError("k must be a 4-D tensor [B, Hkv, S, D]")
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError(f"n_q_heads ({Hq}) must be a multiple of n_kv_heads ({Hkv})")
    for name, t in (("k", k), ("v", v)):
        if t is not None and tuple(t.shape) != (B, Hkv, S, D):
            raise ValueError(f"{name} must have shape {(B, Hkv, S, D)} to match q {tuple(q.shape)}, "
                             f"got {tuple(t.shape)}")
        if t is not None and t.dtype != q.dtype:
            raise ValueError(f"{name} must have q's dtype {q.dtype}, got {t.dtype}")
    _require("q", q, placed=False)
    _require("k", k, q.dtype, (B, Hkv, S, D), placed=False)
    if v is not None:
        _require("v", v, q.dtype, (B, Hkv, S, D), placed=False)


def _stream_ptr(t: torch.Tensor, stream: Optional[torch.cuda.Stream]):
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return s.cuda_stream


def _retain(stream: Optional[torch.cuda.Stream], *tensors):
    """Tensors this binding allocated (on the current stream) and handed to
    kernels enqueued on another `stream`: marked as used there, so that the
    caching allocator does not reuse their memory before that stream has
    passed this point (on the current stream, stream order already does)."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def workspace_size(which: int, q: torch.Tensor, k: torch.Tensor, cu_seqlens=None, sinks: int = 0,
                   window: int = 0, topk: int = 0, scale: float = 0.0) -> int:
    lib = load()
    packed = _Packed(cu_seqlens, "cpu" if not q.is_cuda else q.device)
    sh = make_shape(q, k, packed, scale)
    return int(lib.kvpop_workspace_size(which, ctypes.byref(sh), sinks, window, topk))


def budget_lists_layout(q, k, sinks: int, window: int, topk: int, cu_seqlens=None, scale: float = 0.0) -> dict:
    """Where kvpop_budget_mask_fwd leaves its per-query-block key lists in its
    workspace (kvpop_budget_lists_layout): byte offsets and sizes."""
    lib = load()
    packed = _Packed(cu_seqlens, "cpu" if not q.is_cuda else q.device)
    sh = make_shape(q, k, packed, scale)
    lay = ListsLayout()
    _check(lib.kvpop_budget_lists_layout(ctypes.byref(sh), int(sinks), int(window), int(topk), ctypes.byref(lay)))
    return {f: getattr(lay, f) for f, _ in ListsLayout._fields_}


def attn_fwd_lse(q, k, v, cu_seqlens=None, scale: float = 0.0, need_output: bool = True,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 stream: Optional[torch.cuda.Stream] = None):
    """Causal attention forward with per-query LSE (kvpop_attn_fwd_lse)."""
    lib = load()
    _require_qkv(q, k, v)
    B, Hq, S, D = q.shape
    if lse is not None:
        _require("lse", lse, torch.float32, (B, Hq, S), placed=False)
    if out is not None:
        _require("out", out, q.dtype, q.shape, placed=False)
    _placed(q.device, ("q", q), ("k", k), ("v", v), ("lse", lse), ("out", out))
    made = []
    if lse is None:
        lse = torch.empty(B, Hq, S, dtype=torch.float32, device=q.device)
        made.append(lse)
    if need_output and out is None:
        out = torch.empty_like(q)
        made.append(out)
    packed = _Packed(cu_seqlens, q.device)
    sh = make_shape(q, k, packed, scale)
    _check(lib.kvpop_attn_fwd_lse(ctypes.byref(sh), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                  _dev(out), lse.data_ptr(), _stream_ptr(q, stream)))
    _retain(stream, packed.dev, *made)
    return out, lse


def future_target(q, k, lse, window: int, agg: Union[str, int] = "sum", mean_over_queries: bool = False,
                  eps: float = 0.0, cu_seqlens=None, scale: float = 0.0, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None):
    """Future-attention target by the transposed pass (kvpop_future_target)."""
    lib = load()
    a = _AGG_NAMES[agg] if isinstance(agg, str) else int(agg)
    _require_qkv(q, k)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _require("lse", lse, torch.float32, (B, Hq, S), placed=False)
    Hout = Hq if a == AGG_NONE else Hkv
    if out is not None:
        _require("out", out, torch.float32, (B, Hout, S), placed=False)
    if workspace is not None:
        _require("workspace", workspace, torch.uint8, placed=False)
    _placed(q.device, ("q", q), ("k", k), ("lse", lse), ("out", out), ("workspace", workspace))
    made = []
    if out is None:
        out = torch.empty(B, Hout, S, dtype=torch.float32, device=q.device)
        made.append(out)
    packed = _Packed(cu_seqlens, q.device)
    sh = make_shape(q, k, packed, scale)
    need = int(lib.kvpop_workspace_size(CALL_FUTURE_TARGET, ctypes.byref(sh), 0, window, 0))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        made.append(workspace)
    _check(lib.kvpop_future_target(ctypes.byref(sh), q.data_ptr(), k.data_ptr(), lse.data_ptr(), int(window),
                                   a, int(bool(mean_over_queries)), float(eps), out.data_ptr(),
                                   workspace.data_ptr(), workspace.numel(), _stream_ptr(q, stream)))
    _retain(stream, packed.dev, *made)
    return out


def future_target_noalloc(q, k, lse, window: int, out: torch.Tensor, agg: Union[str, int] = "sum",
                          mean_over_queries: bool = False, eps: float = 0.0, cu_seqlens=None, scale: float = 0.0,
                          stream: Optional[torch.cuda.Stream] = None):
    """kvpop_future_target_noalloc: the target without a workspace (the
    library's fixed per-GPU scratch is used).  `out` is caller-allocated
    ([B, Hkv, S] for SUM/MAX, [B, Hq, S] for NONE); with `cu_seqlens`, pass
    an int32 tensor already on the device's host side (its device copy is
    made here).  Calls overlapping on one GPU race."""
    lib = load()
    a = _AGG_NAMES[agg] if isinstance(agg, str) else int(agg)
    _require_qkv(q, k)
    B, Hq, S, D = q.shape
    Hout = Hq if a == AGG_NONE else k.shape[1]
    _require("lse", lse, torch.float32, (B, Hq, S), placed=False)
    _require("out", out, torch.float32, (B, Hout, S), placed=False)
    _placed(q.device, ("q", q), ("k", k), ("lse", lse), ("out", out))
    packed = _Packed(cu_seqlens, q.device)
    sh = make_shape(q, k, packed, scale)
    _check(lib.kvpop_future_target_noalloc(ctypes.byref(sh), q.data_ptr(), k.data_ptr(), lse.data_ptr(), int(window),
                                           a, int(bool(mean_over_queries)), float(eps), out.data_ptr(),
                                           _stream_ptr(q, stream)))
    _retain(stream, packed.dev)
    return out


def budget_mask_fwd(q, k, v, scores, sinks: int, window: int, topk: int, scale: float = 0.0,
                    return_rank_cutoff: bool = True, out: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    stream: Optional[torch.cuda.Stream] = None, cu_seqlens=None, need_output: bool = True):
    """Fixed-budget sparse attention forward (kvpop_budget_mask_fwd).

    Returns (o, lse, rank, cutoff); rank and cutoff are None unless asked for.
    With need_output=False only the mask is built (o and lse are None; the
    key lists stay in `workspace`).
    """
    lib = load()
    _require_qkv(q, k, v)
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    _require("scores", scores, torch.float32, (B, Hkv, S), placed=False)
    if out is not None:
        _require("out", out, q.dtype, q.shape, placed=False)
    if lse is not None:
        _require("lse", lse, torch.float32, (B, Hq, S), placed=False)
    if workspace is not None:
        _require("workspace", workspace, torch.uint8, placed=False)
    _placed(q.device, ("q", q), ("k", k), ("v", v), ("scores", scores), ("out", out), ("lse", lse),
            ("workspace", workspace))
    made = []
    if need_output and out is None:
        out = torch.empty_like(q)
        made.append(out)
    if need_output and lse is None:
        lse = torch.empty(B, Hq, S, dtype=torch.float32, device=q.device)
        made.append(lse)
    if not need_output:
        out = lse = None
    rank = cutoff = None
    if return_rank_cutoff:
        rank = torch.empty(B, Hkv, S, dtype=torch.int32, device=q.device)
        cutoff = torch.empty(B, Hkv, S, dtype=torch.int32, device=q.device)
        made += [rank, cutoff]
    packed = _Packed(cu_seqlens, q.device)
    sh = make_shape(q, k, packed, scale)
    need = int(lib.kvpop_workspace_size(CALL_BUDGET_MASK_FWD, ctypes.byref(sh), sinks, window, topk))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        made.append(workspace)
    _check(lib.kvpop_budget_mask_fwd(ctypes.byref(sh), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     scores.data_ptr(), int(sinks), int(window), int(topk), _dev(out),
                                     _dev(lse), _dev(rank), _dev(cutoff), workspace.data_ptr(),
                                     workspace.numel(), _stream_ptr(q, stream)))
    _retain(stream, packed.dev, *made)
    return out, lse, rank, cutoff


def teacher_labels(target: torch.Tensor, sinks: int, window: int, topk: int,
                   decay_lambda: Optional[torch.Tensor] = None, decay_step: int = 1,
                   return_ranks: bool = False, workspace: Optional[torch.Tensor] = None,
                   stream: Optional[torch.cuda.Stream] = None):
    """Teacher labels at the eviction boundary (kvpop_teacher_labels).

    target: [B, Hkv, S] fp32.  Returns (label, boundary) int32 [B, Hkv, S],
    plus (rank, brank) when return_ranks."""
    lib = load()
    _require("target", target, torch.float32)
    if target.dim() != 3:
        raise ValueError("target must be [B, Hkv, S]")
    B, H, S = target.shape
    if decay_lambda is not None:
        _require("decay_lambda", decay_lambda, torch.float32, (H,), target.device)
    if workspace is not None:
        _require("workspace", workspace, torch.uint8, device=target.device)
    label = torch.empty(B, H, S, dtype=torch.int32, device=target.device)
    bnd = torch.empty_like(label)
    rank = brank = None
    if return_ranks:
        rank = torch.empty_like(label)
        brank = torch.empty_like(label)
    need = int(lib.kvpop_teacher_workspace_size(B, H, S))
    made = [label, bnd, rank, brank]
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=target.device)
        made.append(workspace)
    _check(lib.kvpop_teacher_labels(B, H, S, target.data_ptr(), _dev(decay_lambda), int(decay_step), int(sinks),
                                    int(window), int(topk), label.data_ptr(), bnd.data_ptr(), _dev(rank),
                                    _dev(brank), workspace.data_ptr(), workspace.numel(),
                                    _stream_ptr(target, stream)))
    _retain(stream, *made)
    return (label, bnd, rank, brank) if return_ranks else (label, bnd)


def boundary_loss(pred: torch.Tensor, label: torch.Tensor, boundary: torch.Tensor, sinks: int, window: int,
                  topk: int, tau: float, weight: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream: Optional[torch.cuda.Stream] = None):
    """Boundary-aware retention loss and its gradient (kvpop_boundary_loss).

    Returns (loss per query position, d(sum loss)/d pred), both [B, Hkv, S] fp32."""
    lib = load()
    _require("pred", pred, torch.float32)
    if pred.dim() != 3:
        raise ValueError("pred must be [B, Hkv, S]")
    B, H, S = pred.shape
    _require("label", label, torch.int32, pred.shape, pred.device)
    _require("boundary", boundary, torch.int32, pred.shape, pred.device)
    if weight is not None:
        _require("weight", weight, torch.float32, pred.shape, pred.device)
    if workspace is not None:
        _require("workspace", workspace, torch.uint8, device=pred.device)
    loss = torch.empty_like(pred)
    grad = torch.empty_like(pred)
    need = int(lib.kvpop_boundary_loss_workspace_size(B, H, S))
    made = [loss, grad]
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=pred.device)
        made.append(workspace)
    _check(lib.kvpop_boundary_loss(B, H, S, pred.data_ptr(), label.data_ptr(), boundary.data_ptr(), int(sinks),
                                   int(window), int(topk), float(tau), _dev(weight), loss.data_ptr(),
                                   grad.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                   _stream_ptr(pred, stream)))
    _retain(stream, *made)
    return loss, grad


class DecodeCache:
    """Fixed-budget decode cache (kvpop_decode_init / kvpop_decode_step).

    Holds the caller-owned state tensor; step() appends the next token and
    returns the attention output and LSE of its query over the retained
    slots."""

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: torch.dtype,
                 sinks: int, window: int, topk: int, scale: float = 0.0, device="cuda",
                 stream: Optional[torch.cuda.Stream] = None):
        lib = load()
        self.shape = DecodeShape(batch, n_q_heads, n_kv_heads, head_dim,
                                 BF16 if dtype == torch.bfloat16 else F32, float(scale), sinks, window, topk)
        if dtype not in (torch.bfloat16, torch.float32):
            raise ValueError("dtype must be bfloat16 or float32")
        self.dtype = dtype
        need = int(lib.kvpop_decode_state_size(ctypes.byref(self.shape)))
        if need == 0:
            raise KvpopError(EINVAL, f"kvpop: invalid decode shape: {last_error()}")
        self.state = torch.empty(need, dtype=torch.uint8, device=device)
        self.position = 0
        s = stream if stream is not None else torch.cuda.current_stream(self.state.device)
        _check(lib.kvpop_decode_init(ctypes.byref(self.shape), self.state.data_ptr(), self.state.numel(),
                                     s.cuda_stream))
        _retain(stream, self.state)

    def step(self, q, k, v, score, out=None, lse=None, stream: Optional[torch.cuda.Stream] = None):
        """q [B,Hq,D], k, v [B,Hkv,D] (the cache dtype), score [B,Hkv] fp32."""
        lib = load()
        sh = self.shape
        dev = self.state.device
        _require("q", q, self.dtype, (sh.batch, sh.n_q_heads, sh.head_dim), dev)
        _require("k", k, self.dtype, (sh.batch, sh.n_kv_heads, sh.head_dim), dev)
        _require("v", v, self.dtype, (sh.batch, sh.n_kv_heads, sh.head_dim), dev)
        _require("score", score, torch.float32, (sh.batch, sh.n_kv_heads), dev)
        if out is not None:
            _require("out", out, self.dtype, q.shape, dev)
        if lse is not None:
            _require("lse", lse, torch.float32, (sh.batch, sh.n_q_heads), dev)
        made = []
        if out is None:
            out = torch.empty_like(q)
            made.append(out)
        if lse is None:
            lse = torch.empty(sh.batch, sh.n_q_heads, dtype=torch.float32, device=q.device)
            made.append(lse)
        _check(lib.kvpop_decode_step(ctypes.byref(sh), self.state.data_ptr(), self.state.numel(), self.position,
                                     q.data_ptr(), k.data_ptr(), v.data_ptr(), score.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), _stream_ptr(q, stream)))
        _retain(stream, *made)
        self.position += 1
        return out, lse


__all__ = ["load", "DocOffsets", "future_target_noalloc", "NOALLOC_SCRATCH_BYTES", "budget_lists_layout", "ListsLayout", "teacher_labels", "boundary_loss", "DecodeCache", "DecodeShape", "attn_fwd_lse", "future_target", "budget_mask_fwd", "workspace_size", "status_str",
           "last_error", "KvpopError", "Shape", "make_shape", "EXPORTS", "CUTOFF_ALL", "CUTOFF_NONE",
           "AGG_SUM", "AGG_MAX", "AGG_NONE", "CALL_FWD_LSE", "CALL_FUTURE_TARGET", "CALL_BUDGET_MASK_FWD",
           "OK", "EINVAL", "EUNSUPPORTED", "EWORKSPACE", "EHIP", "BF16", "F32"]

