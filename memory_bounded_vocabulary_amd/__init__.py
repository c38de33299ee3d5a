"""Memory-bounded vocabulary projection + cross-entropy for MI355X (gfx950).

Thin Python binding over the C-ABI library ``liblce.so`` (see include/lce.h).
Every step of the computation runs in the library's HIP kernels; this module
only marshals arguments: torch supplies device memory, data pointers and the
current stream. There is no fallback path: if the library is missing or no
GPU is present, the compute functions raise.

    loss, lse = forward(hidden, shards, targets)
    d_hidden, d_shards = backward(hidden, shards, targets, lse, dloss)

hidden: bf16 [N][H] cuda tensor; shards: list of P bf16 [V/P][H] cuda tensors
(shard s holds vocabulary ids [s*V/P, (s+1)*V/P)); targets: int32 [N].
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblce.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
REDUCTIONS = {"mean": 0, "sum": 1, "none": 2}
FLAG_ACCUMULATE_DX, FLAG_ACCUMULATE_DW, FLAG_BF16_GRADS, FLAG_KEEP_IGNORED_ROWS = 1, 2, 4, 8
EXPORTED = ("lce_workspace_bytes", "lce_forward", "lce_forward_noalloc", "lce_forward_noalloc_max_bytes",
            "lce_backward", "lce_state_bytes", "lce_ring_payload", "lce_fwd_round", "lce_fwd_finish", "lce_bwd_round",
            "lce_trace_enable", "lce_trace_collect", "lce_status_string", "lce_last_error", "lce_version")


class Dims(ctypes.Structure):
    _fields_ = [("n_tokens", ctypes.c_int64), ("hidden", ctypes.c_int64), ("vocab", ctypes.c_int64),
                ("n_shards", ctypes.c_int32), ("ignore_index", ctypes.c_int32),
                ("reduction", ctypes.c_int32), ("flags", ctypes.c_int32)]


class TraceEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("dropped", ctypes.c_int64),
                ("total_ms", ctypes.c_double), ("flops", ctypes.c_double), ("bytes", ctypes.c_double)]


class LceError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"lce status {status}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblce.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m memory_bounded_vocabulary_amd.build`")
    import torch  # noqa: F401  (loads the HIP runtime the library binds to)
    L = ctypes.CDLL(LIB_PATH)
    vp, i32p, f32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_float)
    dimp = ctypes.POINTER(Dims)
    L.lce_workspace_bytes.argtypes = [dimp]
    L.lce_workspace_bytes.restype = ctypes.c_size_t
    L.lce_forward.argtypes = [dimp, vp, ctypes.POINTER(vp), i32p, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.lce_forward.restype = ctypes.c_int
    L.lce_forward_noalloc.argtypes = [dimp, vp, ctypes.POINTER(vp), i32p, vp, vp, vp, vp, vp]
    L.lce_forward_noalloc.restype = ctypes.c_int
    L.lce_forward_noalloc_max_bytes.argtypes = []
    L.lce_forward_noalloc_max_bytes.restype = ctypes.c_size_t
    L.lce_backward.argtypes = [dimp, vp, ctypes.POINTER(vp), i32p, vp, vp, vp, vp, ctypes.POINTER(vp), vp,
                               ctypes.c_size_t, vp]
    L.lce_backward.restype = ctypes.c_int
    ci, sz = ctypes.c_int, ctypes.c_size_t
    L.lce_state_bytes.argtypes = [dimp]
    L.lce_state_bytes.restype = sz
    L.lce_ring_payload.argtypes = [dimp, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    L.lce_ring_payload.restype = ctypes.c_int
    L.lce_fwd_round.argtypes = [dimp, ci, ci, vp, vp, vp, vp, sz, vp]
    L.lce_fwd_round.restype = ctypes.c_int
    L.lce_fwd_finish.argtypes = [dimp, vp, vp, vp, vp, vp, sz, vp]
    L.lce_fwd_finish.restype = ctypes.c_int
    L.lce_bwd_round.argtypes = [dimp, ci, ci, vp, vp, vp, vp, vp, vp, vp, ci, vp, sz, vp]
    L.lce_bwd_round.restype = ctypes.c_int
    L.lce_trace_enable.argtypes = [ctypes.c_int]
    L.lce_trace_enable.restype = ctypes.c_int
    L.lce_trace_collect.argtypes = [ctypes.POINTER(TraceEntry), ctypes.c_int]
    L.lce_trace_collect.restype = ctypes.c_int
    L.lce_status_string.argtypes = [ctypes.c_int]
    L.lce_status_string.restype = ctypes.c_char_p
    L.lce_last_error.argtypes = []
    L.lce_last_error.restype = ctypes.c_char_p
    L.lce_version.argtypes = []
    L.lce_version.restype = ctypes.c_int
    del f32p
    _lib = L
    return L


def make_dims(n_tokens: int, hidden: int, vocab: int, n_shards: int, ignore_index: int = -100,
              reduction: str = "mean", flags: int = 0) -> Dims:
    return Dims(n_tokens, hidden, vocab, n_shards, ignore_index, REDUCTIONS[reduction], flags)


def workspace_bytes(n_tokens: int, hidden: int, vocab: int, n_shards: int, ignore_index: int = -100,
                    reduction: str = "mean", flags: int = 0) -> int:
    d = make_dims(n_tokens, hidden, vocab, n_shards, ignore_index, reduction, flags)
    return int(lib().lce_workspace_bytes(ctypes.byref(d)))


def _check(status: int) -> None:
    if status != OK:
        L = lib()
        raise LceError(status, f"{L.lce_status_string(status).decode()}: {L.lce_last_error().decode()}")


def _ptr_array(ptrs: Sequence[int]):
    return (ctypes.c_void_p * len(ptrs))(*ptrs)


def _order_array(order: Optional[Sequence[int]]):
    if order is None:
        return None
    return (ctypes.c_int32 * len(order))(*[int(o) for o in order])


def _stream(stream) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _require_cuda(*tensors) -> None:
    for t in tensors:
        if not t.is_cuda:
            raise ValueError("lce runs on the GPU only: every tensor must be a cuda tensor")


def _check_inputs(hidden, shards, targets, lse=None) -> None:
    """Dtypes, shapes and contiguity the C ABI assumes (it sees raw pointers)."""
    import torch
    if hidden.dim() != 2 or hidden.dtype != torch.bfloat16 or not hidden.is_contiguous():
        raise ValueError("hidden must be a contiguous bf16 [N, H] tensor")
    if len(shards) < 1:
        raise ValueError("at least one shard is needed")
    vs = shards[0].shape[0] if shards[0].dim() == 2 else -1
    for s in shards:
        if s.dim() != 2 or s.dtype != torch.bfloat16 or not s.is_contiguous() or tuple(s.shape) != (vs, hidden.shape[1]):
            raise ValueError("every shard must be a contiguous bf16 [V/P, H] tensor of the same shape")
    if targets.dim() != 1 or targets.dtype != torch.int32 or not targets.is_contiguous() or \
            targets.shape[0] != hidden.shape[0]:
        raise ValueError("targets must be a contiguous int32 [N] tensor")
    if lse is not None and (lse.dim() != 1 or lse.dtype != torch.float32 or not lse.is_contiguous() or
                            lse.shape[0] != hidden.shape[0]):
        raise ValueError("lse must be a contiguous fp32 [N] tensor (from forward)")


def state_bytes(dims: Dims) -> int:
    """Leading workspace bytes that carry state between the calls of a round sequence."""
    return int(lib().lce_state_bytes(ctypes.byref(dims)))


def ring_payload(dims: Dims) -> Tuple[str, int, int]:
    """('weights' | 'activations', weight bytes per hop, activation bytes per hop)."""
    w, x = ctypes.c_size_t(), ctypes.c_size_t()
    r = lib().lce_ring_payload(ctypes.byref(dims), ctypes.byref(w), ctypes.byref(x))
    if r < 0:
        _check(r)
    return ("activations" if r == 1 else "weights"), int(w.value), int(x.value)


def alloc_workspace(n_tokens: int, hidden: int, vocab: int, n_shards: int, device=None, ignore_index: int = -100,
                    reduction: str = "mean", flags: int = 0):
    import torch
    nbytes = workspace_bytes(n_tokens, hidden, vocab, n_shards, ignore_index, reduction, flags)
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device or "cuda")


def forward(hidden, shards: Sequence, targets, ignore_index: int = -100, order: Optional[Sequence[int]] = None,
            reduction: str = "mean", workspace=None, token_loss: bool = False, stream=None):
    """Loss and saved normalizer; returns (loss, lse) or (loss, lse, token_loss).

    reduction "none" always returns the token losses (loss is then their sum)."""
    import torch
    _check_inputs(hidden, shards, targets)
    _require_cuda(hidden, targets, *shards)
    n, h = hidden.shape
    p = len(shards)
    v = p * shards[0].shape[0]
    d = make_dims(n, h, v, p, ignore_index, reduction)
    if workspace is None:
        workspace = alloc_workspace(n, h, v, p, hidden.device, ignore_index, reduction)
    _require_cuda(workspace)
    token_loss = token_loss or reduction == "none"
    loss = torch.empty((), dtype=torch.float32, device=hidden.device)
    lse = torch.empty(n, dtype=torch.float32, device=hidden.device)
    tl = torch.empty(n, dtype=torch.float32, device=hidden.device) if token_loss else None
    st = lib().lce_forward(ctypes.byref(d), hidden.data_ptr(), _ptr_array([s.data_ptr() for s in shards]),
                           _order_array(order), targets.data_ptr(), loss.data_ptr(), lse.data_ptr(),
                           tl.data_ptr() if tl is not None else None, workspace.data_ptr(),
                           _nbytes(workspace), _stream(stream))
    _check(st)
    return (loss, lse, tl) if token_loss else (loss, lse)


def forward_noalloc(hidden, shards: Sequence, targets, loss, lse, token_loss=None, ignore_index: int = -100,
                    order: Optional[Sequence[int]] = None, reduction: str = "mean", stream=None) -> None:
    """lce_forward_noalloc: the forward into caller-given outputs (loss fp32 [],
    lse fp32 [N], token_loss fp32 [N] or None), with the library's built-in
    scratch instead of a workspace; allocates nothing."""
    import torch
    _check_inputs(hidden, shards, targets, lse)
    n = hidden.shape[0]
    if loss.dtype != torch.float32 or loss.numel() != 1:
        raise ValueError("loss must be a one-element fp32 tensor")
    if token_loss is not None and (token_loss.dtype != torch.float32 or tuple(token_loss.shape) != (n,) or
                                   not token_loss.is_contiguous()):
        raise ValueError("token_loss must be a contiguous fp32 [N] tensor")
    _require_cuda(hidden, targets, loss, lse, *shards, *([token_loss] if token_loss is not None else []))
    p = len(shards)
    d = make_dims(n, hidden.shape[1], p * shards[0].shape[0], p, ignore_index, reduction)
    _check(lib().lce_forward_noalloc(ctypes.byref(d), hidden.data_ptr(), _ptr_array([s.data_ptr() for s in shards]),
                                     _order_array(order), targets.data_ptr(), loss.data_ptr(), lse.data_ptr(),
                                     token_loss.data_ptr() if token_loss is not None else None, _stream(stream)))


def backward(hidden, shards: Sequence, targets, lse, dloss, ignore_index: int = -100,
             order: Optional[Sequence[int]] = None, reduction: str = "mean", workspace=None,
             d_hidden=None, d_shards: Optional[List] = None, accumulate: bool = False,
             grad_dtype=None, keep_ignored_rows: bool = False, stream=None) -> Tuple[object, List]:
    """Gradients (d_hidden [N][H], [d_shard [V/P][H]]) of the loss scaled by dloss.

    dloss: scalar (mean / sum) or fp32 [N] (reduction "none"). grad_dtype:
    torch.float32 (default) or torch.bfloat16 (accumulated in fp32, rounded
    once). accumulate: add into the given d_hidden / d_shards.
    keep_ignored_rows: run over every token (no gathered copy of the hidden
    rows in the workspace: less memory, same results)."""
    import torch
    _check_inputs(hidden, shards, targets, lse)
    _require_cuda(hidden, targets, lse, *shards)
    n, h = hidden.shape
    p = len(shards)
    vs = shards[0].shape[0]
    grad_dtype = torch.float32 if grad_dtype is None else grad_dtype
    if grad_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("grad_dtype must be torch.float32 or torch.bfloat16")
    flags = FLAG_BF16_GRADS if grad_dtype == torch.bfloat16 else 0
    if accumulate:
        if d_hidden is None or d_shards is None:
            raise ValueError("accumulate needs the d_hidden and d_shards to add into")
        flags |= FLAG_ACCUMULATE_DX | FLAG_ACCUMULATE_DW
    if keep_ignored_rows:
        flags |= FLAG_KEEP_IGNORED_ROWS
    d = make_dims(n, h, p * vs, p, ignore_index, reduction, flags)
    if workspace is None:
        workspace = alloc_workspace(n, h, p * vs, p, hidden.device, ignore_index, reduction, flags)
    if not torch.is_tensor(dloss):
        dloss = torch.tensor(float(dloss), dtype=torch.float32, device=hidden.device)
    if reduction == "none" and dloss.numel() != n:
        raise ValueError("reduction 'none' takes a per-token dloss of N elements")
    if reduction != "none" and dloss.numel() != 1:
        raise ValueError("reductions 'mean' and 'sum' take one dloss value")
    if dloss.dtype != torch.float32 or not dloss.is_contiguous():
        raise ValueError("dloss must be a contiguous fp32 tensor")
    _require_cuda(dloss)
    if d_hidden is None:
        d_hidden = torch.empty((n, h), dtype=grad_dtype, device=hidden.device)
    if d_shards is None:
        d_shards = [torch.empty((vs, h), dtype=grad_dtype, device=hidden.device) for _ in range(p)]
    for t in (d_hidden, *d_shards):
        if t.dtype != grad_dtype or not t.is_contiguous():
            raise ValueError(f"gradient buffers must be contiguous {grad_dtype}")
    if tuple(d_hidden.shape) != (n, h) or len(d_shards) != p or any(tuple(g.shape) != (vs, h) for g in d_shards):
        raise ValueError("gradient buffers must match hidden [N, H] and the shards [V/P, H]")
    _require_cuda(workspace, d_hidden, *d_shards)
    st = lib().lce_backward(ctypes.byref(d), hidden.data_ptr(), _ptr_array([s.data_ptr() for s in shards]),
                            _order_array(order), targets.data_ptr(), lse.data_ptr(), dloss.data_ptr(),
                            d_hidden.data_ptr(), _ptr_array([g.data_ptr() for g in d_shards]),
                            workspace.data_ptr(), _nbytes(workspace), _stream(stream))
    _check(st)
    return d_hidden, d_shards


def _check_round_tensors(dims: Dims, hidden, shard, targets, lse=None) -> None:
    """The per-round calls take their sizes from `dims`: the tensors must agree with it."""
    _check_inputs(hidden, [shard], targets, lse)
    n, h = hidden.shape
    if dims.n_shards < 1 or dims.vocab % dims.n_shards:
        raise ValueError("dims.vocab must be a multiple of dims.n_shards")
    if int(dims.n_tokens) != n or int(dims.hidden) != h:
        raise ValueError(f"dims (n_tokens={dims.n_tokens}, hidden={dims.hidden}) do not match hidden {tuple(hidden.shape)}")
    if int(dims.vocab) // int(dims.n_shards) != shard.shape[0]:
        raise ValueError(f"dims give {dims.vocab // dims.n_shards} rows per shard; the shard has {shard.shape[0]}")


def _check_workspace(dims: Dims, workspace) -> None:
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    if _nbytes(workspace) < int(lib().lce_workspace_bytes(ctypes.byref(dims))):
        raise ValueError("workspace is smaller than workspace_bytes(dims)")


def _grad_dtype(dims: Dims):
    import torch
    return torch.bfloat16 if int(dims.flags) & FLAG_BF16_GRADS else torch.float32


def fwd_round(dims: Dims, round_: int, shard_index: int, hidden, shard, targets, workspace, stream=None) -> None:
    """One forward ring round: fold `shard` (id `shard_index`) into the state held in `workspace`."""
    _check_round_tensors(dims, hidden, shard, targets)
    _check_workspace(dims, workspace)
    _require_cuda(hidden, shard, targets, workspace)
    _check(lib().lce_fwd_round(ctypes.byref(dims), int(round_), int(shard_index), hidden.data_ptr(),
                               shard.data_ptr(), targets.data_ptr(), workspace.data_ptr(), _nbytes(workspace),
                               _stream(stream)))


def fwd_finish(dims: Dims, targets, workspace, token_loss: bool = False, stream=None):
    """After the rounds: (loss, lse) or (loss, lse, token_loss) from the state in `workspace`."""
    import torch
    n = int(dims.n_tokens)
    if targets.dim() != 1 or targets.dtype != torch.int32 or not targets.is_contiguous() or targets.shape[0] != n:
        raise ValueError("targets must be a contiguous int32 [dims.n_tokens] tensor")
    _check_workspace(dims, workspace)
    _require_cuda(targets, workspace)
    loss = torch.empty((), dtype=torch.float32, device=targets.device)
    lse = torch.empty(n, dtype=torch.float32, device=targets.device)
    tl = torch.empty(n, dtype=torch.float32, device=targets.device) if token_loss else None
    _check(lib().lce_fwd_finish(ctypes.byref(dims), targets.data_ptr(), loss.data_ptr(), lse.data_ptr(),
                                tl.data_ptr() if tl is not None else None, workspace.data_ptr(),
                                _nbytes(workspace), _stream(stream)))
    return (loss, lse, tl) if token_loss else (loss, lse)


def bwd_round(dims: Dims, round_: int, shard_index: int, hidden, shard, targets, lse, dloss, d_hidden, d_shard,
              accumulate_dw: bool, workspace, stream=None) -> None:
    """One backward ring round: d_hidden (+)= G W_shard, d_shard (+)= G^T X for this shard.

    Gradient buffers are fp32, or bf16 when dims.flags has FLAG_BF16_GRADS;
    dloss is one fp32 value (mean / sum) or fp32 [N] (reduction "none")."""
    import torch
    _check_round_tensors(dims, hidden, shard, targets, lse)
    if lse is None:
        raise ValueError("lse (from the forward) is required")
    gdt = _grad_dtype(dims)
    n, h = hidden.shape
    for name, t, shape in (("d_hidden", d_hidden, (n, h)), ("d_shard", d_shard, tuple(shard.shape))):
        if t.dtype != gdt or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {gdt} tensor of shape {shape}")
    want = n if int(dims.reduction) == REDUCTIONS["none"] else 1
    if dloss.dtype != torch.float32 or dloss.numel() != want or not dloss.is_contiguous():
        raise ValueError(f"dloss must be a contiguous fp32 tensor of {want} element(s)")
    _check_workspace(dims, workspace)
    _require_cuda(hidden, shard, targets, lse, dloss, d_hidden, d_shard, workspace)
    _check(lib().lce_bwd_round(ctypes.byref(dims), int(round_), int(shard_index), hidden.data_ptr(),
                               shard.data_ptr(), targets.data_ptr(), lse.data_ptr(), dloss.data_ptr(),
                               d_hidden.data_ptr(), d_shard.data_ptr(), int(bool(accumulate_dw)),
                               workspace.data_ptr(), _nbytes(workspace), _stream(stream)))


def trace_enable(capacity: int) -> None:
    """Bracket each kernel launch of this thread's calls with HIP events (0 disables)."""
    _check(lib().lce_trace_enable(int(capacity)))


def trace_collect() -> List[dict]:
    """Wait for the traced launches; per kernel kind: launches, ms, algorithmic flops and bytes."""
    buf = (TraceEntry * 32)()
    n = lib().lce_trace_collect(buf, 32)
    if n < 0:
        _check(n)
    return [dict(name=e.name.decode(), launches=int(e.launches), dropped=int(e.dropped), total_ms=e.total_ms,
                 flops=e.flops, bytes=e.bytes) for e in buf[:min(n, 32)]]


def version() -> Tuple[int, int]:
    v = lib().lce_version()
    return v >> 16, v & 0xFFFF
