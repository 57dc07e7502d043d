"""Blocked vocabulary-projection cross-entropy on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libvpce.so`` (declared in
``include/vpce.h``). This module only marshals arguments: every step of the
computation runs in the library's HIP kernels. PyTorch supplies device memory
(so its allocator accounts for every byte, workspace included) and the current
stream. There is no CPU path: if the library is missing, every call raises.

    loss, lse = forward(H, W, labels, R)
    dH, dW = backward(H, W, labels, lse, dloss, R)

``vocabulary_projection_cross_amd.autograd.cross_entropy`` wraps the pair as
a differentiable scalar loss for torch.autograd.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["forward", "backward", "workspace_bytes", "plan", "ring_mode",
           "forward_noalloc", "forward_noalloc_bytes", "NOALLOC_SCRATCH_BYTES",
           "forward_traced", "backward_traced", "KERNEL_KINDS",
           "state_init", "shard_fold", "state_finish", "shard_backward",
           "VPCEError", "library_path", "IGNORE_INDEX", "VPCE_BF16",
           "VPCE_F32", "MOVE_WEIGHTS", "MOVE_ACTIVATIONS"]

IGNORE_INDEX = -100
VPCE_BF16 = 0
VPCE_F32 = 1
MOVE_WEIGHTS = 0
MOVE_ACTIVATIONS = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "libvpce.so")
_lib = None


class VPCEError(RuntimeError):
    pass


def library_path() -> str:
    return _LIBPATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIBPATH):
        raise VPCEError(
            "libvpce.so is not built; run "
            "`python -m vocabulary_projection_cross_amd.build`")
    lib = ctypes.CDLL(_LIBPATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, \
        ctypes.c_size_t
    lib.vpce_workspace_bytes.restype = sz
    lib.vpce_workspace_bytes.argtypes = [i64, i64, i64, i32, i32]
    lib.vpce_workspace_bytes_chunk.restype = sz
    lib.vpce_workspace_bytes_chunk.argtypes = [i64, i64, i64, i32, i32, i64]
    lib.vpce_plan.restype = i32
    lib.vpce_plan.argtypes = [i64, i64, i64, i32, i32, sz,
                              ctypes.POINTER(i64), ctypes.POINTER(sz),
                              ctypes.POINTER(sz)]
    lib.vpce_forward.restype = i32
    lib.vpce_forward.argtypes = [vp, vp, vp, i64, i64, i64, i32, i64, i32,
                                 vp, vp, vp, sz, vp]
    lib.vpce_forward_noalloc.restype = i32
    lib.vpce_forward_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, i32, i64,
                                         i32, vp, vp, vp]
    lib.vpce_forward_noalloc_bytes.restype = sz
    lib.vpce_forward_noalloc_bytes.argtypes = [i64, i64, i64, i32, i32]
    for name, n_args in (("vpce_forward_traced", 14),
                         ("vpce_backward_traced", 16)):
        f = getattr(lib, name)
        f.restype = i32
        base = (lib.vpce_forward.argtypes if n_args == 14
                else [vp, vp, vp, vp, vp, i64, i64, i64, i32, i64, i32, vp,
                      vp, vp, sz, vp])
        f.argtypes = list(base) + [ctypes.POINTER(vp), i32,
                                   ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.vpce_backward.restype = i32
    lib.vpce_backward.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i64,
                                  i32, vp, vp, vp, sz, vp]
    lib.vpce_ring_mode.restype = i32
    lib.vpce_ring_mode.argtypes = [i64, i64, i64, i32, i32,
                                   ctypes.POINTER(i32), ctypes.POINTER(sz),
                                   ctypes.POINTER(sz)]
    lib.vpce_state_init.restype = i32
    lib.vpce_state_init.argtypes = [vp, i64, vp]
    lib.vpce_shard_fold.restype = i32
    lib.vpce_shard_fold.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                    i32, vp, vp, sz, vp]
    lib.vpce_state_finish.restype = i32
    lib.vpce_state_finish.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, sz,
                                      vp]
    lib.vpce_shard_backward.restype = i32
    lib.vpce_shard_backward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                        i64, i64, i64, i32, vp, vp, vp, sz, vp]
    lib.vpce_status_string.restype = ctypes.c_char_p
    lib.vpce_status_string.argtypes = [i32]
    _lib = lib
    return lib


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return VPCE_BF16
    if t == torch.float32:
        return VPCE_F32
    raise VPCEError(f"unsupported dtype {t}; expected bfloat16 or float32")


def _check(status: int):
    if status != 0:
        msg = _load().vpce_status_string(status).decode()
        raise VPCEError(f"vpce status {status}: {msg}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _validate(H, W, labels):
    for name, t in (("H", H), ("W", W), ("labels", labels)):
        if not isinstance(t, torch.Tensor):
            raise VPCEError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise VPCEError(f"{name} must be on a GPU device")
        if not t.is_contiguous():
            raise VPCEError(f"{name} must be contiguous")
    if H.dim() != 2 or W.dim() != 2 or labels.dim() != 1:
        raise VPCEError("expected H [N, d], W [V, d], labels [N]")
    if H.shape[1] != W.shape[1] or labels.shape[0] != H.shape[0]:
        raise VPCEError("shape mismatch between H, W and labels")
    if H.dtype != W.dtype:
        raise VPCEError("H and W must have the same dtype")
    if labels.dtype != torch.int64:
        raise VPCEError("labels must be int64")
    if not (H.device == W.device == labels.device):
        raise VPCEError("H, W and labels must be on the same device")


def workspace_bytes(N: int, d: int, V: int, R: int,
                    dtype: torch.dtype = torch.bfloat16,
                    chunk_cols: Optional[int] = None) -> int:
    """Workspace bytes for forward + backward (0 for invalid arguments): at
    the widest backward chunk, or at chunk_cols (a multiple of 256 in
    [256, 8192])."""
    if chunk_cols is None:
        return int(_load().vpce_workspace_bytes(N, d, V, R,
                                                _dtype_code(dtype)))
    return int(_load().vpce_workspace_bytes_chunk(N, d, V, R,
                                                  _dtype_code(dtype),
                                                  chunk_cols))


def plan(N: int, d: int, V: int, R: int, budget_bytes: int,
         dtype: torch.dtype = torch.bfloat16) -> dict:
    """The widest backward chunk whose step fits in budget_bytes of device
    memory (the caller's inputs and outputs plus one shared workspace), with
    the workspace size and the exact peak device bytes of a forward +
    backward step, known before anything is launched."""
    lib = _load()
    c = ctypes.c_int64(0)
    ws = ctypes.c_size_t(0)
    peak = ctypes.c_size_t(0)
    _check(lib.vpce_plan(N, d, V, R, _dtype_code(dtype), budget_bytes,
                         ctypes.byref(c), ctypes.byref(ws),
                         ctypes.byref(peak)))
    return {"chunk_cols": int(c.value), "workspace_bytes": int(ws.value),
            "peak_bytes": int(peak.value)}


def _workspace(H, W, R, workspace):
    """The caller's workspace (the library checks that it is large enough
    and fits the backward chunk to it), or a new one of the full size."""
    if workspace is not None:
        if (workspace.device != H.device or not workspace.is_contiguous()
                or workspace.dtype != torch.uint8):
            raise VPCEError("workspace must be a contiguous uint8 tensor on "
                            "H's device")
        return workspace
    need = workspace_bytes(H.shape[0], H.shape[1], W.shape[0], R, H.dtype)
    if need == 0:
        raise VPCEError("invalid shape for the vocabulary-projection CE")
    return torch.empty(need, dtype=torch.uint8, device=H.device)


def forward(H: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, R: int,
            ignore_index: int = IGNORE_INDEX,
            workspace: Optional[torch.Tensor] = None
            ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Mean cross-entropy of softmax(H W^T) against labels, computed shard by
    shard with an online log-sum-exp. Returns (loss [] fp32, lse [N] fp32)."""
    _validate(H, W, labels)
    lib = _load()
    N, d = H.shape
    V = W.shape[0]
    ws = _workspace(H, W, R, workspace)
    loss = torch.empty((), dtype=torch.float32, device=H.device)
    lse = torch.empty(N, dtype=torch.float32, device=H.device)
    stream = torch.cuda.current_stream(H.device).cuda_stream
    with torch.cuda.device(H.device):
        st = lib.vpce_forward(_ptr(H), _ptr(W), _ptr(labels), N, d, V, R,
                              ignore_index, _dtype_code(H.dtype), _ptr(loss),
                              _ptr(lse), _ptr(ws), ws.numel(),
                              ctypes.c_void_p(stream))
    _check(st)
    return loss, lse


NOALLOC_SCRATCH_BYTES = 64 << 20


def forward_noalloc(H: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                    R: int, loss: torch.Tensor, lse: torch.Tensor,
                    ignore_index: int = IGNORE_INDEX) -> None:
    """vpce_forward_noalloc: the forward into the caller's loss [] and lse
    [N] (fp32, on H's device), with the library's static device scratch in
    place of a workspace; nothing is allocated, here or in the library.
    Calls on one GPU that overlap in time race on that scratch."""
    _validate(H, W, labels)
    N, d = H.shape
    for name, t, n in (("loss", loss, 1), ("lse", lse, N)):
        if (t.device != H.device or t.dtype != torch.float32
                or t.numel() != n or not t.is_contiguous()):
            raise VPCEError(f"{name} must be a contiguous fp32 tensor of {n} "
                            "elements on H's device")
    with torch.cuda.device(H.device):
        st = _load().vpce_forward_noalloc(
            _ptr(H), _ptr(W), _ptr(labels), N, d, W.shape[0], R,
            ignore_index, _dtype_code(H.dtype), _ptr(loss), _ptr(lse),
            _stream(H))
    _check(st)


def forward_noalloc_bytes(N: int, d: int, V: int, R: int,
                          dtype: torch.dtype = torch.bfloat16) -> int:
    """Scratch bytes vpce_forward_noalloc needs (at most
    NOALLOC_SCRATCH_BYTES is available); 0 for invalid arguments."""
    return int(_load().vpce_forward_noalloc_bytes(N, d, V, R,
                                                  _dtype_code(dtype)))


def backward(H: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
             lse: torch.Tensor, dloss: Optional[torch.Tensor], R: int,
             ignore_index: int = IGNORE_INDEX,
             workspace: Optional[torch.Tensor] = None
             ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gradients of the mean loss times dloss (a device scalar; None = 1).
    Returns (dH [N, d] fp32, dW [V, d] fp32)."""
    _validate(H, W, labels)
    lib = _load()
    N, d = H.shape
    V = W.shape[0]
    if (lse.device != H.device or lse.dtype != torch.float32
            or lse.numel() != N or not lse.is_contiguous()):
        raise VPCEError("lse must be a contiguous fp32 [N] tensor on H's "
                        "device")
    if dloss is not None:
        if (dloss.device != H.device or dloss.dtype != torch.float32
                or dloss.numel() != 1):
            raise VPCEError("dloss must be a one-element fp32 tensor on H's "
                            "device")
        dloss = dloss.contiguous()
    ws = _workspace(H, W, R, workspace)
    dH = torch.empty((N, d), dtype=torch.float32, device=H.device)
    dW = torch.empty((V, d), dtype=torch.float32, device=H.device)
    stream = torch.cuda.current_stream(H.device).cuda_stream
    with torch.cuda.device(H.device):
        st = lib.vpce_backward(_ptr(H), _ptr(W), _ptr(labels), _ptr(lse),
                               _ptr(dloss), N, d, V, R, ignore_index,
                               _dtype_code(H.dtype), _ptr(dH), _ptr(dW),
                               _ptr(ws), ws.numel(), ctypes.c_void_p(stream))
    _check(st)
    return dH, dW


# ---- timed variants (measurement) -----------------------------------------

KERNEL_KINDS = {1: "forward_tile", 2: "merge", 3: "recompute",
                4: "products", 7: "other"}


def _trace_args(events):
    """ctypes arguments for an event list: every event must already exist
    (torch creates an event on its first record)."""
    handles = [int(e.cuda_event) for e in events]
    if len(handles) % 2 or any(h == 0 for h in handles):
        raise VPCEError("events must be an even number of recorded "
                        "torch.cuda.Event objects")
    n = len(handles) // 2
    arr = (ctypes.c_void_p * max(1, len(handles)))(*handles)
    kinds = (ctypes.c_int32 * max(1, n))()
    return arr, n, kinds, ctypes.c_int32(0)


def forward_traced(H, W, labels, R, events, ignore_index=IGNORE_INDEX,
                   workspace=None):
    """vpce_forward_traced: forward() plus timing events around its kernel
    launches (pair i = events[2i], events[2i+1]). Returns (loss, lse,
    [kind of each bracketed launch], number of launches)."""
    _validate(H, W, labels)
    lib = _load()
    N, d = H.shape
    V = W.shape[0]
    ws = _workspace(H, W, R, workspace)
    loss = torch.empty((), dtype=torch.float32, device=H.device)
    lse = torch.empty(N, dtype=torch.float32, device=H.device)
    arr, n, kinds, used = _trace_args(events)
    with torch.cuda.device(H.device):
        st = lib.vpce_forward_traced(
            _ptr(H), _ptr(W), _ptr(labels), N, d, V, R, ignore_index,
            _dtype_code(H.dtype), _ptr(loss), _ptr(lse), _ptr(ws), ws.numel(),
            _stream(H), arr, n, kinds, ctypes.byref(used))
    _check(st)
    return loss, lse, [KERNEL_KINDS[kinds[i]] for i in
                       range(min(n, used.value))], int(used.value)


def backward_traced(H, W, labels, lse, dloss, R, events,
                    ignore_index=IGNORE_INDEX, workspace=None):
    """vpce_backward_traced: backward() plus timing events around its kernel
    launches. Returns (dH, dW, [kind of each bracketed launch], number of
    launches)."""
    _validate(H, W, labels)
    lib = _load()
    N, d = H.shape
    V = W.shape[0]
    ws = _workspace(H, W, R, workspace)
    dH = torch.empty((N, d), dtype=torch.float32, device=H.device)
    dW = torch.empty((V, d), dtype=torch.float32, device=H.device)
    arr, n, kinds, used = _trace_args(events)
    with torch.cuda.device(H.device):
        st = lib.vpce_backward_traced(
            _ptr(H), _ptr(W), _ptr(labels), _ptr(lse), _ptr(dloss), N, d, V,
            R, ignore_index, _dtype_code(H.dtype), _ptr(dH), _ptr(dW),
            _ptr(ws), ws.numel(), _stream(H), arr, n, kinds,
            ctypes.byref(used))
    _check(st)
    return dH, dW, [KERNEL_KINDS[kinds[i]] for i in
                    range(min(n, used.value))], int(used.value)


# ---- shard-level calls: one batch meets one vocabulary shard ---------------

def ring_mode(N: int, d: int, V: int, R: int,
              dtype: torch.dtype = torch.bfloat16) -> dict:
    """Which tensor a ring of R ranks with N tokens each sends per hop
    (MOVE_WEIGHTS or MOVE_ACTIVATIONS) and both per-hop payloads in bytes."""
    lib = _load()
    mode = ctypes.c_int32(-1)
    act = ctypes.c_size_t(0)
    wts = ctypes.c_size_t(0)
    _check(lib.vpce_ring_mode(N, d, V, R, _dtype_code(dtype),
                              ctypes.byref(mode), ctypes.byref(act),
                              ctypes.byref(wts)))
    return {"mode": int(mode.value), "activation_bytes": int(act.value),
            "weight_bytes": int(wts.value)}


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _shard_workspace(H, V, workspace):
    if workspace is not None:
        return workspace
    need = workspace_bytes(H.shape[0], H.shape[1], V, 1, H.dtype)
    if need == 0:
        raise VPCEError("invalid shape for the vocabulary-projection CE")
    return torch.empty(need, dtype=torch.uint8, device=H.device)


def _check_state(state, N, device):
    if (state.device != device or state.dtype != torch.float32
            or state.numel() != 3 * N or not state.is_contiguous()):
        raise VPCEError("state must be a contiguous fp32 [3, N] tensor on H's "
                        "device")


def state_init(N: int, device) -> torch.Tensor:
    """A new empty running state [3, N] (m = -inf, s = 0, t = NaN)."""
    state = torch.empty((3, N), dtype=torch.float32, device=device)
    with torch.cuda.device(state.device):
        _check(_load().vpce_state_init(_ptr(state), N, _stream(state)))
    return state


def shard_fold(H: torch.Tensor, W_shard: torch.Tensor, labels: torch.Tensor,
               V: int, v_begin: int, state: torch.Tensor,
               ignore_index: int = IGNORE_INDEX,
               workspace: Optional[torch.Tensor] = None) -> None:
    """Fold vocabulary rows [v_begin, v_begin + len(W_shard)) into the
    batch's running state, in place."""
    _validate(H, W_shard, labels)
    N, d = H.shape
    _check_state(state, N, H.device)
    ws = _shard_workspace(H, V, workspace)
    with torch.cuda.device(H.device):
        st = _load().vpce_shard_fold(
            _ptr(H), _ptr(W_shard), _ptr(labels), N, d, V, v_begin,
            W_shard.shape[0], ignore_index, _dtype_code(H.dtype), _ptr(state),
            _ptr(ws), ws.numel(), _stream(H))
    _check(st)


def state_finish(state: torch.Tensor, labels: torch.Tensor,
                 totals: torch.Tensor, ignore_index: int = IGNORE_INDEX,
                 workspace: Optional[torch.Tensor] = None
                 ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Close a batch that has met every shard: returns lse [N] and the mean
    loss over every batch accumulated into totals (fp64 [2], in place)."""
    N = labels.shape[0]
    _check_state(state, N, labels.device)
    if (totals.device != labels.device or totals.dtype != torch.float64
            or totals.numel() != 2):
        raise VPCEError("totals must be an fp64 [2] tensor on the device")
    if labels.dtype != torch.int64 or not labels.is_contiguous():
        raise VPCEError("labels must be contiguous int64")
    lse = torch.empty(N, dtype=torch.float32, device=labels.device)
    loss = torch.empty((), dtype=torch.float32, device=labels.device)
    ws = workspace if workspace is not None else torch.empty(
        4096 + 16 * N, dtype=torch.uint8, device=labels.device)
    with torch.cuda.device(labels.device):
        st = _load().vpce_state_finish(
            _ptr(state), _ptr(labels), N, ignore_index, _ptr(lse),
            _ptr(totals), _ptr(loss), _ptr(ws), ws.numel(), _stream(labels))
    _check(st)
    return lse, loss


def shard_backward(H: torch.Tensor, W_shard: torch.Tensor,
                   labels: torch.Tensor, lse: torch.Tensor,
                   totals: torch.Tensor, dloss: Optional[torch.Tensor],
                   V: int, v_begin: int, dH: torch.Tensor,
                   dW_shard: torch.Tensor, ignore_index: int = IGNORE_INDEX,
                   workspace: Optional[torch.Tensor] = None) -> None:
    """Accumulate one (batch, shard) meeting's gradients into dH [N, d] and
    dW_shard [len(W_shard), d] (fp32, in place)."""
    _validate(H, W_shard, labels)
    N, d = H.shape
    for name, t, shape in (("dH", dH, (N, d)),
                           ("dW_shard", dW_shard, tuple(W_shard.shape))):
        if (t.device != H.device or t.dtype != torch.float32
                or tuple(t.shape) != shape or not t.is_contiguous()):
            raise VPCEError(f"{name} must be a contiguous fp32 {shape} tensor "
                            "on H's device")
    if (lse.device != H.device or lse.dtype != torch.float32
            or lse.numel() != N or not lse.is_contiguous()):
        raise VPCEError("lse must be a contiguous fp32 [N] tensor")
    if (totals.device != H.device or totals.dtype != torch.float64
            or totals.numel() != 2):
        raise VPCEError("totals must be an fp64 [2] tensor on the device")
    if dloss is not None and (dloss.device != H.device or dloss.numel() != 1
                              or dloss.dtype != torch.float32):
        raise VPCEError("dloss must be a one-element fp32 tensor")
    ws = _shard_workspace(H, V, workspace)
    with torch.cuda.device(H.device):
        st = _load().vpce_shard_backward(
            _ptr(H), _ptr(W_shard), _ptr(labels), _ptr(lse), _ptr(totals),
            _ptr(dloss), N, d, V, v_begin, W_shard.shape[0], ignore_index,
            _dtype_code(H.dtype), _ptr(dH), _ptr(dW_shard), _ptr(ws),
            ws.numel(), _stream(H))
    _check(st)
