"""Fused chunked KL-divergence loss for offline top-K distillation on MI355X.

Thin Python binding over ``libkdkl.so`` (C-ABI declared in ``include/kdkl.h``).
Every step of the loss runs in the library's HIP kernels; this module only
marshals torch tensors (device memory) and the current HIP stream. There is
no CPU fallback: without the built library, or without a GPU, calls raise.

The loss is the fused chunked KL of P1 "Making knowledge distillation cheap
enough to run at scale" (section "Two system changes"): per slice of
positions, project hidden states to logits, fold into the running loss, drop
the slice; recompute each slice in backward.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Tuple

import torch

from ._lib import (KDKL_BF16, KDKL_F32, KDKL_LOSS_JSD, KDKL_LOSS_KL, KDKL_LOSS_SKL, KDKL_LOSS_SRKL, KDKL_LOSS_TRKL,
                   KdklError,
                   KernelStat, Options, Plan,
                   check, load as _load)

__all__ = [
    "workspace_size",
    "saved_shape",
    "plan_info",
    "kdkl_forward",
    "kdkl_backward",
    "kdkl_forward_noalloc",
    "FusedKLLoss",
    "fused_kl_loss",
    "logits_forward",
    "logits_backward",
    "ForwardChunkedKLLoss",
    "forward_chunked_kl_loss",
    "dense_sizes",
    "dense_forward",
    "dense_backward",
    "check_ids",
    "profile_begin",
    "profile_end",
    "KdklError",
]


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDKL_BF16
    if t.dtype == torch.float32:
        return KDKL_F32
    raise TypeError(f"H/W must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return C.c_void_p(stream.cuda_stream)


def _need_gpu(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("inputs must be contiguous tensors on a ROCm device")


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _want(t, shape, dtype, device, name):
    """A caller-provided output must match exactly: the library writes it
    through a raw pointer."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")


OPTION_FIELDS = ("loss", "chunks_per_group", "vocab_slices", "dh_w_in_place", "beta")


def _options(options):
    """kdkl_options from None (defaults) or a dict with any of OPTION_FIELDS."""
    if options is None:
        return None
    unknown = set(options) - set(OPTION_FIELDS)
    if unknown:
        raise ValueError(f"unknown options {sorted(unknown)}; known: {OPTION_FIELDS}")
    o = Options()
    for k, v in options.items():
        setattr(o, k, float(v) if k == "beta" else int(v))
    return C.byref(o)


def saved_shape(N: int, options=None) -> Tuple[int, ...]:
    """Shape of the per-position state the forward saves for the backward
    (``row_lse``): [N] for the KL, [2, N] for the alternative losses (JSD,
    skew KL, skew reverse KL: logsumexp, then sum_v q_v g_v; reverse KL over
    the top-K support: logsumexp over the support, then the loss)."""
    if options is not None and int(options.get("loss", KDKL_LOSS_KL)) != KDKL_LOSS_KL:
        return (2, N)
    return (N,)


def workspace_size(N: int, d: int, V: int, K: int, chunk: int, dtype: torch.dtype,
                   options=None) -> Tuple[int, int]:
    """(forward bytes, backward bytes) of device workspace."""
    f = C.c_size_t()
    b = C.c_size_t()
    code = KDKL_BF16 if dtype == torch.bfloat16 else KDKL_F32
    check(_load().kdkl_workspace_size(N, d, V, K, chunk, code, _options(options), C.byref(f),
                                      C.byref(b)),
          "kdkl_workspace_size")
    return f.value, b.value


def plan_info(N: int, d: int, V: int, K: int, chunk: int, dtype: torch.dtype, options=None) -> dict:
    """The blocking the calls use (``kdkl_plan``) as a dict."""
    p = Plan()
    code = KDKL_BF16 if dtype == torch.bfloat16 else KDKL_F32
    check(_load().kdkl_plan_info(N, d, V, K, chunk, code, _options(options), C.byref(p)),
          "kdkl_plan_info")
    return {name: getattr(p, name) for name, _ in Plan._fields_ if name != "reserved"}


def _check_shapes(H, W, ids, logits):
    N, d = H.shape
    V, d2 = W.shape
    if d2 != d or ids.shape != logits.shape or ids.shape[0] != N:
        raise ValueError("shape mismatch among H [N,d], W [V,d], ids/logits [N,K]")
    if H.dtype != W.dtype or ids.dtype != torch.int32 or logits.dtype != torch.float32:
        raise TypeError("H and W share a dtype; ids int32; logits float32")
    return N, d, V, ids.shape[1]


def kdkl_forward(H, W, ids, logits, T: float, chunk: int, *, loss=None, row_lse=None,
                 row_kl=None, workspace=None, stream=None, want_row_kl: bool = True, options=None):
    """Run ``kdkl_forward``; returns (loss [1] fp32, row_lse [N], row_kl [N] or None)."""
    _need_gpu(H, W, ids, logits)
    N, d, V, K = _check_shapes(H, W, ids, logits)
    dev = H.device
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=dev)
    if row_lse is None:
        row_lse = torch.empty(saved_shape(N, options), dtype=torch.float32, device=dev)
    if row_kl is None and want_row_kl:
        row_kl = torch.empty(N, dtype=torch.float32, device=dev)
    _want(loss, (1,), torch.float32, dev, "loss")
    _want(row_lse, saved_shape(N, options), torch.float32, dev, "row_lse")
    if row_kl is not None:
        _want(row_kl, (N,), torch.float32, dev, "row_kl")
    fb, _ = workspace_size(N, d, V, K, chunk, H.dtype, options)
    if workspace is None:
        workspace = torch.empty(fb, dtype=torch.uint8, device=dev)
    _need_gpu(workspace)
    check(_load().kdkl_forward(_ptr(H), _ptr(W), _ptr(ids), _ptr(logits), N, d, V, K,
                              float(T), chunk, _dtype_code(H), _options(options), _ptr(loss),
                              _ptr(row_lse),
                              _ptr(row_kl), _ptr(workspace), _nbytes(workspace),
                              _stream(dev, stream)),
          "kdkl_forward")
    return loss, row_lse, row_kl


def kdkl_backward(H, W, ids, logits, T: float, chunk: int, row_lse, grad_loss=None, *,
                  dH=None, dW=None, accumulate_dW: bool = False, workspace=None, stream=None,
                  options=None):
    """Run ``kdkl_backward``; returns (dH [N,d] in H's dtype, dW [V,d] fp32)."""
    _need_gpu(H, W, ids, logits, row_lse, grad_loss)
    N, d, V, K = _check_shapes(H, W, ids, logits)
    dev = H.device
    if dH is None:
        dH = torch.empty_like(H)
    if dW is None:
        dW = torch.empty((V, d), dtype=torch.float32, device=dev)
    if grad_loss is not None and grad_loss.dtype != torch.float32:
        raise TypeError("grad_loss must be float32")
    _want(row_lse, saved_shape(N, options), torch.float32, dev, "row_lse")
    _want(dH, tuple(H.shape), H.dtype, dev, "dH")
    _want(dW, (V, d), torch.float32, dev, "dW")
    if grad_loss is not None:
        _want(grad_loss, (1,), torch.float32, dev, "grad_loss")
    _, bb = workspace_size(N, d, V, K, chunk, H.dtype, options)
    if workspace is None:
        workspace = torch.empty(bb, dtype=torch.uint8, device=dev)
    _need_gpu(workspace)
    check(_load().kdkl_backward(_ptr(H), _ptr(W), _ptr(ids), _ptr(logits), N, d, V, K,
                               float(T), chunk, _dtype_code(H), _options(options), _ptr(row_lse),
                               _ptr(grad_loss), _ptr(dH), _ptr(dW), int(bool(accumulate_dW)),
                               _ptr(workspace), _nbytes(workspace), _stream(dev, stream)),
          "kdkl_backward")
    return dH, dW


def kdkl_forward_noalloc(H, W, ids, logits, T: float, chunk: int, *, loss, row_lse, row_kl,
                         stream=None, options=None):
    """Run ``kdkl_forward_noalloc``: the forward on the library's static
    device scratch; every output is the caller's (nothing is allocated)."""
    _need_gpu(H, W, ids, logits, loss, row_lse, row_kl)
    N, d, V, K = _check_shapes(H, W, ids, logits)
    dev = H.device
    _want(loss, (1,), torch.float32, dev, "loss")
    _want(row_lse, saved_shape(N, options), torch.float32, dev, "row_lse")
    _want(row_kl, (N,), torch.float32, dev, "row_kl")
    check(_load().kdkl_forward_noalloc(_ptr(H), _ptr(W), _ptr(ids), _ptr(logits), N, d, V, K,
                                      float(T), chunk, _dtype_code(H), _options(options), _ptr(loss),
                                      _ptr(row_lse), _ptr(row_kl), _stream(dev, stream)),
          "kdkl_forward_noalloc")
    return loss, row_lse, row_kl


class FusedKLLoss(torch.autograd.Function):
    """Autograd wrapper: forward saves only row_lse (N floats); backward
    recomputes each chunk's logits inside the library."""

    @staticmethod
    def forward(ctx, H, W, ids, logits, T: float, chunk: int, options=None):
        loss, row_lse, _ = kdkl_forward(H, W, ids, logits, T, chunk, want_row_kl=False,
                                        options=options)
        ctx.save_for_backward(H, W, ids, logits, row_lse)
        ctx.T = T
        ctx.chunk = chunk
        ctx.options = options
        return loss[0]

    @staticmethod
    def backward(ctx, g):
        H, W, ids, logits, row_lse = ctx.saved_tensors
        g = g.reshape(1).to(torch.float32).contiguous()
        dH, dW = kdkl_backward(H, W, ids, logits, ctx.T, ctx.chunk, row_lse, g, options=ctx.options)
        return dH, dW.to(W.dtype), None, None, None, None, None


def fused_kl_loss(H, W, ids, logits, T: float = 1.0, chunk: int = 2048, options=None):
    """Mean over positions of KL(teacher top-K || student), differentiable in H and W."""
    return FusedKLLoss.apply(H, W, ids, logits, T, chunk, options)


def _check_logits_shapes(Z, ids, logits):
    if Z.dim() != 2 or not Z.is_contiguous():
        raise ValueError("Z must be a contiguous [N, V] tensor")
    N, V = Z.shape
    if ids.shape != logits.shape or ids.dim() != 2 or ids.shape[0] != N:
        raise ValueError("shape mismatch among Z [N,V], ids/logits [N,K]")
    if Z.dtype not in (torch.float32, torch.bfloat16) or ids.dtype != torch.int32 \
            or logits.dtype != torch.float32:
        raise TypeError("Z float32 or bfloat16; ids int32; logits float32")
    return N, V, ids.shape[1]


def logits_forward(Z, ids, logits, T: float, *, loss=None, row_lse=None, row_kl=None,
                   stream=None):
    """Forward-chunked KL from the student's logit grid ``Z [N, V]``
    (``kdkl_logits_forward``); returns (loss [1] fp32, row_lse [N], row_kl [N])."""
    _need_gpu(Z, ids, logits)
    N, V, K = _check_logits_shapes(Z, ids, logits)
    dev = Z.device
    if loss is None:
        loss = torch.empty(1, dtype=torch.float32, device=dev)
    if row_lse is None:
        row_lse = torch.empty(N, dtype=torch.float32, device=dev)
    if row_kl is None:
        row_kl = torch.empty(N, dtype=torch.float32, device=dev)
    _want(loss, (1,), torch.float32, dev, "loss")
    _want(row_lse, (N,), torch.float32, dev, "row_lse")
    _want(row_kl, (N,), torch.float32, dev, "row_kl")
    check(_load().kdkl_logits_forward(_ptr(Z), _ptr(ids), _ptr(logits), N, V, K, float(T),
                                      _dtype_code(Z), _ptr(loss), _ptr(row_lse), _ptr(row_kl),
                                      _stream(dev, stream)),
          "kdkl_logits_forward")
    return loss, row_lse, row_kl


LOGITS_BWD_WORKSPACE = 256  # KDKL_LOGITS_BWD_WORKSPACE


def logits_backward(Z, ids, logits, T: float, row_lse, grad_loss=None, *, dZ=None,
                    workspace=None, stream=None):
    """Gradient of the forward-chunked KL with respect to ``Z``
    (``kdkl_logits_backward``); ``dZ=Z`` overwrites the logits in place."""
    _need_gpu(Z, ids, logits, row_lse, grad_loss)
    N, V, K = _check_logits_shapes(Z, ids, logits)
    if dZ is None:
        dZ = torch.empty_like(Z)
    if dZ.shape != Z.shape or dZ.dtype != Z.dtype or not dZ.is_contiguous():
        raise ValueError("dZ must be a contiguous tensor of Z's shape and dtype")
    if grad_loss is not None and grad_loss.dtype != torch.float32:
        raise TypeError("grad_loss must be float32")
    _want(row_lse, (N,), torch.float32, Z.device, "row_lse")
    if grad_loss is not None:
        _want(grad_loss, (1,), torch.float32, Z.device, "grad_loss")
    if workspace is None:
        workspace = torch.empty(LOGITS_BWD_WORKSPACE, dtype=torch.uint8, device=Z.device)
    _need_gpu(workspace)
    check(_load().kdkl_logits_backward(_ptr(Z), _ptr(ids), _ptr(logits), N, V, K, float(T),
                                       _dtype_code(Z), _ptr(row_lse), _ptr(grad_loss),
                                       _ptr(dZ), _ptr(workspace), _nbytes(workspace),
                                       _stream(Z.device, stream)),
          "kdkl_logits_backward")
    return dZ


class ForwardChunkedKLLoss(torch.autograd.Function):
    """Autograd wrapper of the forward-chunked KL: the logit grid is an input
    (saved for the backward pass together with row_lse)."""

    @staticmethod
    def forward(ctx, Z, ids, logits, T: float):
        loss, row_lse, _ = logits_forward(Z, ids, logits, T)
        ctx.save_for_backward(Z, ids, logits, row_lse)
        ctx.T = T
        return loss[0]

    @staticmethod
    def backward(ctx, g):
        Z, ids, logits, row_lse = ctx.saved_tensors
        g = g.reshape(1).to(torch.float32).contiguous()
        return logits_backward(Z, ids, logits, ctx.T, row_lse, g), None, None, None


def forward_chunked_kl_loss(Z, ids, logits, T: float = 1.0):
    """Mean over positions of KL(teacher top-K || softmax(Z / T)), differentiable in Z."""
    return ForwardChunkedKLLoss.apply(Z, ids, logits, T)


CHECK_IDS_WORKSPACE = 16384  # KDKL_CHECK_IDS_WORKSPACE


def check_ids(ids, V: int, *, stream=None) -> Tuple[int, int]:
    """``kdkl_check_ids``: (ids outside [0, V), positions holding a repeated
    id), both over the kept positions; synchronises the stream to read them."""
    _need_gpu(ids)
    if ids.dim() != 2 or ids.dtype != torch.int32 or not ids.is_contiguous():
        raise ValueError("ids must be a contiguous int32 [N, K] tensor")
    N, K = ids.shape
    counts = torch.zeros(2, dtype=torch.int64, device=ids.device)
    ws = torch.empty(CHECK_IDS_WORKSPACE, dtype=torch.uint8, device=ids.device)
    check(_load().kdkl_check_ids(_ptr(ids), N, K, int(V), _ptr(counts), _ptr(ws), _nbytes(ws),
                                 _stream(ids.device, stream)),
          "kdkl_check_ids")
    c = counts.cpu()
    return int(c[0]), int(c[1])


def dense_sizes(N: int, d: int, V: int, K: int, dtype: torch.dtype) -> Tuple[int, int, int]:
    """(forward workspace, saved grids, backward workspace) bytes of the dense path."""
    f, sv, b = C.c_size_t(), C.c_size_t(), C.c_size_t()
    code = KDKL_BF16 if dtype == torch.bfloat16 else KDKL_F32
    check(_load().kdkl_dense_sizes(N, d, V, K, code, C.byref(f), C.byref(sv), C.byref(b)),
          "kdkl_dense_sizes")
    return f.value, sv.value, b.value


def dense_forward(H, W, ids, logits, T: float, *, saved=None, loss=None, row_lse=None,
                  row_kl=None, workspace=None, stream=None):
    """The pages' dense baseline (``kdkl_dense_forward``); returns (loss, row_lse,
    row_kl, saved) where ``saved`` holds the two full grids for the backward."""
    _need_gpu(H, W, ids, logits)
    N, d, V, K = _check_shapes(H, W, ids, logits)
    dev = H.device
    fb, sb, _ = dense_sizes(N, d, V, K, H.dtype)
    loss = torch.empty(1, dtype=torch.float32, device=dev) if loss is None else loss
    row_lse = torch.empty(N, dtype=torch.float32, device=dev) if row_lse is None else row_lse
    row_kl = torch.empty(N, dtype=torch.float32, device=dev) if row_kl is None else row_kl
    saved = torch.empty(sb, dtype=torch.uint8, device=dev) if saved is None else saved
    workspace = torch.empty(fb, dtype=torch.uint8, device=dev) if workspace is None else workspace
    _want(loss, (1,), torch.float32, dev, "loss")
    _want(row_lse, (N,), torch.float32, dev, "row_lse")
    _want(row_kl, (N,), torch.float32, dev, "row_kl")
    _need_gpu(saved, workspace)
    check(_load().kdkl_dense_forward(_ptr(H), _ptr(W), _ptr(ids), _ptr(logits), N, d, V, K, float(T),
                                     _dtype_code(H), _ptr(loss), _ptr(row_lse), _ptr(row_kl),
                                     _ptr(saved), _nbytes(saved), _ptr(workspace), _nbytes(workspace),
                                     _stream(dev, stream)),
          "kdkl_dense_forward")
    return loss, row_lse, row_kl, saved


def dense_backward(H, W, ids, logits, T: float, saved, grad_loss=None, *, dH=None, dW=None,
                   accumulate_dW: bool = False, workspace=None, stream=None):
    """Gradients of the dense baseline from its saved grids (``kdkl_dense_backward``)."""
    _need_gpu(H, W, ids, logits, saved, grad_loss)
    N, d, V, K = _check_shapes(H, W, ids, logits)
    dev = H.device
    _, _, bb = dense_sizes(N, d, V, K, H.dtype)
    dH = torch.empty_like(H) if dH is None else dH
    dW = torch.empty((V, d), dtype=torch.float32, device=dev) if dW is None else dW
    if grad_loss is not None and grad_loss.dtype != torch.float32:
        raise TypeError("grad_loss must be float32")
    workspace = torch.empty(bb, dtype=torch.uint8, device=dev) if workspace is None else workspace
    _want(dH, tuple(H.shape), H.dtype, dev, "dH")
    _want(dW, (V, d), torch.float32, dev, "dW")
    if grad_loss is not None:
        _want(grad_loss, (1,), torch.float32, dev, "grad_loss")
    _need_gpu(workspace)
    check(_load().kdkl_dense_backward(_ptr(H), _ptr(W), _ptr(ids), _ptr(logits), N, d, V, K,
                                      float(T), _dtype_code(H), _ptr(saved), _nbytes(saved),
                                      _ptr(grad_loss), _ptr(dH), _ptr(dW), int(bool(accumulate_dW)),
                                      _ptr(workspace), _nbytes(workspace), _stream(dev, stream)),
          "kdkl_dense_backward")
    return dH, dW


def profile_begin():
    check(_load().kdkl_profile_begin(), "kdkl_profile_begin")


def profile_end():
    """Stop profiling; returns {kernel name: dict(launches, total_ms, flops, bytes)}."""
    cap = 32
    arr = (KernelStat * cap)()
    n = C.c_int()
    check(_load().kdkl_profile_end(arr, cap, C.byref(n)), "kdkl_profile_end")
    out = {}
    for i in range(min(n.value, cap)):
        s = arr[i]
        out[s.name.decode()] = {"launches": s.launches, "total_ms": s.total_ms,
                                "flops": s.flops, "bytes": s.bytes}
    return out
