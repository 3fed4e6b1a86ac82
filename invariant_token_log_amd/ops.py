"""PyTorch-facing binding of the C ABI (argument marshalling only).

PyTorch supplies device memory and the current HIP stream; every step of the
computation runs in the library's kernels.  Tensors must live on a ROCm
device; the library checks everything else and its status becomes a
LogpError.
"""

import torch

from . import _lib
from ._lib import LOGP_BF16, LOGP_F16, LOGP_F32, LOGP_I32, LOGP_I64, check

_DTYPES = {torch.float32: LOGP_F32, torch.bfloat16: LOGP_BF16, torch.float16: LOGP_F16}
_INDEX = {torch.int64: LOGP_I64, torch.int32: LOGP_I32}


def _dtype_code(t):
    if t.dtype not in _DTYPES:
        raise TypeError(f"logits dtype {t.dtype} is not supported (float32, bfloat16, float16)")
    return _DTYPES[t.dtype]


def _rows(x):
    """[*lead, V] -> ([N, V] view, row stride in elements) without copying."""
    if not x.is_cuda:
        raise ValueError("tensors must be on a ROCm device")
    if x.dim() < 1:
        raise ValueError("need a trailing vocabulary dimension")
    v = x.shape[-1]
    if x.stride(-1) != 1:
        raise ValueError("the vocabulary dimension must be contiguous")
    x2 = x.reshape(-1, v) if x.dim() != 2 else x
    if x2.data_ptr() != x.data_ptr() and x.numel():
        raise ValueError("leading dimensions must flatten without a copy")
    ld = x2.stride(0) if x2.shape[0] > 1 else v
    return x2, v, ld


def _targets(t, n):
    if t.dtype not in _INDEX:
        raise TypeError("targets must be int64 or int32")
    if not t.is_cuda:
        raise ValueError("targets must be on a ROCm device")
    t1 = t.reshape(-1)
    if t1.numel() != n:
        raise ValueError("targets must have one entry per logits row")
    if not t1.is_contiguous():
        raise ValueError("targets must be contiguous")
    return t1


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def logp_fwd(logits, targets, ignore_index=-100, tile_width=4096, num_shards=1,
             validate=False, logp_out=None, lse_out=None, workspace=None):
    """Selected-token log-probability.  Returns (logp shaped like targets,
    lse [N]) as float32."""
    x2, v, ld = _rows(logits)
    n = x2.shape[0]
    t1 = _targets(targets, n)
    dev = logits.device
    if logp_out is None:
        logp_out = torch.empty(n, dtype=torch.float32, device=dev)
    if lse_out is None:
        lse_out = torch.empty(n, dtype=torch.float32, device=dev)
    L = _lib.lib()
    need = L.logp_fwd_workspace_bytes(n, v, tile_width, num_shards, int(bool(validate)))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = L.logp_fwd(x2.data_ptr(), _dtype_code(logits), n, v, ld, t1.data_ptr(),
                    _INDEX[t1.dtype], int(ignore_index), int(tile_width), int(num_shards),
                    int(bool(validate)), logp_out.data_ptr(), lse_out.data_ptr(), ws_ptr, ws_len,
                    _stream(dev))
    check("logp_fwd", st)
    return logp_out.view(targets.shape), lse_out


def logp_bwd(logits, targets, lse, grad_logp, ignore_index=-100, tile_width=4096,
             dlogits_out=None):
    """dlogits = g * (onehot - softmax) in the logits dtype, shaped like logits."""
    x2, v, ld = _rows(logits)
    n = x2.shape[0]
    t1 = _targets(targets, n)
    g = grad_logp.reshape(-1)
    if g.dtype != torch.float32 or lse.dtype != torch.float32:
        raise TypeError("lse and grad_logp must be float32")
    if g.numel() != n or lse.numel() != n or not g.is_contiguous() or not lse.is_contiguous():
        raise ValueError("lse and grad_logp must be contiguous with one entry per row")
    if dlogits_out is None:
        dlogits_out = torch.empty_like(logits)
    d2, v2, ld_out = _rows(dlogits_out)
    if v2 != v or d2.shape[0] != n or dlogits_out.dtype != logits.dtype:
        raise ValueError("dlogits_out must match the logits shape and dtype")
    st = _lib.lib().logp_bwd(x2.data_ptr(), _dtype_code(logits), n, v, ld, t1.data_ptr(),
                             _INDEX[t1.dtype], int(ignore_index), int(tile_width),
                             lse.data_ptr(),
                             g.data_ptr(), d2.data_ptr(), ld_out, _stream(logits.device))
    check("logp_bwd", st)
    return dlogits_out


LINEAR_TILE = 256


def linear_logp_fwd(hidden, weight, targets, ignore_index=-100, tile_width=LINEAR_TILE,
                    logp_out=None, lse_out=None, workspace=None):
    """Fused LM-head + selected-token log-probability without storing logits.
    hidden bf16 [N, H], weight bf16 [V, H].  Returns (logp [N], lse [N])."""
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.stride(1) != 1 or weight.stride(1) != 1:
        raise ValueError("hidden [N, H] and weight [V, H] need a contiguous last dimension")
    n, h = hidden.shape
    v, h2 = weight.shape
    if h2 != h:
        raise ValueError("hidden and weight must share H")
    t1 = _targets(targets, n)
    dev = hidden.device
    if logp_out is None:
        logp_out = torch.empty(n, dtype=torch.float32, device=dev)
    if lse_out is None:
        lse_out = torch.empty(n, dtype=torch.float32, device=dev)
    L = _lib.lib()
    need = L.linear_logp_fwd_workspace_bytes(n, v, tile_width)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ld_h = hidden.stride(0) if n > 1 else h
    ld_w = weight.stride(0) if v > 1 else h
    st = L.linear_logp_fwd(hidden.data_ptr(), ld_h, weight.data_ptr(), ld_w, n, h, v,
                           t1.data_ptr(), _INDEX[t1.dtype], int(ignore_index), int(tile_width),
                           logp_out.data_ptr(), lse_out.data_ptr(), workspace.data_ptr(),
                           workspace.numel(), _stream(dev))
    check("linear_logp_fwd", st)
    return logp_out, lse_out


def linear_logp_bwd(hidden, weight, targets, lse, grad_logp, ignore_index=-100,
                    tile_width=LINEAR_TILE, need_dhidden=True, need_dweight=True,
                    out_dtype=torch.float32, dhidden_out=None, dweight_out=None,
                    workspace=None):
    """Backward of the fused LM head + logp: (dhidden [N, H] or None,
    dweight [V, H] or None) in out_dtype (float32 accumulators or their
    bfloat16 rounding), from the forward's lse and the upstream gradient."""
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.stride(1) != 1 or weight.stride(1) != 1:
        raise ValueError("hidden [N, H] and weight [V, H] need a contiguous last dimension")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    n, h = hidden.shape
    v, h2 = weight.shape
    if h2 != h:
        raise ValueError("hidden and weight must share H")
    t1 = _targets(targets, n)
    g = grad_logp.reshape(-1)
    if g.dtype != torch.float32 or lse.dtype != torch.float32:
        raise TypeError("lse and grad_logp must be float32")
    if g.numel() != n or lse.numel() != n or not g.is_contiguous() or not lse.is_contiguous():
        raise ValueError("lse and grad_logp must be contiguous with one entry per row")
    dev = hidden.device
    if need_dhidden and dhidden_out is None:
        dhidden_out = torch.empty(n, h, dtype=out_dtype, device=dev)
    if need_dweight and dweight_out is None:
        dweight_out = torch.empty(v, h, dtype=out_dtype, device=dev)
    dh = dhidden_out if need_dhidden else None
    dw = dweight_out if need_dweight else None
    for o, rows in ((dh, n), (dw, v)):
        if o is not None and (o.dtype != out_dtype or o.dim() != 2 or o.shape[0] != rows
                              or o.shape[1] != h or o.stride(1) != 1):
            raise ValueError("output buffers must be [rows, H] of out_dtype, rows contiguous")
    L = _lib.lib()
    need = L.linear_logp_bwd_workspace_bytes(n, h, v, tile_width)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() if workspace is not None else 0
    ld_h = hidden.stride(0) if n > 1 else h
    ld_w = weight.stride(0) if v > 1 else h
    st = L.linear_logp_bwd(hidden.data_ptr(), ld_h, weight.data_ptr(), ld_w, n, h, v,
                           t1.data_ptr(), _INDEX[t1.dtype], int(ignore_index),
                           int(tile_width), lse.data_ptr(),
                           g.data_ptr(), _DTYPES[out_dtype],
                           dh.data_ptr() if dh is not None else None,
                           (dh.stride(0) if n > 1 else h) if dh is not None else 0,
                           dw.data_ptr() if dw is not None else None,
                           (dw.stride(0) if v > 1 else h) if dw is not None else 0,
                           ws_ptr, ws_len, _stream(dev))
    check("linear_logp_bwd", st)
    return dh, dw


class _LinearLogp(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, weight, targets, ignore_index):
        logp, lse = linear_logp_fwd(hidden, weight, targets, ignore_index)
        ctx.save_for_backward(hidden, weight, targets, lse)
        ctx.ignore_index = ignore_index
        return logp

    @staticmethod
    def backward(ctx, grad):
        hidden, weight, targets, lse = ctx.saved_tensors
        g = grad.to(torch.float32).contiguous()
        dh, dw = linear_logp_bwd(hidden, weight, targets, lse, g, ctx.ignore_index,
                                 need_dhidden=ctx.needs_input_grad[0],
                                 need_dweight=ctx.needs_input_grad[1],
                                 out_dtype=torch.bfloat16)
        return dh, dw, None, None


def linear_logp(hidden, weight, target_ids, ignore_index=-100):
    """Differentiable fused LM head + selected-token log-probability:
    hidden bf16 [N, H], weight bf16 [V, H] -> float32 logp [N]; backward fills
    the bf16 gradients of hidden and weight through linear_logp_bwd."""
    return _LinearLogp.apply(hidden, weight, target_ids, ignore_index)


class _BatchInvariantLogp(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, targets, ignore_index, tile_width, validate):
        logp, lse = logp_fwd(logits, targets, ignore_index, tile_width, 1, validate)
        ctx.save_for_backward(logits, targets, lse)
        ctx.ignore_index = ignore_index
        ctx.tile_width = tile_width
        return logp

    @staticmethod
    def backward(ctx, grad):
        logits, targets, lse = ctx.saved_tensors
        g = grad.to(torch.float32).contiguous()
        d = logp_bwd(logits, targets, lse, g, ctx.ignore_index, ctx.tile_width)
        return d, None, None, None, None


def batch_invariant_logp(logits, target_ids, ignore_index=-100, tile_width=4096,
                         validate=False):
    """Differentiable selected-token log-probability ("Batch-Invariant LogP",
    Entry Point): logits [*lead, V] -> float32 [*lead]; backward fills the
    logits gradient through logp_bwd."""
    return _BatchInvariantLogp.apply(logits, target_ids, ignore_index, tile_width, validate)
