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


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _row_vector(x, n, name):
    if x is None:
        return None
    x1 = x.reshape(-1)
    if x1.dtype != torch.float32 or x1.numel() != n or not x1.is_contiguous():
        raise ValueError(f"{name} must be contiguous float32 with one entry per row")
    return x1


def logp_fwd(logits, targets, ignore_index=-100, tile_width=4096, num_shards=1,
             validate=False, logp_out=None, lse_out=None, workspace=None,
             return_entropy=False, entropy_out=None):
    """Selected-token log-probability.  Returns (logp shaped like targets,
    lse [N]) as float32, and the row entropy [N] as a third element when
    return_entropy is set."""
    x2, v, ld = _rows(logits)
    n = x2.shape[0]
    t1 = _targets(targets, n)
    dev = logits.device
    if logp_out is None:
        logp_out = torch.empty(n, dtype=torch.float32, device=dev)
    if lse_out is None:
        lse_out = torch.empty(n, dtype=torch.float32, device=dev)
    if return_entropy and entropy_out is None:
        entropy_out = torch.empty(n, dtype=torch.float32, device=dev)
    ent = entropy_out if return_entropy else None
    L = _lib.lib()
    need = L.logp_fwd_workspace_bytes(n, v, tile_width, num_shards, int(bool(validate)))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    with torch.cuda.device(dev):
        st = L.logp_fwd(x2.data_ptr(), _dtype_code(logits), n, v, ld, t1.data_ptr(),
                        _INDEX[t1.dtype], int(ignore_index), int(tile_width), int(num_shards),
                        int(bool(validate)), logp_out.data_ptr(), lse_out.data_ptr(), _ptr(ent),
                        _ptr(workspace), ws_len, _stream(dev))
    check("logp_fwd", st)
    if return_entropy:
        return logp_out.view(targets.shape), lse_out, ent
    return logp_out.view(targets.shape), lse_out


def logp_bwd(logits, targets, lse, grad_logp, ignore_index=-100, tile_width=4096,
             dlogits_out=None, entropy=None, grad_entropy=None):
    """dlogits = g * (onehot - softmax) (- gH * p * (log p + H) when the row
    entropy and its upstream gradient are given) in the logits dtype, shaped
    like logits."""
    x2, v, ld = _rows(logits)
    n = x2.shape[0]
    t1 = _targets(targets, n)
    g = _row_vector(grad_logp, n, "grad_logp")
    lse = _row_vector(lse, n, "lse")
    ent = _row_vector(entropy, n, "entropy")
    gent = _row_vector(grad_entropy, n, "grad_entropy")
    if (ent is None) != (gent is None):
        raise ValueError("entropy and grad_entropy go together")
    if dlogits_out is None:
        dlogits_out = torch.empty_like(logits)
    d2, v2, ld_out = _rows(dlogits_out)
    if v2 != v or d2.shape[0] != n or dlogits_out.dtype != logits.dtype:
        raise ValueError("dlogits_out must match the logits shape and dtype")
    with torch.cuda.device(logits.device):
        st = _lib.lib().logp_bwd(x2.data_ptr(), _dtype_code(logits), n, v, ld, t1.data_ptr(),
                                 _INDEX[t1.dtype], int(ignore_index), int(tile_width),
                                 lse.data_ptr(), g.data_ptr(), _ptr(ent), _ptr(gent),
                                 d2.data_ptr(), ld_out, _stream(logits.device))
    check("logp_bwd", st)
    return dlogits_out


LINEAR_TILE = 256


def _linear_operands(hidden, weight):
    if hidden.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("hidden and weight must be bfloat16")
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.stride(1) != 1 or weight.stride(1) != 1:
        raise ValueError("hidden [N, H] and weight [V, H] need a contiguous last dimension")
    n, h = hidden.shape
    v, h2 = weight.shape
    if h2 != h:
        raise ValueError("hidden and weight must share H")
    ld_h = hidden.stride(0) if n > 1 else h
    ld_w = weight.stride(0) if v > 1 else h
    return n, h, v, ld_h, ld_w


def _rounding(round_logits):
    return _lib.LOGP_ROUND_BF16 if round_logits else _lib.LOGP_ROUND_NONE


def linear_logp_fwd(hidden, weight, targets, ignore_index=-100, tile_width=LINEAR_TILE,
                    logp_out=None, lse_out=None, workspace=None, temperature=1.0,
                    return_entropy=False, entropy_out=None, return_logits=False,
                    logits_dtype=torch.bfloat16, logits_out=None, round_logits=False,
                    prepared_weight=None):
    """Fused LM-head + selected-token log-probability without storing logits.
    hidden bf16 [N, H], weight bf16 [V, H].  Returns (logp [N], lse [N]), then
    the entropy [N] with return_entropy and the unscaled logits [N, V] with
    return_logits.  The statistics see the logits times 1 / temperature; with
    round_logits the logits are first rounded to bf16 (RNE), as an unfused
    bf16 LM head would store them.  prepared_weight: prepare_weight(weight),
    read instead of the weight (same bits)."""
    return _linear_fwd(hidden, weight, targets, ignore_index, tile_width, logp_out, lse_out,
                       workspace, temperature, return_entropy, entropy_out, return_logits,
                       logits_dtype, logits_out, round_logits, prepared_weight, noalloc=False)


def linear_logp_fwd_noalloc(hidden, weight, targets, ignore_index=-100,
                            tile_width=LINEAR_TILE, logp_out=None, lse_out=None,
                            temperature=1.0, return_entropy=False, entropy_out=None,
                            return_logits=False, logits_dtype=torch.bfloat16, logits_out=None,
                            round_logits=False, prepared_weight=None):
    """linear_logp_fwd through the entry point that takes no workspace: the
    library's static per-GPU scratch array stands in for it (see
    NOALLOC_SCRATCH_BYTES for its size).  Pass every output buffer to keep
    the call free of allocations (e.g. under graph capture); calls that
    overlap on one GPU race on the shared array."""
    return _linear_fwd(hidden, weight, targets, ignore_index, tile_width, logp_out, lse_out,
                       None, temperature, return_entropy, entropy_out, return_logits,
                       logits_dtype, logits_out, round_logits, prepared_weight, noalloc=True)


def _linear_fwd(hidden, weight, targets, ignore_index, tile_width, logp_out, lse_out,
                workspace, temperature, return_entropy, entropy_out, return_logits,
                logits_dtype, logits_out, round_logits, prepared_weight, noalloc):
    n, h, v, ld_h, ld_w = _linear_operands(hidden, weight)
    pbuf = _prepared_buffer(prepared_weight, weight)
    t1 = _targets(targets, n)
    dev = hidden.device
    if logp_out is None:
        logp_out = torch.empty(n, dtype=torch.float32, device=dev)
    if lse_out is None:
        lse_out = torch.empty(n, dtype=torch.float32, device=dev)
    if return_entropy and entropy_out is None:
        entropy_out = torch.empty(n, dtype=torch.float32, device=dev)
    ent = entropy_out if return_entropy else None
    if logits_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("logits_dtype must be float32 or bfloat16")
    if return_logits and logits_out is None:
        logits_out = torch.empty(n, v, dtype=logits_dtype, device=dev)
    z = logits_out if return_logits else None
    if z is not None and (z.dtype != logits_dtype or z.dim() != 2 or tuple(z.shape) != (n, v)
                          or z.stride(1) != 1):
        raise ValueError("logits_out must be [N, V] of logits_dtype with contiguous rows")
    L = _lib.lib()
    pw = _prepared(pbuf, L, v, h, dev)
    args = (hidden.data_ptr(), ld_h, weight.data_ptr(), ld_w, n, h, v, t1.data_ptr(),
            _INDEX[t1.dtype], int(ignore_index), int(tile_width), float(temperature),
            _rounding(round_logits), logp_out.data_ptr(), lse_out.data_ptr(), _ptr(ent), _ptr(z),
            _DTYPES[logits_dtype], (z.stride(0) if n > 1 else v) if z is not None else 0,
            _ptr(pw), _nbytes(pw))
    with torch.cuda.device(dev):
        if noalloc:
            st = L.linear_logp_fwd_noalloc(*args, _stream(dev))
        else:
            if workspace is None:
                need = L.linear_logp_fwd_workspace_bytes(n, h, v, tile_width)
                workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            st = L.linear_logp_fwd(*args, workspace.data_ptr(), _nbytes(workspace),
                                   _stream(dev))
    check("linear_logp_fwd_noalloc" if noalloc else "linear_logp_fwd", st)
    out = (logp_out, lse_out)
    if return_entropy:
        out += (ent,)
    if return_logits:
        out += (z,)
    return out


def linear_logp_bwd_workspace_bytes(n, h, v, need_dhidden=True, need_dweight=True,
                                    prepared=False, saved_logits=False,
                                    out_dtype=torch.float32, vocab_chunk=0,
                                    tile_width=LINEAR_TILE):
    """Workspace bytes linear_logp_bwd needs for a call with these options."""
    flags = ((_lib.LOGP_BWD_DHIDDEN if need_dhidden else 0)
             | (_lib.LOGP_BWD_DWEIGHT if need_dweight else 0)
             | (_lib.LOGP_BWD_PREPARED if prepared else 0)
             | (_lib.LOGP_BWD_SAVED_LOGITS if saved_logits else 0)
             | (_lib.LOGP_BWD_BF16_OUT if out_dtype == torch.bfloat16 else 0))
    return _lib.lib().linear_logp_bwd_workspace_bytes(n, h, v, tile_width, flags, vocab_chunk)


def linear_logp_bwd(hidden, weight, targets, lse, grad_logp, ignore_index=-100,
                    tile_width=LINEAR_TILE, need_dhidden=True, need_dweight=True,
                    out_dtype=torch.float32, dhidden_out=None, dweight_out=None,
                    workspace=None, temperature=1.0, entropy=None, grad_entropy=None,
                    round_logits=False, saved_logits=None, prepared_weight=None,
                    vocab_chunk=0):
    """Backward of the fused LM head + logp: (dhidden [N, H] or None,
    dweight [V, H] or None) in out_dtype (float32 accumulators or their
    bfloat16 rounding), from the forward's lse (and entropy) and the upstream
    gradients.  temperature and round_logits must be the forward's.
    saved_logits: the forward's logits output ([N, V] float32, or bfloat16
    with round_logits), read instead of recomputing h W^T; same bits.
    prepared_weight: prepare_weight(weight), read instead of the weight and
    its transpose made on every call; same bits.  vocab_chunk: vocabulary
    columns per pass (0 = the library's default); any value gives the same
    bits, smaller ones need less workspace."""
    n, h, v, ld_h, ld_w = _linear_operands(hidden, weight)
    pbuf = _prepared_buffer(prepared_weight, weight)
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    t1 = _targets(targets, n)
    g = _row_vector(grad_logp, n, "grad_logp")
    lse = _row_vector(lse, n, "lse")
    ent = _row_vector(entropy, n, "entropy")
    gent = _row_vector(grad_entropy, n, "grad_entropy")
    if (ent is None) != (gent is None):
        raise ValueError("entropy and grad_entropy go together")
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
    z = saved_logits
    if z is not None and (z.dim() != 2 or tuple(z.shape) != (n, v) or z.stride(1) != 1
                          or z.dtype not in (torch.float32, torch.bfloat16)):
        raise ValueError("saved_logits must be [N, V] float32 / bfloat16 with contiguous rows")
    L = _lib.lib()
    pw = _prepared(pbuf, L, v, h, dev)
    need = linear_logp_bwd_workspace_bytes(n, h, v, dh is not None, dw is not None,
                                           pw is not None, z is not None, out_dtype,
                                           int(vocab_chunk), tile_width)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_len = workspace.numel() if workspace is not None else 0
    with torch.cuda.device(dev):
        st = L.linear_logp_bwd(hidden.data_ptr(), ld_h, weight.data_ptr(), ld_w, n, h, v,
                               t1.data_ptr(), _INDEX[t1.dtype], int(ignore_index), int(tile_width),
                               float(temperature), _rounding(round_logits), _ptr(z),
                               _DTYPES[z.dtype] if z is not None else 0,
                               max(z.stride(0), v) if z is not None else 0, _ptr(pw),
                               _nbytes(pw), lse.data_ptr(),
                               g.data_ptr(), _ptr(ent),
                               _ptr(gent), _DTYPES[out_dtype], _ptr(dh),
                               (dh.stride(0) if n > 1 else h) if dh is not None else 0,
                               _ptr(dw), (dw.stride(0) if v > 1 else h) if dw is not None else 0,
                               int(vocab_chunk), _ptr(workspace), ws_len, _stream(dev))
    check("linear_logp_bwd", st)
    return dh, dw


def _nbytes(t):
    return t.numel() * t.element_size() if t is not None else 0


class PreparedWeight:
    """What prepare_weight returns: `buffer`, the weight re-laid for the fused
    products (uint8 device tensor), and the identity of the weight it was made
    from (data pointer, shape, device and in-place version counter).  Every
    use checks that identity, so a weight that was updated in place (an
    optimiser step) or replaced is refused instead of giving wrong results."""

    __slots__ = ("buffer", "weight_ptr", "shape", "device", "version")

    def __init__(self, buffer, weight):
        self.buffer = buffer
        self.weight_ptr = weight.data_ptr()
        self.shape = tuple(weight.shape)
        self.device = weight.device
        self.version = weight._version

    def check(self, weight):
        """Raise ValueError unless `weight` is the tensor this was prepared
        from, unchanged since."""
        if (weight.data_ptr() != self.weight_ptr or tuple(weight.shape) != self.shape
                or weight.device != self.device):
            raise ValueError("prepared_weight was prepared from another weight tensor; "
                             "call prepare_weight(weight) for this one")
        if weight._version != self.version:
            raise ValueError("prepared_weight is stale: the weight changed in place after "
                             "prepare_weight; prepare it again")


def _prepared_buffer(p, weight):
    """The prepared buffer for `weight`, after the identity check (before any
    device work)."""
    if p is None:
        return None
    if not isinstance(p, PreparedWeight):
        raise TypeError("prepared_weight must be the result of prepare_weight(weight)")
    p.check(weight)
    return p.buffer


def _prepared(buf, L, v, h, dev):
    if buf is not None and (not buf.is_contiguous() or buf.device != dev
                            or _nbytes(buf) < L.linear_logp_prepared_bytes(v, h)):
        raise ValueError("prepared_weight's buffer is too small or not on the weight's device")
    return buf


def prepare_weight(weight, out=None):
    """The LM-head weight [V, H] bfloat16 re-laid for the fused products'
    loads (the weight and its transpose, vocabulary padded with zeros to a
    multiple of 256, in the library's own layout), as a PreparedWeight whose
    `buffer` is a uint8 tensor of linear_logp_prepared_bytes(V, H) bytes (or
    `out`, a contiguous buffer at least that large), for linear_logp_fwd,
    linear_logp_bwd and linear_logp.  Reuse it over the calls of one weight
    version; after the weight changes (an optimiser step, a weight update)
    every use raises until it is prepared again."""
    if weight.dtype != torch.bfloat16 or weight.dim() != 2 or weight.stride(1) != 1:
        raise ValueError("weight must be [V, H] bfloat16 with contiguous rows")
    v, h = weight.shape
    if not weight.is_cuda:
        raise ValueError("weight must be a GPU tensor")
    L = _lib.lib()
    need = L.linear_logp_prepared_bytes(v, h)
    if need == 0:
        raise ValueError("H must be a positive multiple of 64")
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=weight.device)
    if not out.is_contiguous() or out.numel() * out.element_size() < need:
        raise ValueError(f"out must be a contiguous buffer of at least {need} bytes")
    with torch.cuda.device(weight.device):
        st = L.linear_logp_prepare_weight(weight.data_ptr(), weight.stride(0) if v > 1 else h,
                                          v, h, out.data_ptr(), out.numel() * out.element_size(),
                                          _stream(weight.device))
    check("linear_logp_prepare_weight", st)
    return PreparedWeight(out, weight)


def _grad_or_zeros(g, ref):
    return torch.zeros_like(ref) if g is None else g.to(torch.float32).contiguous()


class _BatchInvariantLogp(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, targets, ignore_index, tile_width, validate, with_entropy):
        out = logp_fwd(logits, targets, ignore_index, tile_width, 1, validate,
                       return_entropy=with_entropy)
        logp, lse = out[0], out[1]
        ent = out[2] if with_entropy else None
        ctx.save_for_backward(logits, targets, lse, ent)
        ctx.ignore_index = ignore_index
        ctx.tile_width = tile_width
        ctx.with_entropy = with_entropy
        if with_entropy:
            return logp, ent.view(targets.shape)
        return logp

    @staticmethod
    def backward(ctx, grad, *rest):
        logits, targets, lse, ent = ctx.saved_tensors
        g = _grad_or_zeros(grad, lse).reshape(-1)
        gent = _grad_or_zeros(rest[0], lse).reshape(-1) if ctx.with_entropy else None
        d = logp_bwd(logits, targets, lse, g, ctx.ignore_index, ctx.tile_width,
                     entropy=ent if ctx.with_entropy else None, grad_entropy=gent)
        return d, None, None, None, None, None


def batch_invariant_logp(logits, target_ids, ignore_index=-100, tile_width=4096,
                         validate=False, return_entropy=False):
    """Differentiable selected-token log-probability ("Batch-Invariant LogP",
    Entry Point): logits [*lead, V] -> float32 [*lead]; with return_entropy,
    also the differentiable full-vocabulary entropy [*lead].  The backward
    fills the logits gradient through logp_bwd."""
    return _BatchInvariantLogp.apply(logits, target_ids, ignore_index, tile_width, validate,
                                     return_entropy)


def _padded_logits(n, v, dtype, device):
    """[n, v] view of a buffer whose rows are padded to 16 bytes, so the
    backward can read it with 16-byte loads."""
    per = 16 // torch.empty((), dtype=dtype).element_size()
    ld = (v + per - 1) // per * per
    return torch.empty(n, ld, dtype=dtype, device=device)[:, :v]


class _LinearLogp(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, weight, targets, ignore_index, temperature, with_entropy,
                round_logits, save_logits, prepared_weight):
        zdt = torch.bfloat16 if round_logits else torch.float32
        zbuf = _padded_logits(hidden.shape[0], weight.shape[0], zdt, hidden.device) \
            if save_logits else None
        out = linear_logp_fwd(hidden, weight, targets, ignore_index, temperature=temperature,
                              return_entropy=with_entropy, round_logits=round_logits,
                              return_logits=save_logits, logits_dtype=zdt, logits_out=zbuf,
                              prepared_weight=prepared_weight)
        logp, lse = out[0], out[1]
        ent = out[2] if with_entropy else None
        z = out[-1] if save_logits else None
        ctx.save_for_backward(hidden, weight, targets, lse, ent, z)
        ctx.ignore_index = ignore_index
        ctx.temperature = temperature
        ctx.with_entropy = with_entropy
        ctx.round_logits = round_logits
        ctx.prepared_weight = prepared_weight
        if with_entropy:
            return logp, ent
        return logp

    @staticmethod
    def backward(ctx, grad, *rest):
        hidden, weight, targets, lse, ent, z = ctx.saved_tensors
        if ctx.prepared_weight is not None:
            ctx.prepared_weight.check(weight)
        g = _grad_or_zeros(grad, lse)
        gent = _grad_or_zeros(rest[0], lse) if ctx.with_entropy else None
        dh, dw = linear_logp_bwd(hidden, weight, targets, lse, g, ctx.ignore_index,
                                 need_dhidden=ctx.needs_input_grad[0],
                                 need_dweight=ctx.needs_input_grad[1],
                                 out_dtype=torch.bfloat16, temperature=ctx.temperature,
                                 entropy=ent if ctx.with_entropy else None, grad_entropy=gent,
                                 round_logits=ctx.round_logits, saved_logits=z,
                                 prepared_weight=ctx.prepared_weight)
        return dh, dw, None, None, None, None, None, None, None


def linear_logp(hidden, weight, target_ids, ignore_index=-100, temperature=1.0,
                return_entropy=False, round_logits=False, save_logits=False,
                prepared_weight=None):
    """Differentiable fused LM head + selected-token log-probability:
    hidden bf16 [N, H], weight bf16 [V, H] -> float32 logp [N] (and the
    entropy [N] with return_entropy) of softmax(hidden weight^T / temperature);
    round_logits rounds the logits to bf16 first (the unfused bf16 LM head's
    values; the gradient passes the rounding unchanged).  Backward fills the
    bf16 gradients of hidden and weight through linear_logp_bwd, recomputing
    the logits, or, with save_logits, reading the logits the forward kept
    ([N, V] float32, bfloat16 with round_logits; same bits, more memory).
    prepared_weight: prepare_weight(weight) of this weight version, read by
    the forward and the backward instead of the weight (same bits)."""
    return _LinearLogp.apply(hidden, weight, target_ids, ignore_index, temperature,
                             return_entropy, round_logits, save_logits, prepared_weight)
