"""Shared helpers of the GPU parity tests (comparison rules only; no
log-probability arithmetic lives here)."""

import numpy as np
import torch

# Tolerance on fp32 logp / lse against the float64 oracle: |gpu - ref| <=
# ATOL + RTOL * |ref| (the bound the logp path is held to).
ATOL = 1e-5
RTOL = 1e-5
# Relative tolerance of bf16 dlogits against the unrounded float64 gradient.
BWD_RTOL = 2e-3


def dev():
    return torch.device("cuda", 0)


def to_np(t):
    """Host float64 copy (bf16 and fp32 widen exactly)."""
    return t.detach().to(torch.float64).cpu().numpy()


def bits(t):
    """Raw bit pattern of a float32 tensor, for bitwise comparisons."""
    return t.detach().contiguous().view(torch.int32).cpu()


def assert_logp_parity(logp, lse, ref_logp, ref_lse, targets, ignore_index=-100, what=""):
    """Active rows within ATOL + RTOL*|ref|; ignored rows exactly +0."""
    t = targets.reshape(-1).cpu().numpy()
    active = t != ignore_index
    g_logp = to_np(logp.reshape(-1))
    g_lse = to_np(lse.reshape(-1))
    err = np.abs(g_logp - ref_logp)
    bound = ATOL + RTOL * np.abs(ref_logp)
    bad = active & ~(err <= bound)
    assert not bad.any(), (what, "logp", np.flatnonzero(bad)[:8], err[bad][:8])
    err = np.abs(g_lse - ref_lse)
    bad = active & ~(err <= ATOL + RTOL * np.abs(ref_lse))
    assert not bad.any(), (what, "lse", np.flatnonzero(bad)[:8], err[bad][:8])
    ign = ~active
    if ign.any():
        zb = bits(logp.reshape(-1)).numpy()[ign]
        assert (zb == 0).all(), (what, "ignored logp is not +0")
        zb = bits(lse.reshape(-1)).numpy()[ign]
        assert (zb == 0).all(), (what, "ignored lse is not +0")
    return float(np.max(np.abs(g_logp - ref_logp)[active])) if active.any() else 0.0


def assert_grad_parity(d_gpu, d_ref, x, lse_ref, g, targets, ignore_index=-100, what=""):
    """dlogits against the unrounded float64 gradient:
    |gpu - ref| <= BWD_RTOL*|ref| + |g| * p * (ATOL + RTOL*|x - lse|),
    the second term carrying the forward's lse tolerance through exp.
    Ignored rows are exactly +0."""
    d = to_np(d_gpu).reshape(d_ref.shape)
    t = targets.reshape(-1).cpu().numpy()
    active = t != ignore_index
    p = np.exp(x - lse_ref[:, None])
    gg = np.abs(np.asarray(g, dtype=np.float64).reshape(-1))[:, None]
    bound = BWD_RTOL * np.abs(d_ref) + gg * p * (ATOL + RTOL * np.abs(x - lse_ref[:, None]))
    bad = (np.abs(d - d_ref) > bound) & active[:, None]
    assert not bad.any(), (what, np.argwhere(bad)[:8], d[bad][:8], d_ref[bad][:8])
    if (~active).any():
        raw = d_gpu.reshape(d_ref.shape)[torch.from_numpy(~active).to(d_gpu.device)]
        assert (raw.view(torch.int16 if raw.dtype == torch.bfloat16 else torch.int32) == 0).all()
