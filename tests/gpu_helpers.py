"""Shared helpers of the GPU parity tests (comparison rules only; no
log-probability arithmetic lives here)."""

import numpy as np
import torch

# Tolerance on fp32 logp / lse against the float64 oracle: |gpu - ref| <=
# ATOL + RTOL * |ref| (the bound the logp path is held to).
ATOL = 1e-5
RTOL = 1e-5
# The hardware exponential returns no subnormals: exp values below the
# smallest normal float32 come out as +0, so a gradient element may be +-0
# where the exact one is below |g| * FLT_MIN.
FLT_MIN = 2.0 ** -126
# Relative tolerance of fp32 dlogits against the unrounded float64 gradient
# (bf16 dlogits are checked against their two bf16 neighbours instead, since
# rounding to bf16 alone moves a value by up to 2^-8 = 3.9e-3 relative).
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


def rne_bf16(d):
    """Round float64 values to the nearest bf16 value, ties to even (one
    rounding, straight from float64).  bf16 keeps 8 significant bits: for
    d = m * 2^e with 0.5 <= |m| < 1 the spacing is 2^(e-8).  Below the
    smallest normal, 2^-126 (e <= -126), bf16 values are subnormal and the
    spacing stays at 2^-133."""
    d = np.asarray(d, dtype=np.float64)
    _, e = np.frexp(d)
    ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    q = d / ulp  # exact: a power-of-two scaling
    lo = np.floor(q)
    frac = q - lo
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(lo, 2.0) == 1.0))
    return np.where(up, lo + 1.0, lo) * ulp


def assert_grad_parity(d_gpu, d_ref, x, lse_ref, g, targets, ignore_index=-100, what=""):
    """dlogits against the unrounded float64 gradient d64.

    The fp32 value d32 the kernel rounds may differ from d64 by the forward's
    lse tolerance carried through exp plus a few fp32 ulp, and by |g| times
    the smallest normal float32 where exp flushes to +0:
        budget = |g| * p * (ATOL + RTOL * |x - lse|) + 1e-6 * |d64| + |g| * FLT_MIN.
    fp32 outputs: |gpu - d64| <= BWD_RTOL * |d64| + budget.
    bf16 outputs: rounding to bf16 alone moves a value by up to 2^-8
    relative, more than BWD_RTOL, so the check is sharper instead: RNE is
    monotone, so gpu = RNE(d32) must lie in [RNE(d64 - budget),
    RNE(d64 + budget)]; when no rounding midpoint lies within the budget
    this interval is the single value RNE(d64).
    Ignored rows are exactly +0."""
    d = to_np(d_gpu).reshape(d_ref.shape)
    t = targets.reshape(-1).cpu().numpy()
    active = t != ignore_index
    p = np.exp(x - lse_ref[:, None])
    gg = np.abs(np.asarray(g, dtype=np.float64).reshape(-1))[:, None]
    # a masked (-inf) logit has p = 0 and no error to carry (0 * inf would be NaN)
    with np.errstate(invalid="ignore"):
        carried = np.where(p > 0, p * (ATOL + RTOL * np.abs(x - lse_ref[:, None])), 0.0)
    budget = gg * carried + 1e-6 * np.abs(d_ref) + gg * FLT_MIN
    if d_gpu.dtype == torch.bfloat16:
        ok = (d >= rne_bf16(d_ref - budget)) & (d <= rne_bf16(d_ref + budget))
    elif d_gpu.dtype == torch.float16:
        # numpy's float64 -> float16 cast rounds to nearest even, subnormals included
        with np.errstate(over="ignore"):  # bounds past the float16 range become +-inf
            lo = (d_ref - budget).astype(np.float16).astype(np.float64)
            hi = (d_ref + budget).astype(np.float16).astype(np.float64)
        ok = (d >= lo) & (d <= hi)
    else:
        ok = np.abs(d - d_ref) <= BWD_RTOL * np.abs(d_ref) + budget
    bad = ~ok & active[:, None]
    assert not bad.any(), (what, np.argwhere(bad)[:8], d[bad][:8], d_ref[bad][:8])
    if (~active).any():
        raw = d_gpu.reshape(d_ref.shape)[torch.from_numpy(~active).to(d_gpu.device)]
        assert (raw.view(torch.int32 if raw.dtype == torch.float32 else torch.int16) == 0).all()
