"""Host checks of the comparison helpers the GPU parity tests rely on.

A wrong rounding helper would make a parity test accept a wrong kernel output
or reject a right one, so it is pinned here against brute force."""

import numpy as np
import torch

from gpu_helpers import rne_bf16


def _bf16_grid():
    """Every finite bf16 value (as float64, exact) with its bit pattern,
    sorted by value; -0 is dropped in favour of +0."""
    pat = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    val = pat.view(torch.bfloat16).to(torch.float64).numpy()
    bits = np.arange(0, 1 << 16, dtype=np.int64)
    keep = np.isfinite(val) & ~((val == 0) & (bits != 0))
    order = np.argsort(val[keep], kind="stable")
    return val[keep][order], bits[keep][order]


def _nearest_bf16(d, grid, bits):
    """Brute force: the closer of the two grid neighbours; on a tie the one
    whose lowest significand bit is 0."""
    i = np.clip(np.searchsorted(grid, d), 1, len(grid) - 1)
    lo, hi = grid[i - 1], grid[i]
    dl, dh = d - lo, hi - d
    pick_hi = (dh < dl) | ((dh == dl) & ((bits[i] & 1) == 0))
    return np.where(pick_hi, hi, lo)


def test_rne_bf16_matches_brute_force():
    grid, bits = _bf16_grid()
    rng = np.random.default_rng(7)
    # magnitudes across normals and subnormals (bf16 subnormals reach 2^-133)
    e = rng.uniform(-140.0, 20.0, size=200000)
    d = np.sign(rng.standard_normal(e.size)) * np.exp2(e)
    # exact midpoints between neighbours (the ties) and the grid values themselves
    fin = grid[np.abs(grid) < 2.0 ** 20]
    mids = (fin[:-1] + fin[1:]) / 2.0
    d = np.concatenate([d, mids, fin, [0.0, -0.0, 2.0 ** -134, -(2.0 ** -134), 3 * 2.0 ** -134]])
    got = rne_bf16(d)
    want = _nearest_bf16(d, grid, bits)
    bad = got != want
    assert not bad.any(), (d[bad][:8], got[bad][:8], want[bad][:8])


def test_rne_bf16_subnormal_values():
    # 2^-133 is the smallest bf16 subnormal: half of it ties to even (0),
    # three halves tie to 2 * 2^-133
    s = 2.0 ** -133
    assert rne_bf16(0.5 * s) == 0.0
    assert rne_bf16(0.51 * s) == s
    assert rne_bf16(1.5 * s) == 2 * s
    assert rne_bf16(-16.56 * s) == -17 * s
