"""GPU parity and invariance of the fused LM-head + logp against the float64
oracle ("[RFC][ROCm] End-to-end optimization of bitwise VIME R/R beyond
native P/P", Workstream 3)."""

import math

import numpy as np
import pytest
import torch

import invariant_token_log_amd as itl
import oracle
import synth
from gpu_helpers import assert_logp_parity, bits, dev, to_np

pytestmark = pytest.mark.gpu


def _oracle(h, w, t, ignore_index=-100):
    return oracle.linear_logp_fwd(h.float().cpu().numpy(), w.float().cpu().numpy(),
                                  t.cpu().numpy(), ignore_index)


@pytest.mark.parametrize("n,hd,v", [(64, 256, 4096), (200, 128, 1000), (1, 64, 256),
                                    (129, 512, 2 * 256 + 17), (300, 4096, 4096)])
def test_tiny_brute(n, hd, v):
    """Small problems with ragged N (not a multiple of 128) and ragged V."""
    c = synth.qwen3_linear(seed=n + v, n=n, h=hd, v=v, device=dev(), ignore_frac=0.05)
    logp, lse = itl.linear_logp_fwd(c["hidden"], c["weight"], c["targets"])
    ref = _oracle(c["hidden"], c["weight"], c["targets"])
    assert_logp_parity(logp, lse, *ref, c["targets"], what=f"linear {n} {hd} {v}")


def test_identity_weight_matches_logp():
    """W = I (V = H): z = h exactly in fp32 under any K order, so the fused
    result matches the oracle's logp of h itself."""
    n, hd = 96, 256
    h = synth.normal_matrix(n, hd, 3.0, torch.bfloat16, seed=1).to(dev())
    w = torch.eye(hd, dtype=torch.bfloat16, device=dev())
    t = synth.uniform_targets(n, hd, seed=2, ignore_rows=torch.tensor([4])).to(dev())
    logp, lse = itl.linear_logp_fwd(h, w, t)
    ref = oracle.logp_fwd(h.float().cpu().numpy(), t.cpu().numpy())
    assert_logp_parity(logp, lse, *ref, t, what="identity")


@pytest.mark.parametrize("v", [256, 1000, synth.QWEN3_VOCAB])
def test_zero_weight_is_minus_log_v(v):
    """W = 0: every z is 0, the sums are exact integers, and the result has
    the same bits as logp_fwd on a zero row."""
    n, hd = 8, 64
    h = synth.normal_matrix(n, hd, 1.0, torch.bfloat16, seed=3).to(dev())
    w = torch.zeros(v, hd, dtype=torch.bfloat16, device=dev())
    t = torch.arange(n, device=dev()) * (v // n)
    logp, lse = itl.linear_logp_fwd(h, w, t)
    want = np.float32(-math.log(v))
    assert (np.abs(to_np(logp) - float(want)) <= 2 * abs(float(np.spacing(want)))).all()
    zrow = torch.zeros(n, v, dtype=torch.float32, device=dev())
    lz, sz = itl.logp_fwd(zrow, t, -100, 256)
    assert torch.equal(bits(logp), bits(lz)) and torch.equal(bits(lse), bits(sz))


def test_empty_and_all_ignored():
    """N = 0: the fused forward and the streaming backward return empty
    outputs.  Every row ignored: logp, lse and entropy are +0, and dh and dW
    (sums of zero dz terms) are +0 too."""
    hd, v = 64, 1000
    w = synth.normal_matrix(v, hd, 0.02, torch.bfloat16, seed=5).to(dev())
    h0 = torch.empty(0, hd, dtype=torch.bfloat16, device=dev())
    t0 = torch.empty(0, dtype=torch.int64, device=dev())
    logp, lse, ent = itl.linear_logp_fwd(h0, w, t0, return_entropy=True)
    assert logp.numel() == 0 and lse.numel() == 0 and ent.numel() == 0
    e0 = torch.empty(0, dtype=torch.float32, device=dev())
    d = itl.logp_bwd(torch.empty(0, v, dtype=torch.bfloat16, device=dev()), t0, e0, e0, -100, 512)
    assert d.shape == (0, v)
    n = 300
    h = synth.normal_matrix(n, hd, 1.0, torch.bfloat16, seed=6).to(dev())
    t = torch.full((n,), -100, dtype=torch.int64, device=dev())
    logp, lse, ent = itl.linear_logp_fwd(h, w, t, return_entropy=True)
    for x in (logp, lse, ent):
        assert (bits(x) == 0).all()
    dh, dw = itl.linear_logp_bwd(h, w, t, lse, torch.ones(n, device=dev()))
    assert (bits(dh) == 0).all() and (bits(dw) == 0).all()


def test_row_invariance():
    """A row's z, statistics and logp do not depend on N, its position in the
    128-row block, or its neighbours."""
    c = synth.qwen3_linear(seed=44, n=300, h=512, v=5000, device=dev())
    h, w, t = c["hidden"], c["weight"], c["targets"]
    base, _ = itl.linear_logp_fwd(h, w, t)
    b0 = bits(base)
    for r in [0, 5, 127, 128, 299]:
        lr, _ = itl.linear_logp_fwd(h[r:r + 1].contiguous(), w, t[r:r + 1].contiguous())
        assert torch.equal(bits(lr), b0[r:r + 1]), r
    perm = torch.randperm(300, generator=torch.Generator().manual_seed(0)).to(dev())
    lp, _ = itl.linear_logp_fwd(h[perm].contiguous(), w, t[perm].contiguous())
    assert torch.equal(bits(lp), b0[perm.cpu()])
    again, _ = itl.linear_logp_fwd(h, w, t)
    assert torch.equal(bits(again), b0)


def test_full_size_sampled():
    """Qwen3-8B LM head (N = 4096, H = 4096, V = 151936) at the benchmarked
    launch: 48 sampled rows against the float64 oracle."""
    c = synth.qwen3_linear(device=dev())
    h, w, t = c["hidden"], c["weight"], c["targets"]
    logp, lse = itl.linear_logp_fwd(h, w, t)
    rows = torch.tensor(list(range(0, 4096, 89)) + [4095], device=dev())
    ref = _oracle(h[rows], w, t[rows])
    assert_logp_parity(logp[rows], lse[rows], *ref, t[rows], what="linear full")
    assert torch.isfinite(logp).all()
    # the prepared weight (the forward's blocked copy) gives the same bits
    pw = itl.prepare_weight(w)
    lp2, lse2 = itl.linear_logp_fwd(h, w, t, prepared_weight=pw)
    assert torch.equal(bits(lp2), bits(logp)) and torch.equal(bits(lse2), bits(lse))


def test_int32_targets_same_bits():
    c = synth.qwen3_linear(seed=77, n=140, h=256, v=3000, device=dev(), ignore_frac=0.05)
    a, la = itl.linear_logp_fwd(c["hidden"], c["weight"], c["targets"])
    b, lb = itl.linear_logp_fwd(c["hidden"], c["weight"], c["targets"].to(torch.int32))
    assert torch.equal(bits(a), bits(b)) and torch.equal(bits(la), bits(lb))


def test_narrow_and_wide_tiles_same_bits():
    """N <= 64 runs the 64-row tile, N <= 128 the 128-row tile, N > 128 the
    256-row tile: the same rows get the same bits from all three (logp, lse,
    entropy and the logits output)."""
    c = synth.qwen3_linear(seed=91, n=129, h=512, v=3000, device=dev(), ignore_frac=0.05)
    h, w, t = c["hidden"], c["weight"], c["targets"]
    wide = itl.linear_logp_fwd(h, w, t, return_entropy=True, return_logits=True,
                               logits_dtype=torch.float32)
    for rows in (128, 65, 64, 1):
        narrow = itl.linear_logp_fwd(h[:rows].contiguous(), w, t[:rows].contiguous(),
                                     return_entropy=True, return_logits=True,
                                     logits_dtype=torch.float32)
        for a, b in zip(wide, narrow):
            assert torch.equal(bits(a[:rows]), bits(b)), rows


@pytest.mark.parametrize("n,hd,v", [(300, 256, 190 * 256 + 77), (1000, 256, 40000),
                                    (300, 256, 40000)])
def test_tile_queue_grids(n, hd, v):
    """Tile counts where the 256-row kernel hands its last tiles out at run
    time (ranges of unequal length over the XCDs, extra workgroups that find
    nothing left), and (300 x 40000: 314 tiles, a final round under a quarter
    full) where the last 29 vocabulary blocks go to the 64-row tile instead:
    every row has the bits the 64-row tile gives it alone, repeated calls
    agree, and sampled rows match the oracle."""
    c = synth.qwen3_linear(seed=n + 7, n=n, h=hd, v=v, device=dev(), ignore_frac=0.05)
    h, w, t = c["hidden"], c["weight"], c["targets"]
    wide = itl.linear_logp_fwd(h, w, t, return_entropy=True, return_logits=True,
                               logits_dtype=torch.float32)
    again = itl.linear_logp_fwd(h, w, t, return_entropy=True, return_logits=True,
                                logits_dtype=torch.float32)
    for a, b in zip(wide, again):
        assert torch.equal(bits(a), bits(b))
    for r0 in (0, n - 64):
        narrow = itl.linear_logp_fwd(h[r0:r0 + 64].contiguous(), w, t[r0:r0 + 64].contiguous(),
                                     return_entropy=True, return_logits=True,
                                     logits_dtype=torch.float32)
        for a, b in zip(wide, narrow):
            assert torch.equal(bits(a[r0:r0 + 64]), bits(b)), r0
    rows = torch.tensor([0, 1, n // 3, n // 2, n - 2, n - 1], device=dev())
    ref = _oracle(h[rows], w, t[rows])
    assert_logp_parity(wide[0][rows], wide[1][rows], *ref, t[rows], what=f"queue {n} {v}")
