"""GPU parity of the bf16-rounded-logits variant of the fused LM head
("[RFC][ROCm] End-to-end optimization of bitwise VIME R/R beyond native
P/P": the FP32/BF16 rounding points belong to the versioned contract, and a
fused epilogue rounds to BF16 explicitly before the next step sees the
value).  The statistics see z = RNE_bf16(h W^T) in place of the fp32 z.

Exactness.  On lattice inputs (hidden in {-1, 0, 1}, weight k / 256) every
float32 accumulation is exact, so the kernel rounds the same z the float64
oracle rounds: the rounded logits match bit for bit and logp / lse are held
to the plain 1e-5 + 1e-5 |ref| bound.

Normal inputs.  The fp32 accumulator differs from the float64 z by at most
E = (K / 32 + 32) * 2^-24 * sum_k |h_k W_jk| (one rounding per MFMA step and
per term inside one), so where a rounding midpoint lies within E of z the
two sides may pick neighbouring bf16 values.  Those elements widen the
bound: lse by sum_j p_j * spacing_j over them, logp also by the target's
spacing when the target is one of them."""

import numpy as np
import pytest
import torch

import invariant_token_log_amd as itl
import oracle
import synth
from gpu_helpers import ATOL, RTOL, assert_logp_parity, bits, dev, rne_bf16, to_np

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _oracle(c, temperature=1.0, round_logits=True):
    return oracle.linear_logp_fwd(_np(c["hidden"]), _np(c["weight"]), c["targets"].cpu().numpy(),
                                  temperature=temperature, round_logits=round_logits)


@pytest.mark.parametrize("n,hd,v", [(64, 256, 4096), (200, 128, 1000), (1, 64, 256),
                                    (300, 4096, 2 * 256 + 17)])
@pytest.mark.parametrize("temperature", [1.0, 0.7])
def test_lattice_exact(n, hd, v, temperature):
    c = synth.lattice_linear(seed=n + v, n=n, h=hd, v=v, device=dev(), ignore_frac=0.05)
    logp, lse, z = itl.linear_logp_fwd(c["hidden"], c["weight"], c["targets"],
                                       temperature=temperature, round_logits=True,
                                       return_logits=True, logits_dtype=torch.float32)
    ref = _oracle(c, temperature)
    assert_logp_parity(logp, lse, *ref, c["targets"], what=f"round {n} {hd} {v} {temperature}")
    zr = oracle.round_bf16(_np(c["hidden"]) @ _np(c["weight"]).T)
    assert np.array_equal(to_np(z), zr)
    # the variant really differs from the plain contract on these inputs
    plain = _oracle(c, temperature, round_logits=False)
    active = c["targets"].cpu().numpy() != -100
    diff = np.maximum(np.abs(plain[0] - ref[0]), np.abs(plain[1] - ref[1]))[active]
    assert diff.max() > 2e-5


def test_normal_inputs_with_midpoint_slack():
    n, hd, v = 256, 4096, 8192
    c = synth.qwen3_linear(seed=77, n=n, h=hd, v=v, device=dev(), ignore_frac=0.05)
    logp, lse = itl.linear_logp_fwd(c["hidden"], c["weight"], c["targets"], round_logits=True)
    h, w, t = _np(c["hidden"]), _np(c["weight"]), c["targets"].cpu().numpy()
    ref_logp, ref_lse = _oracle(c)
    z = h @ w.T
    zr = oracle.round_bf16(z)
    acc_err = (hd / 32 + 32) * 2.0 ** -24 * (np.abs(h) @ np.abs(w).T)
    # spacing of bf16 around z and the distance of z to the nearest midpoint
    _, e = np.frexp(z)
    spacing = np.ldexp(1.0, np.maximum(e, -125) - 8)
    dist_mid = np.abs(np.abs(z - zr) - spacing / 2)
    ambiguous = dist_mid <= acc_err
    p = np.exp(zr - ref_lse[:, None])
    slack = (p * spacing * ambiguous).sum(1)
    active = t != -100
    rows = np.flatnonzero(active)
    slack_t = np.zeros(n)
    slack_t[rows] = (spacing * ambiguous)[rows, t[rows]]
    g_logp, g_lse = to_np(logp), to_np(lse)
    assert (np.abs(g_lse - ref_lse)[active] <=
            (ATOL + RTOL * np.abs(ref_lse) + slack)[active]).all()
    assert (np.abs(g_logp - ref_logp)[active] <=
            (ATOL + RTOL * np.abs(ref_logp) + slack + slack_t)[active]).all()
    assert (bits(logp)[torch.from_numpy(~active)] == 0).all()
    # most rows do not need the slack at all
    assert (slack_t[active] == 0).mean() > 0.5


def test_logits_output_and_invariance():
    """The returned logits are the rounded values (bf16 and fp32 outputs
    agree); logp / lse have the same bits with and without the logits output
    and for a row computed alone or in a permuted batch."""
    c = synth.qwen3_linear(seed=78, n=300, h=512, v=5000, device=dev(), ignore_frac=0.05)
    h, w, t = c["hidden"], c["weight"], c["targets"]
    l0, s0 = itl.linear_logp_fwd(h, w, t, round_logits=True)
    l1, s1, zb = itl.linear_logp_fwd(h, w, t, round_logits=True, return_logits=True)
    l2, s2, zf = itl.linear_logp_fwd(h, w, t, round_logits=True, return_logits=True,
                                     logits_dtype=torch.float32)
    for a, b in ((l0, l1), (l0, l2), (s0, s1), (s0, s2)):
        assert torch.equal(bits(a), bits(b))
    assert torch.equal(zb.float(), zf)
    plain = itl.linear_logp_fwd(h, w, t, return_logits=True, logits_dtype=torch.float32)[2]
    assert torch.equal(plain.to(torch.bfloat16), zb)
    b0 = bits(l0)
    for r in (0, 127, 128, 299):
        lr, _ = itl.linear_logp_fwd(h[r:r + 1].contiguous(), w, t[r:r + 1].contiguous(),
                                    round_logits=True)
        assert torch.equal(bits(lr), b0[r:r + 1]), r
    perm = torch.randperm(300, generator=torch.Generator().manual_seed(1)).to(dev())
    lp, _ = itl.linear_logp_fwd(h[perm].contiguous(), w, t[perm].contiguous(), round_logits=True)
    assert torch.equal(bits(lp), b0[perm.cpu()])


def test_entropy_lattice():
    c = synth.lattice_linear(seed=79, n=128, h=256, v=3000, device=dev(), ignore_frac=0.05)
    _, _, ent = itl.linear_logp_fwd(c["hidden"], c["weight"], c["targets"], round_logits=True,
                                    return_entropy=True, temperature=1.5)
    ref = oracle.linear_entropy(_np(c["hidden"]), _np(c["weight"]), c["targets"].cpu().numpy(),
                                temperature=1.5, round_logits=True)
    active = c["targets"].cpu().numpy() != -100
    err = np.abs(to_np(ent) - ref)
    assert (err[active] <= (ATOL + RTOL * np.abs(ref))[active]).all(), err.max()


@pytest.mark.parametrize("n,hd,v", [(64, 256, 4096), (257, 64, 300)])
def test_bwd_lattice(n, hd, v):
    """dh and dW of the variant against the oracle's (p from the rounded
    logits).  The kernel's dz is RNE_bf16 of a float32 value within the
    forward's tolerance of the float64 dz, so each dh / dW element is held to
    2^-8 sum |dz64| |operand| + 1e-6 (the plain backward's rule) and, on top,
    both sides' dz must round alike away from midpoints: checked through the
    exact dz recomputed from the oracle's lse."""
    c = synth.lattice_linear(seed=n * 3 + v, n=n, h=hd, v=v, device=dev(), ignore_frac=0.05)
    h, w, t = c["hidden"], c["weight"], c["targets"]
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=n + 5)[0].to(dev())
    _, lse = itl.linear_logp_fwd(h, w, t, round_logits=True)
    dh, dw = itl.linear_logp_bwd(h, w, t, lse, g, round_logits=True)
    hn, wn, tn, gn = _np(h), _np(w), t.cpu().numpy(), _np(g)
    dh64, dw64 = oracle.linear_logp_bwd(hn, wn, tn, gn, round_logits=True)
    _, lse64 = oracle.linear_logp_fwd(hn, wn, tn, round_logits=True)
    x = oracle.round_bf16(hn @ wn.T)
    p = np.exp(x - lse64[:, None])
    active = tn != -100
    dz = gn[:, None] * ((np.arange(v)[None, :] == tn[:, None]) - p)
    dz[~active] = 0.0
    tgt = np.zeros_like(dz)
    rows = np.flatnonzero(active)
    tgt[rows, tn[rows]] = np.abs(gn[rows]) * p[rows, tn[rows]] * 1e-3
    bh = 2.0 ** -8 * (np.abs(dz) @ np.abs(wn)) + tgt @ np.abs(wn) + 1e-6
    bw = 2.0 ** -8 * (np.abs(dz).T @ np.abs(hn)) + tgt.T @ np.abs(hn) + 1e-6
    assert (np.abs(_np(dh) - dh64) <= bh).all()
    assert (np.abs(_np(dw) - dw64) <= bw).all()
    # the plain backward on the same inputs differs (the rounding matters here)
    dhp, _ = itl.linear_logp_bwd(h, w, t, itl.linear_logp_fwd(h, w, t)[1], g)
    assert not torch.equal(dhp, dh)
    assert (bits(dh[torch.from_numpy(~active).to(dev())]) == 0).all()


def test_autograd_round_logits():
    c = synth.lattice_linear(seed=80, n=96, h=128, v=700, device=dev(), ignore_frac=0.05)
    h = c["hidden"].clone().requires_grad_(True)
    w = c["weight"].clone().requires_grad_(True)
    logp = itl.linear_logp(h, w, c["targets"], round_logits=True)
    g = synth.normal_matrix(1, 96, 1.0, torch.float32, seed=81)[0].to(dev())
    (logp * g).sum().backward()
    _, lse = itl.linear_logp_fwd(c["hidden"], c["weight"], c["targets"], round_logits=True)
    dh, dw = itl.linear_logp_bwd(c["hidden"], c["weight"], c["targets"], lse, g,
                                 out_dtype=torch.bfloat16, round_logits=True)
    assert torch.equal(h.grad, dh) and torch.equal(w.grad, dw)
