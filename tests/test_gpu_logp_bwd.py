"""GPU parity and invariance of logp_bwd against the float64 oracle.

Sources: "Batch-Invariant LogP" (Batch-Invariance: tile-wise backward from
the saved per-row lse; Reference Semantics: ignored rows get zero gradient;
Entry Point: logp.sum().backward())."""

import numpy as np
import pytest
import torch

import invariant_token_log_amd as itl
import oracle
import synth
from gpu_helpers import assert_grad_parity, assert_logp_parity, bits, dev, to_np

pytestmark = pytest.mark.gpu

V = synth.QWEN3_VOCAB


def _check(x, t, g, w, what):
    logp, lse = itl.logp_fwd(x, t, -100, w)
    d = itl.logp_bwd(x, t, lse, g, -100, w)
    xn = x.detach().float().cpu().numpy().astype(np.float64)
    tn = t.cpu().numpy()
    _, lse64 = oracle.logp_fwd(xn, tn)
    d64 = oracle.logp_bwd(xn, tn, g.cpu().numpy(), lse=lse64)
    assert_grad_parity(d, d64, xn, lse64, g.cpu().numpy(), t, what=what)
    return d


def test_tiny_fp32():
    c = synth.tiny_fp32()
    g = synth.normal_matrix(1, 64, 1.0, torch.float32, seed=21)[0].to(dev())
    _check(c["logits"].to(dev()), c["targets"].to(dev()), g, 512, "tiny fp32")


@pytest.mark.parametrize("v,w", [(8, 512), (300, 512), (4099, 1024), (V, 4096)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_ragged(v, w, dtype):
    n = 24
    x = synth.normal_matrix(n, v, 3.0, dtype, seed=v).to(dev())
    t = synth.uniform_targets(n, v, seed=v + 1, ignore_rows=torch.tensor([2, 5])).to(dev())
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=v + 2)[0].to(dev())
    _check(x, t, g, w, f"ragged {v} {dtype}")


def test_qwen_rows_with_spikes():
    c = synth.qwen3_fwd(n=256, device=dev())
    g = synth.normal_matrix(1, 256, 1.0, torch.float32, seed=5)[0].to(dev())
    # put some targets on the spikes: the target column then has 1 - p ~ 0
    t = c["targets"].clone()
    sr = c["spike_rows"][c["spike_rows"] < 256]
    t[sr.to(dev())] = c["spike_cols"][c["spike_rows"] < 256].to(dev())
    _check(c["logits"], t, g, 4096, "qwen spikes")


def test_in_place_and_invariance():
    """dlogits may overwrite the logits; rows are invariant to batch order."""
    n = 64
    x = synth.normal_matrix(n, V, 3.0, torch.bfloat16, seed=8).to(dev())
    t = synth.uniform_targets(n, V, seed=9, ignore_rows=torch.tensor([1, 60])).to(dev())
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=10)[0].to(dev())
    _, lse = itl.logp_fwd(x, t, -100, 4096)
    d = itl.logp_bwd(x, t, lse, g, -100, 4096)
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(1)).to(dev())
    dp = itl.logp_bwd(x[perm].contiguous(), t[perm].contiguous(), lse[perm].contiguous(),
                      g[perm].contiguous(), -100, 4096)
    assert torch.equal(dp.view(torch.int16), d[perm].view(torch.int16))
    x2 = x.clone()
    itl.logp_bwd(x2, t, lse, g, -100, 4096, dlogits_out=x2)
    assert torch.equal(x2.view(torch.int16), d.view(torch.int16))
    # a row alone, unaligned
    buf = torch.empty(1, V + 1, dtype=torch.bfloat16, device=dev())
    xr = buf[:, 1:]
    xr.copy_(x[7:8])
    dr = itl.logp_bwd(xr, t[7:8].clone(), lse[7:8].clone(), g[7:8].clone(), -100, 4096)
    assert torch.equal(dr.view(torch.int16), d[7:8].view(torch.int16))


def test_tile_width_is_bit_neutral():
    n = 8
    x = synth.normal_matrix(n, 5000, 2.0, torch.bfloat16, seed=3).to(dev())
    t = synth.uniform_targets(n, 5000, seed=4).to(dev())
    g = torch.ones(n, device=dev())
    _, lse = itl.logp_fwd(x, t, -100, 512)
    a = itl.logp_bwd(x, t, lse, g, -100, 512)
    b = itl.logp_bwd(x, t, lse, g, -100, 8192)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_autograd_sum_backward():
    """logp.sum().backward() fills logits.grad with g = 1."""
    x = synth.normal_matrix(2 * 4, 300, 1.0, torch.bfloat16, seed=0).view(2, 4, 300).to(dev())
    x.requires_grad_(True)
    t = synth.uniform_targets(8, 300, seed=1).view(2, 4).to(dev())
    t[0, 0] = -100
    out = itl.batch_invariant_logp(x, t, -100, 512)
    out.sum().backward()
    assert x.grad.shape == x.shape and x.grad.dtype == torch.bfloat16
    assert (x.grad[0, 0].view(torch.int16) == 0).all()
    xn = x.detach().float().cpu().numpy().reshape(8, 300).astype(np.float64)
    tn = t.reshape(-1).cpu().numpy()
    _, lse64 = oracle.logp_fwd(xn, tn)
    d64 = oracle.logp_bwd(xn, tn, np.ones(8), lse=lse64)
    assert_grad_parity(x.grad.reshape(8, 300), d64, xn, lse64, np.ones(8), t, what="autograd")


def test_full_size_sampled():
    """N = 8192 Qwen3-vocab forward+backward at the benchmarked launch:
    sampled rows against the oracle, every ignored row exactly zero, and the
    gradient row sums near zero."""
    c = synth.qwen3_fwd_bwd(device=dev())
    x, t, g = c["logits"], c["targets"], c["grad"]
    logp, lse = itl.logp_fwd(x, t, -100, 4096)
    d = itl.logp_bwd(x, t, lse, g, -100, 4096)
    rows = torch.tensor(list(range(0, 8192, 97)) + [8191], device=dev())
    xn = x[rows].float().cpu().numpy().astype(np.float64)
    tn = t[rows].cpu().numpy()
    _, lse64 = oracle.logp_fwd(xn, tn)
    d64 = oracle.logp_bwd(xn, tn, g[rows].cpu().numpy(), lse=lse64)
    assert_grad_parity(d[rows], d64, xn, lse64, g[rows].cpu().numpy(), t[rows], what="full")
    ign = (t == -100)
    assert (d[ign].view(torch.int16) == 0).all()
    rs = d[~ign][:512].float().sum(dim=1).abs() / g[~ign][:512].abs()
    assert (rs < 0.05).all()


def test_past_two_to_the_31_elements():
    """14200 Qwen3-vocab rows hold 2.16e9 logits, more than 2^31: rows on both
    sides of element 2^31 and the last rows get the oracle's logp, lse and
    dlogits, the last rows computed alone give the same bits, and the 2-shard
    forward agrees bit for bit, so no offset wraps at 32 bits."""
    n = 14200
    assert n * V > 2 ** 31
    x = synth.normal_matrix(n, V, 3.0, torch.bfloat16, seed=81, device=dev())
    t = synth.uniform_targets(n, V, seed=82, device=dev())
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=83, device=dev())[0]
    logp, lse = itl.logp_fwd(x, t, -100, 4096)
    d = itl.logp_bwd(x, t, lse, g, -100, 4096)
    first_past = -(-(2 ** 31) // V)  # the first row that starts past element 2^31
    rows = torch.tensor([0, first_past - 1, first_past, n - 2, n - 1], device=dev())
    xn = x[rows].float().cpu().numpy().astype(np.float64)
    tn = t[rows].cpu().numpy()
    ref_logp, ref_lse = oracle.logp_fwd(xn, tn)
    assert_logp_parity(logp[rows], lse[rows], ref_logp, ref_lse, t[rows], what="2^31 fwd")
    d64 = oracle.logp_bwd(xn, tn, g[rows].cpu().numpy(), lse=ref_lse)
    assert_grad_parity(d[rows], d64, xn, ref_lse, g[rows].cpu().numpy(), t[rows], what="2^31 bwd")
    tail = slice(n - 8, n)
    lp_a, lse_a = itl.logp_fwd(x[tail].contiguous(), t[tail].contiguous(), -100, 4096)
    assert torch.equal(bits(lp_a), bits(logp[tail])) and torch.equal(bits(lse_a), bits(lse[tail]))
    d_a = itl.logp_bwd(x[tail].contiguous(), t[tail].contiguous(), lse_a, g[tail].contiguous(),
                       -100, 4096)
    assert torch.equal(d_a.view(torch.int16), d[tail].view(torch.int16))
    lp2, lse2 = itl.logp_fwd(x, t, -100, 4096, num_shards=2)
    assert torch.equal(bits(lp2), bits(logp)) and torch.equal(bits(lse2), bits(lse))


@pytest.mark.parametrize("v,w", [(300, 512), (V, 4096)])
def test_fp16_backward(v, w):
    """fp16 dlogits: each value is the nearest fp16 (subnormals included) of
    the fp32 gradient within the error budget."""
    n = 24
    x = synth.normal_matrix(n, v, 3.0, torch.float16, seed=v + 3).to(dev())
    t = synth.uniform_targets(n, v, seed=v + 4, ignore_rows=torch.tensor([1])).to(dev())
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=v + 5)[0].to(dev())
    d = _check(x, t, g, w, f"fp16 {v}")
    assert d.dtype == torch.float16


def test_int32_targets_same_bits():
    x = synth.normal_matrix(16, 3000, 2.0, torch.bfloat16, seed=31).to(dev())
    t = synth.uniform_targets(16, 3000, seed=32, ignore_rows=torch.tensor([3])).to(dev())
    g = torch.linspace(-2, 2, 16, device=dev())
    _, lse = itl.logp_fwd(x, t, -100, 512)
    a = itl.logp_bwd(x, t, lse, g, -100, 512)
    b = itl.logp_bwd(x, t.to(torch.int32), lse, g, -100, 512)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_tall_batch_grid_stride():
    """More rows than one grid dimension holds (65535): the backward walks the
    rows grid-stride, the forward runs one workgroup per row; parity on every
    element, the 2-shard forward has the same bits, and dlogits of the rows
    past 65535 equal those of the same rows computed alone."""
    n, v = 70000, 512
    x = synth.normal_matrix(n, v, 3.0, torch.bfloat16, seed=71).to(dev())
    ign = synth.choose_rows(n, 0.05, seed=72)
    t = synth.uniform_targets(n, v, seed=73, ignore_rows=ign).to(dev())
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=74)[0].to(dev())
    d = _check(x, t, g, 512, "tall")
    logp1, lse1 = itl.logp_fwd(x, t, -100, 512)
    logp2, lse2 = itl.logp_fwd(x, t, -100, 512, num_shards=2)
    assert torch.equal(logp1.view(torch.int32), logp2.view(torch.int32))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))
    tail = slice(65530, n)
    d_tail = itl.logp_bwd(x[tail].contiguous(), t[tail].contiguous(), lse1[tail].contiguous(),
                          g[tail].contiguous(), -100, 512)
    assert torch.equal(d_tail.view(torch.int16), d[tail].view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_invalid_target_rows_get_minus_p(dtype):
    """A row whose active target lies outside [0, V) gets d = RNE(-g p) on
    every column: the gradient with no one-hot term.  Reference: the oracle's
    gradient of the same row with a valid target t' (the oracle refuses an
    invalid one) minus g at column t'.  Valid rows of the same batch keep the
    plain parity, ignored rows stay +0."""
    v = 5000
    x = synth.normal_matrix(6, v, 2.0, dtype, seed=31).to(dev())
    t = torch.tensor([1, v, -100, -1, v - 1, 123456789], device=dev())
    g = synth.normal_matrix(1, 6, 1.0, torch.float32, seed=32)[0].to(dev())
    _, lse = itl.logp_fwd(x, t, -100, 512)
    d = itl.logp_bwd(x, t, lse, g, -100, 512)
    xn = x.float().cpu().numpy().astype(np.float64)
    gn = g.cpu().numpy().astype(np.float64)
    tn = t.cpu().numpy()
    t_valid = np.where((tn >= 0) & (tn < v), tn, 0)
    t_valid[tn == -100] = -100
    _, lse64 = oracle.logp_fwd(xn, t_valid)
    d64 = oracle.logp_bwd(xn, t_valid, gn, lse=lse64)
    invalid = np.flatnonzero((tn != -100) & ((tn < 0) | (tn >= v)))
    d64[invalid, 0] -= gn[invalid]  # remove the one-hot term of the stand-in target 0
    assert_grad_parity(d, d64, xn, lse64, gn, t, what="invalid targets")
