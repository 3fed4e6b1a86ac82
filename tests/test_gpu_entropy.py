"""GPU parity and invariance of the entropy, temperature and logits options
against the float64 oracle.

Sources: "Batch-Invariant LogP" (VIME CP=2 runtime provider: full-vocabulary
entropy on request, merged in the same fixed order as the LSE) and the fused
operator proposed in "[RFC][ROCm] End-to-end optimization of bitwise VIME R/R
beyond native P/P", Workstream 3 (temperature, return_entropy, return_logits;
logp and lse byte-identical with return_logits on or off).

Entropy tolerance (derived).  H = log(acc) - b / acc where b / acc is the
softmax mean of (x - M).  Each fp32 fold (at most 64 lane terms, 6 butterfly
levels, T merge terms) perturbs acc and b by ~1e-6 relative, and |b / acc| <=
max|x - M| <= X, so |H - H64| <= 1e-5 + 1e-5 |H64| + 1e-6 X covers it."""

import math

import numpy as np
import pytest
import torch

import invariant_token_log_amd as itl
import oracle
import synth
from gpu_helpers import ATOL, FLT_MIN, RTOL, assert_logp_parity, bits, dev, rne_bf16, to_np

pytestmark = pytest.mark.gpu

V = synth.QWEN3_VOCAB


def _ent_ok(h_gpu, x64, t, what):
    """Entropy of active rows within the derived bound; ignored rows +0."""
    h64 = oracle.entropy(x64, t)
    active = t != -100
    spread = np.zeros(len(t))
    if active.any():
        xa = x64[active]
        spread[active] = xa.max(axis=1) - xa.min(axis=1)
    g = to_np(h_gpu.reshape(-1))
    err = np.abs(g - h64)
    bound = ATOL + RTOL * np.abs(h64) + 1e-6 * spread
    bad = active & ~(err <= bound)
    assert not bad.any(), (what, np.flatnonzero(bad)[:5], err[bad][:5])
    if (~active).any():
        assert (bits(h_gpu.reshape(-1))[torch.from_numpy(~active)] == 0).all(), what
    return float(err[active].max()) if active.any() else 0.0


@pytest.mark.parametrize("dtype,v,w", [(torch.float32, 4096, 512), (torch.bfloat16, V, 4096),
                                       (torch.float16, 12345, 2048), (torch.bfloat16, 300, 512)])
def test_entropy_parity(dtype, v, w):
    n = 40
    x = synth.normal_matrix(n, v, 3.0, dtype, seed=v + 7).to(dev())
    t = synth.uniform_targets(n, v, seed=v + 8, ignore_rows=torch.tensor([2, 31])).to(dev())
    logp, lse, ent = itl.logp_fwd(x, t, -100, w, return_entropy=True)
    x64 = to_np(x)
    tn = t.cpu().numpy()
    assert_logp_parity(logp, lse, *oracle.logp_fwd(x64, tn), t, what="with entropy")
    _ent_ok(ent, x64, tn, f"entropy {dtype} {v}")


def test_entropy_closed_forms():
    """Uniform row: H = log V (up to the device log); one-hot spike: H ~ 0;
    -inf (masked) logits add nothing."""
    x = torch.zeros(3, 5000, device=dev())
    x[1, 123] = 60.0
    x[2, 2500:] = -float("inf")
    t = torch.tensor([0, 123, 7], device=dev())
    _, _, ent = itl.logp_fwd(x, t, -100, 512, return_entropy=True)
    e = ent.cpu().numpy().astype(np.float64)
    assert abs(e[0] - math.log(5000)) <= 4e-6
    assert 0.0 <= e[1] <= 1e-20 + 5000 * math.exp(-60) * 61
    assert abs(e[2] - math.log(2500)) <= 4e-6
    assert np.isfinite(e).all()


def test_entropy_bits_invariant():
    """logp and lse keep their bits with entropy on; the entropy has the same
    bits for S = 1, 2, 4 and for a row alone or permuted."""
    c = synth.qwen3_fwd(n=256, device=dev())
    x, t = c["logits"], c["targets"]
    l0, s0 = itl.logp_fwd(x, t, -100, 4096)
    l1, s1, e1 = itl.logp_fwd(x, t, -100, 4096, return_entropy=True)
    assert torch.equal(bits(l0), bits(l1)) and torch.equal(bits(s0), bits(s1))
    for shards in (2, 4):
        ls, ss, es = itl.logp_fwd(x, t, -100, 4096, shards, return_entropy=True)
        assert torch.equal(bits(es), bits(e1)) and torch.equal(bits(ls), bits(l1)), shards
    perm = torch.randperm(256, generator=torch.Generator().manual_seed(4)).to(dev())
    _, _, ep = itl.logp_fwd(x[perm].contiguous(), t[perm].contiguous(), -100, 4096,
                            return_entropy=True)
    assert torch.equal(bits(ep), bits(e1)[perm.cpu()])
    for r in (0, 17, 255):
        _, _, er = itl.logp_fwd(x[r:r + 1].clone(), t[r:r + 1].clone(), -100, 4096,
                                return_entropy=True)
        assert torch.equal(bits(er), bits(e1)[r:r + 1])


def _grad_ent_ok(d, x64, t, g, gh, what):
    """bf16 / fp32 gradient with the entropy term against float64, by the
    bracket rule of gpu_helpers with a budget widened by the entropy term."""
    _, lse64 = oracle.logp_fwd(x64, t)
    h64 = oracle.entropy(x64, t)
    d64 = oracle.logp_bwd(x64, t, g, lse=lse64) + oracle.entropy_bwd(x64, t, gh)
    logp_all = x64 - lse64[:, None]
    p = np.exp(logp_all)
    u = np.abs(logp_all + h64[:, None])
    budget = (np.abs(g)[:, None] * p * (ATOL + RTOL * np.abs(logp_all))
              + np.abs(gh)[:, None] * p * ((2 * ATOL + RTOL * np.abs(logp_all)
                                            + RTOL * np.abs(h64)[:, None]) * (1 + u))
              + 1e-6 * np.abs(d64)
              + (np.abs(g)[:, None] + np.abs(gh)[:, None] * (1 + u)) * FLT_MIN)
    got = to_np(d).reshape(d64.shape)
    if d.dtype == torch.bfloat16:
        ok = (got >= rne_bf16(d64 - budget)) & (got <= rne_bf16(d64 + budget))
    elif d.dtype == torch.float16:
        # numpy's float64 -> float16 cast rounds to nearest even, subnormals
        # included (a bound past the float16 range becomes +-inf)
        with np.errstate(over="ignore"):
            ok = ((got >= (d64 - budget).astype(np.float16).astype(np.float64))
                  & (got <= (d64 + budget).astype(np.float16).astype(np.float64)))
    else:
        ok = np.abs(got - d64) <= 2e-3 * np.abs(d64) + budget
    active = t != -100
    bad = ~ok & active[:, None]
    assert not bad.any(), (what, np.argwhere(bad)[:5], got[bad][:5], d64[bad][:5])


@pytest.mark.parametrize("dtype,v,w", [(torch.float32, 4096, 512), (torch.bfloat16, V, 4096)])
def test_entropy_backward_parity(dtype, v, w):
    n = 24
    x = synth.normal_matrix(n, v, 3.0, dtype, seed=v + 9).to(dev())
    t = synth.uniform_targets(n, v, seed=v + 10, ignore_rows=torch.tensor([5])).to(dev())
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=v + 11)[0].to(dev())
    gh = synth.normal_matrix(1, n, 1.0, torch.float32, seed=v + 12)[0].to(dev())
    _, lse, ent = itl.logp_fwd(x, t, -100, w, return_entropy=True)
    d = itl.logp_bwd(x, t, lse, g, -100, w, entropy=ent, grad_entropy=gh)
    _grad_ent_ok(d, to_np(x), t.cpu().numpy(), to_np(g), to_np(gh), f"ent bwd {dtype}")
    ign = (t == -100)
    assert (d[ign].view(torch.int16 if dtype != torch.float32 else torch.int32) == 0).all()


def test_entropy_backward_zero_grad_same_bits():
    """gH = 0 leaves every gradient bit of the plain backward unchanged."""
    x = synth.normal_matrix(16, 5000, 2.0, torch.bfloat16, seed=3).to(dev())
    t = synth.uniform_targets(16, 5000, seed=4).to(dev())
    g = torch.linspace(-1, 1, 16, device=dev())
    _, lse, ent = itl.logp_fwd(x, t, -100, 512, return_entropy=True)
    a = itl.logp_bwd(x, t, lse, g, -100, 512)
    b = itl.logp_bwd(x, t, lse, g, -100, 512, entropy=ent, grad_entropy=torch.zeros_like(g))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_autograd_logp_and_entropy():
    """batch_invariant_logp(..., return_entropy=True): (logp, H) both
    differentiable; the gradient equals one logp_bwd call with the entropy
    term (bit for bit)."""
    x = synth.normal_matrix(24, 700, 2.0, torch.bfloat16, seed=5).view(2, 12, 700).to(dev())
    t = synth.uniform_targets(24, 700, seed=6).view(2, 12).to(dev())
    t[1, 3] = -100
    xx = x.clone().requires_grad_(True)
    logp, ent = itl.batch_invariant_logp(xx, t, -100, 512, return_entropy=True)
    assert logp.shape == t.shape and ent.shape == t.shape
    (logp.sum() + 0.5 * ent.sum()).backward()
    _, lse, e2 = itl.logp_fwd(x, t, -100, 512, return_entropy=True)
    d = itl.logp_bwd(x, t, lse, torch.ones(24, device=dev()), -100, 512, entropy=e2,
                     grad_entropy=torch.full((24,), 0.5, device=dev()))
    assert torch.equal(xx.grad.view(torch.int16), d.view(torch.int16))


# ----- fused LM head: temperature, entropy, logits -----------------------------

@pytest.mark.parametrize("temp", [0.7, 1.0, 2.0, 1.3, 0.05, 25.0])
def test_linear_temperature_entropy_parity(temp):
    c = synth.qwen3_linear(seed=21, n=200, h=256, v=3000, device=dev(), ignore_frac=0.05)
    h, w, t = c["hidden"], c["weight"], c["targets"]
    logp, lse, ent = itl.linear_logp_fwd(h, w, t, temperature=temp, return_entropy=True)
    hn, wn, tn = to_np(h), to_np(w), t.cpu().numpy()
    ref = oracle.linear_logp_fwd(hn, wn, tn, temperature=temp)
    assert_logp_parity(logp, lse, *ref, t, what=f"linear T={temp}")
    x64 = oracle.linear_logits(hn, wn) / temp
    _ent_ok(ent, x64, tn, f"linear entropy T={temp}")


def test_linear_options_keep_bits():
    """logp and lse are byte-identical with return_logits / return_entropy on
    or off; temperature 1 is the plain operator; bf16 logits are the RNE of
    the fp32 logits, which match the oracle's h W^T within the K walk."""
    c = synth.qwen3_linear(seed=22, n=300, h=512, v=2000, device=dev(), ignore_frac=0.05)
    h, w, t = c["hidden"], c["weight"], c["targets"]
    l0, s0 = itl.linear_logp_fwd(h, w, t)
    l1, s1, e1, z32 = itl.linear_logp_fwd(h, w, t, temperature=1.0, return_entropy=True,
                                          return_logits=True, logits_dtype=torch.float32)
    l2, s2, z16 = itl.linear_logp_fwd(h, w, t, return_logits=True)
    for a, b in ((l0, l1), (s0, s1), (l0, l2), (s0, s2)):
        assert torch.equal(bits(a), bits(b))
    assert torch.equal(z16.view(torch.int16), z32.to(torch.bfloat16).view(torch.int16))
    z64 = oracle.linear_logits(to_np(h), to_np(w))
    scale = np.abs(to_np(h)) @ np.abs(to_np(w)).T
    assert (np.abs(to_np(z32) - z64) <= 1e-5 * scale + 1e-6).all()
    # the zero-weight closed form: z = 0, logp = -log V, H = log V
    wz = torch.zeros_like(w)
    _, _, ez = itl.linear_logp_fwd(h, wz, t, temperature=0.5, return_entropy=True)
    act = (t != -100).cpu()
    assert (np.abs(ez.cpu()[act].numpy() - math.log(2000)) <= 4e-6).all()


def _linear_bwd_bounds(hn, wn, tn, gn, ghn, temp):
    """Elementwise bounds of dh, dW with temperature and the entropy term."""
    x = oracle.linear_logits(hn, wn) / temp
    _, lse = oracle.logp_fwd(x, tn)
    ent = oracle.entropy(x, tn)
    dx = oracle.logp_bwd(x, tn, gn, lse=lse) + oracle.entropy_bwd(x, tn, ghn)
    dz = dx / temp
    active = tn != -100
    p = np.exp(x - lse[:, None])
    u = np.abs(x - lse[:, None] + ent[:, None])
    extra = (np.abs(gn)[:, None] * p * 1e-3 + np.abs(ghn)[:, None] * p * 1e-3 * (1 + u)) / temp
    extra[~active] = 0.0
    adz = np.abs(dz)
    bh = 2.0 ** -8 * (adz @ np.abs(wn)) + extra @ np.abs(wn) + 1e-6
    bw = 2.0 ** -8 * (adz.T @ np.abs(hn)) + extra.T @ np.abs(hn) + 1e-6
    return bh, bw


@pytest.mark.parametrize("temp", [1.0, 0.8, 0.05, 25.0])
def test_linear_bwd_temperature_entropy_parity(temp):
    c = synth.qwen3_linear(seed=23, n=130, h=256, v=1500, device=dev(), ignore_frac=0.05)
    h, w, t = c["hidden"], c["weight"], c["targets"]
    g = synth.normal_matrix(1, 130, 1.0, torch.float32, seed=24)[0].to(dev())
    gh = synth.normal_matrix(1, 130, 1.0, torch.float32, seed=25)[0].to(dev())
    _, lse, ent = itl.linear_logp_fwd(h, w, t, temperature=temp, return_entropy=True)
    dh, dw = itl.linear_logp_bwd(h, w, t, lse, g, temperature=temp, entropy=ent,
                                 grad_entropy=gh)
    hn, wn, tn, gn, ghn = to_np(h), to_np(w), t.cpu().numpy(), to_np(g), to_np(gh)
    dh64, dw64 = oracle.linear_logp_bwd(hn, wn, tn, gn, temperature=temp, grad_entropy=ghn)
    bh, bw = _linear_bwd_bounds(hn, wn, tn, gn, ghn, temp)
    eh, ew = np.abs(to_np(dh) - dh64), np.abs(to_np(dw) - dw64)
    assert (eh <= bh).all(), (np.argwhere(eh > bh)[:5], eh.max())
    assert (ew <= bw).all(), (np.argwhere(ew > bw)[:5], ew.max())
    # gH = 0 and T = 1 reproduce the plain backward bit for bit
    if temp == 1.0:
        a = itl.linear_logp_bwd(h, w, t, lse, g)
        b = itl.linear_logp_bwd(h, w, t, lse, g, entropy=ent, grad_entropy=torch.zeros_like(gh))
        assert torch.equal(bits(a[0]), bits(b[0])) and torch.equal(bits(a[1]), bits(b[1]))


def test_linear_autograd_with_entropy():
    c = synth.qwen3_linear(seed=26, n=96, h=128, v=700, device=dev())
    h, w, t = c["hidden"], c["weight"], c["targets"]
    hh = h.clone().requires_grad_(True)
    ww = w.clone().requires_grad_(True)
    logp, ent = itl.linear_logp(hh, ww, t, temperature=0.9, return_entropy=True)
    (logp.sum() - 0.25 * ent.sum()).backward()
    _, lse, e2 = itl.linear_logp_fwd(h, w, t, temperature=0.9, return_entropy=True)
    dh, dw = itl.linear_logp_bwd(h, w, t, lse, torch.ones(96, device=dev()), temperature=0.9,
                                 entropy=e2, grad_entropy=torch.full((96,), -0.25, device=dev()),
                                 out_dtype=torch.bfloat16)
    assert torch.equal(hh.grad.view(torch.int16), dh.view(torch.int16))
    assert torch.equal(ww.grad.view(torch.int16), dw.view(torch.int16))
