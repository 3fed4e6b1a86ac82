"""Pins of the CPU oracle to things other than itself (CPU only).

Each test fixes the oracle against a closed form, a brute-force evaluation,
an independent library routine or an invariant of the mathematics, chosen so
that a plausible slip in the oracle (a dropped max shift, a wrong sign, a
wrong column, a transposed operand, a lost padding rule) fails at least one.
Sources: "Batch-Invariant LogP" (opening definition, Reference Semantics,
Tensor Parallel, Batch-Invariance) and the fused LM-head operator of
"[RFC][ROCm] End-to-end optimization of bitwise VIME R/R beyond native P/P"
(Workstream 3).
"""

import json
import math
import os
from decimal import Decimal

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _golden_row(spec, v):
    kind = spec["kind"]
    if kind == "constant":
        return np.full(v, spec["value"], dtype=np.float64)
    if kind == "log_ladder":
        return np.array([math.log(j + 1) for j in range(v)], dtype=np.float64)
    if kind == "two_level":
        x = np.full(v, spec["b"], dtype=np.float64)
        x[: spec["k"]] = spec["a"]
        return x
    if kind == "spike":
        x = np.zeros(v, dtype=np.float64)
        x[spec["col"]] = spec["height"]
        return x
    raise ValueError(kind)


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_closed_forms(case):
    """logp, lse and gradient against decimal closed forms (golden file)."""
    v = case["v"]
    x = _golden_row(case["row"], v)
    targets = [e["target"] for e in case["targets"]]
    rows = np.tile(x, (len(targets), 1))
    logp, lse = oracle.logp_fwd(rows, targets)
    want_lse = float(Decimal(case["lse"]))
    for i, e in enumerate(case["targets"]):
        want = float(Decimal(e["logp"]))
        assert abs(logp[i] - want) <= 1e-12 * max(1.0, abs(want)), (i, logp[i], want)
        assert abs(lse[i] - want_lse) <= 1e-12 * max(1.0, abs(want_lse))
    d = oracle.logp_bwd(rows, targets, np.ones(len(targets)))
    for i, e in enumerate(case["targets"]):
        for j, val in e["grad_g1"].items():
            assert abs(d[i, int(j)] - float(Decimal(val))) <= 1e-12, (i, j)


def _brute(x_row, t):
    total = math.fsum(math.exp(float(a)) for a in x_row)
    return math.log(math.exp(float(x_row[t])) / total)


def test_brute_force_v8():
    """Tiny V: direct log(exp(x_t)/sum exp(x)) without any max shift."""
    c = synth.tiny_v8(n=64)
    x = c["logits"].numpy()
    t = c["targets"].numpy()
    logp, lse = oracle.logp_fwd(x, t)
    for r in range(x.shape[0]):
        assert abs(logp[r] - _brute(x[r], t[r])) <= 1e-14
        lse_b = math.log(math.fsum(math.exp(float(a)) for a in x[r]))
        assert abs(lse[r] - lse_b) <= 1e-14 * max(1.0, abs(lse_b))


def test_library_log_softmax():
    """The pages' reference semantics evaluated by torch in float64."""
    c = synth.tiny_fp32()
    x = c["logits"].double()
    t = c["targets"]
    logp, lse = oracle.logp_fwd(c["logits"].numpy(), t.numpy(), c["ignore_index"])
    active = t != c["ignore_index"]
    ref = torch.log_softmax(x, dim=-1).gather(
        -1, t.clamp(min=0).unsqueeze(-1)).squeeze(-1)
    ref = torch.where(active, ref, torch.zeros_like(ref)).numpy()
    np.testing.assert_allclose(logp, ref, rtol=1e-13, atol=1e-13)
    ref_lse = torch.logsumexp(x, dim=-1).numpy()
    np.testing.assert_allclose(lse[active.numpy()], ref_lse[active.numpy()],
                               rtol=1e-13, atol=0)
    assert np.all(logp[~active.numpy()] == 0.0)
    assert np.all(lse[~active.numpy()] == 0.0)


def test_library_log_softmax_large_v():
    """bf16 Qwen3-vocab rows (widened exactly to float32) vs torch float64."""
    c = synth.qwen3_fwd(n=24)
    x32 = c["logits"].float()
    t = c["targets"]
    logp, lse = oracle.logp_fwd(x32.numpy(), t.numpy())
    active = (t != -100)
    ref = torch.log_softmax(x32.double(), -1).gather(
        -1, t.clamp(min=0).unsqueeze(-1)).squeeze(-1).numpy()
    a = active.numpy()
    np.testing.assert_allclose(logp[a], ref[a], rtol=1e-13, atol=1e-12)


def test_shift_invariance():
    """logp(x + c) = logp(x) and lse(x + c) = lse(x) + c."""
    c = synth.tiny_fp32()
    x = c["logits"].numpy().astype(np.float64)
    t = c["targets"].numpy()
    logp0, lse0 = oracle.logp_fwd(x, t)
    for shift in (7.25, -30.0, 1000.0):
        logp1, lse1 = oracle.logp_fwd(x + shift, t)
        a = t != -100
        np.testing.assert_allclose(logp1[a], logp0[a], atol=1e-10, rtol=0)
        np.testing.assert_allclose(lse1[a], lse0[a] + shift, rtol=1e-13)


@pytest.mark.parametrize("v", [8, 300, 4096])
def test_normalisation(v):
    """sum over every target of exp(logp) is 1, and logp_j = x_j - lse."""
    g = np.random.default_rng(v)
    x = g.normal(0, 2.0, v)
    rows = np.tile(x, (v, 1))
    logp, lse = oracle.logp_fwd(rows, np.arange(v))
    assert abs(math.fsum(np.exp(logp)) - 1.0) <= 1e-13
    assert np.all(lse == lse[0])
    np.testing.assert_allclose(logp, x - lse[0], rtol=0, atol=1e-13)


def test_spike_bound():
    """Target on a one-hot spike: logp is within the two bounds set by the
    gap from the spike to the next-largest logit."""
    v = 151936
    g = np.random.default_rng(5)
    x = g.normal(0, 3.0, v)
    x[1234] = x.max() + 20.0
    gap = x[1234] - np.partition(x, -2)[-2]
    logp, _ = oracle.logp_fwd(x[None, :], [1234])
    # log(1 + e^-gap) <= -logp = log(1 + sum_{j != t} e^(x_j - x_t)) <= (V-1) e^-gap
    assert logp[0] <= 0.0
    assert abs(logp[0]) <= (v - 1) * math.exp(-gap) * (1 + 1e-9)
    assert abs(logp[0]) >= math.log1p(math.exp(-gap)) * (1 - 1e-9)


def test_ignore_and_invalid_targets():
    x = np.random.default_rng(0).normal(size=(4, 16))
    logp, lse = oracle.logp_fwd(x, [3, -100, 0, 15])
    assert logp[1] == 0.0 and lse[1] == 0.0
    assert logp[0] != 0.0
    with pytest.raises(oracle.InvalidTargetError):
        oracle.logp_fwd(x, [3, 16, 0, 0])
    with pytest.raises(oracle.InvalidTargetError):
        oracle.logp_fwd(x, [3, -1, 0, 0])
    # target -1 is an ignored row only when ignore_index is -1
    logp, _ = oracle.logp_fwd(x, [3, -1, 0, 0], ignore_index=-1)
    assert logp[1] == 0.0
    with pytest.raises(oracle.InvalidTargetError):
        oracle.logp_fwd(x, [3, -100, 0, 0], ignore_index=-1)
    d = oracle.logp_bwd(x, [3, -100, 0, 15], np.ones(4))
    assert np.all(d[1] == 0.0)


def test_sign_bound():
    c = synth.tiny_fp32()
    logp, _ = oracle.logp_fwd(c["logits"].numpy(), c["targets"].numpy())
    assert np.all(logp <= 0.0)


def test_leading_shape_flatten():
    """[B, T, V] logits are the same rows as the flattened [B*T, V]."""
    g = np.random.default_rng(1)
    x = g.normal(size=(2, 4, 300))
    t = g.integers(0, 300, size=(2, 4))
    t[0, 0] = -100
    logp3, _ = oracle.logp_fwd(x, t)
    logp2, _ = oracle.logp_fwd(x.reshape(8, 300), t.reshape(8))
    assert np.array_equal(logp3, logp2)
    assert logp3[0] == 0.0


# ----- tiled construction: merge identity and bookkeeping -----------------

def test_shard_tile_ranges_qwen3():
    v, w = 151936, 4096
    assert oracle.num_tiles(v, w) == 38
    assert oracle.shard_tile_ranges(v, w, 1) == [(0, 38)]
    assert oracle.shard_tile_ranges(v, w, 2) == [(0, 19), (19, 38)]
    assert oracle.shard_tile_ranges(v, w, 4) == [(0, 10), (10, 19), (19, 28), (28, 38)]
    with pytest.raises(ValueError):
        oracle.shard_tile_ranges(v, w, 3)


@pytest.mark.parametrize("v,w,s", [(151936, 4096, 4), (4096, 512, 2), (8, 512, 8),
                                   (300, 7, 3), (1000, 64, 5), (64, 1, 64)])
def test_shard_ranges_partition(v, w, s):
    """Every tile has exactly one owner, owners are ascending and contiguous,
    and each tile's first column lies in its owner's nominal range."""
    ranges = oracle.shard_tile_ranges(v, w, s)
    t = oracle.num_tiles(v, w)
    assert ranges[0][0] == 0 and ranges[-1][1] == t
    for (a, b), (c, _) in zip(ranges, ranges[1:]):
        assert b == c and a <= b
    per = v // s
    for i, (lo, hi) in enumerate(ranges):
        for k in range(lo, hi):
            assert i * per <= k * w < (i + 1) * per


def test_tile_partials_brute():
    """(m_k, s_k) against Python loops, with the -inf padded last tile."""
    g = np.random.default_rng(2)
    x = g.normal(0, 3, 37)
    m, s = oracle.tile_partials(x, 8)
    assert m.shape == (5,)
    for k in range(5):
        cols = [float(a) for a in x[8 * k: 8 * k + 8]]
        assert m[k] == max(cols)
        assert abs(s[k] - math.fsum(math.exp(a - max(cols)) for a in cols)) <= 1e-14
    assert s[4] <= 5.0 + 1e-12  # 5 real columns in the padded tile


@pytest.mark.parametrize("w", [1, 7, 512, 4096])
@pytest.mark.parametrize("s", [1, 2, 4])
def test_tiled_merge_identity(w, s):
    """fp64 tile partials merged in the fixed order equal the untiled LSE
    (associativity of the (max, sumexp) merge in real arithmetic)."""
    g = np.random.default_rng(w * 10 + s)
    for v in (8, 300, 4096, 151936):
        if v % s or (v > 4096 and w < 512):
            continue
        x = g.normal(0, 3.0, (3, v))
        t = g.integers(0, v, 3)
        logp0, lse0 = oracle.logp_fwd(x, t)
        logp1, lse1 = oracle.tiled_logp_fwd(x, t, -100, w, s)
        np.testing.assert_allclose(lse1, lse0, rtol=1e-12)
        np.testing.assert_allclose(logp1, logp0, rtol=1e-12, atol=1e-12)


def test_tiled_fp32_contract_error():
    """The float32 tiled construction stays well inside 1e-5 abs + 1e-5 rel
    of the exact value on the Qwen3-vocab distribution (the tolerance the
    GPU path is held to)."""
    c = synth.qwen3_fwd(n=16)
    x = c["logits"].float().numpy()
    t = c["targets"].numpy()
    logp0, lse0 = oracle.logp_fwd(x, t)
    logp1, lse1 = oracle.tiled_logp_fwd(x, t, -100, 4096, 1, dtype=np.float32)
    err = np.abs(logp1 - logp0)
    assert np.all(err <= 1e-5 + 1e-5 * np.abs(logp0))
    assert np.all(np.abs(lse1 - lse0) <= 1e-5 + 1e-5 * np.abs(lse0))


# ----- backward ------------------------------------------------------------

def test_bwd_finite_difference():
    """Central differences of the float64 forward reproduce g*(onehot - p)."""
    g = np.random.default_rng(3)
    x = g.normal(0, 2.0, (4, 8))
    t = np.array([0, 3, 7, 5])
    gr = np.array([1.0, -0.5, 2.0, 0.25])
    d = oracle.logp_bwd(x, t, gr)
    h = 1e-6
    for r in range(4):
        for j in range(8):
            xp = x[r].copy(); xp[j] += h
            xm = x[r].copy(); xm[j] -= h
            fp, _ = oracle.logp_fwd(xp[None], [t[r]])
            fm, _ = oracle.logp_fwd(xm[None], [t[r]])
            fd = gr[r] * (fp[0] - fm[0]) / (2 * h)
            assert abs(fd - d[r, j]) <= 1e-8, (r, j, fd, d[r, j])


def test_bwd_library_autograd():
    """torch float64 autograd of log_softmax.gather, scaled by g."""
    c = synth.tiny_fp32()
    x = c["logits"].double().requires_grad_(True)
    t = c["targets"]
    gr = torch.linspace(-1.5, 2.0, x.shape[0], dtype=torch.float64)
    active = t != -100
    sel = torch.log_softmax(x, -1).gather(-1, t.clamp(min=0)[:, None])[:, 0]
    (torch.where(active, sel, torch.zeros_like(sel)) * gr).sum().backward()
    d = oracle.logp_bwd(c["logits"].numpy(), t.numpy(), gr.numpy())
    np.testing.assert_allclose(d, x.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_bwd_row_sum_zero():
    c = synth.tiny_fp32()
    gr = np.random.default_rng(4).normal(size=64)
    d = oracle.logp_bwd(c["logits"].numpy(), c["targets"].numpy(), gr)
    assert np.all(np.abs(d.sum(axis=1)) <= 1e-12)
    ign = c["targets"].numpy() == -100
    assert np.all(d[ign] == 0.0)


# ----- fused LM head ---------------------------------------------------------

def test_linear_identity_weight():
    """W = I: z = h exactly, so the fused result is logp_fwd(h)."""
    g = np.random.default_rng(6)
    h = g.normal(size=(16, 64)).astype(np.float32)
    t = g.integers(0, 64, 16)
    t[3] = -100
    a = oracle.linear_logp_fwd(h, np.eye(64, dtype=np.float32), t)
    b = oracle.logp_fwd(h, t)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_linear_zero_weight():
    """W = 0: every logit is 0, logp = -log V."""
    h = np.random.default_rng(7).normal(size=(5, 32))
    logp, lse = oracle.linear_logp_fwd(h, np.zeros((1000, 32)), [0, 1, 2, 999, 500])
    np.testing.assert_allclose(logp, -math.log(1000), rtol=1e-15)
    np.testing.assert_allclose(lse, math.log(1000), rtol=1e-15)


def test_linear_brute_force():
    """Pure-Python dot products and log-sum-exp on a tiny problem; a
    transposed weight (z = h W instead of h W^T) cannot pass this."""
    g = np.random.default_rng(8)
    n, hd, v = 4, 8, 16
    h = g.normal(size=(n, hd))
    w = g.normal(size=(v, hd))
    t = [0, 5, 15, 9]
    logp, lse = oracle.linear_logp_fwd(h, w, t)
    for r in range(n):
        z = [math.fsum(float(h[r, k]) * float(w[j, k]) for k in range(hd))
             for j in range(v)]
        assert abs(logp[r] - _brute(z, t[r])) <= 1e-13
    with pytest.raises(ValueError):
        oracle.linear_logp_fwd(h, w.T, t)


# ----- fused LM head backward --------------------------------------------------

def _objective(h, w, t, g):
    """sum_r g_r * logp_r written out with math.fsum (no numpy reductions)."""
    total = []
    for r in range(h.shape[0]):
        if t[r] == -100:
            continue
        z = [math.fsum(float(h[r, k]) * float(w[j, k]) for k in range(h.shape[1]))
             for j in range(w.shape[0])]
        m = max(z)
        lse = m + math.log(math.fsum(math.exp(a - m) for a in z))
        total.append(g[r] * (z[t[r]] - lse))
    return math.fsum(total)


def test_linear_bwd_finite_difference():
    """Central differences of sum g*logp in h and in W reproduce dh and dW
    (a transposed product, a dropped g or a wrong sign fails)."""
    rng = np.random.default_rng(21)
    n, hd, v = 3, 4, 5
    h = rng.normal(size=(n, hd))
    w = rng.normal(size=(v, hd))
    t = [2, -100, 4]
    g = np.array([0.7, 1.3, -1.1])
    dh, dw = oracle.linear_logp_bwd(h, w, t, g)
    eps = 1e-6
    for (arr, grad) in ((h, dh), (w, dw)):
        for idx in np.ndindex(arr.shape):
            a = arr.copy(); a[idx] += eps
            b = arr.copy(); b[idx] -= eps
            if arr is h:
                fp, fm = _objective(a, w, t, g), _objective(b, w, t, g)
            else:
                fp, fm = _objective(h, a, t, g), _objective(h, b, t, g)
            num = (fp - fm) / (2 * eps)
            assert abs(num - grad[idx]) <= 1e-7, (idx, num, grad[idx])
    assert np.all(dh[1] == 0.0)


def test_linear_bwd_library_autograd():
    """torch float64 autograd of log_softmax(h W^T).gather(t), weighted by g
    ("Batch-Invariant LogP", Reference Semantics), gives the same dh, dW."""
    rng = np.random.default_rng(22)
    n, hd, v = 12, 16, 40
    h = rng.normal(size=(n, hd))
    w = rng.normal(size=(v, hd)) * 0.5
    t = rng.integers(0, v, n)
    t[5] = -100
    g = rng.normal(size=n)
    dh, dw = oracle.linear_logp_bwd(h, w, t, g)
    th = torch.tensor(h, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    z = th @ tw.T
    lp = torch.log_softmax(z, dim=-1)
    tt = torch.tensor(t)
    mask = tt != -100
    sel = lp[mask].gather(1, tt[mask].unsqueeze(1)).squeeze(1)
    (sel * torch.tensor(g)[mask]).sum().backward()
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_linear_bwd_identity_and_equal_rows():
    """W = I: dz is logp_bwd of h itself, dh = dz and dW = dz^T h.  A weight
    whose rows are all equal gives dh = 0 (each gradient row sums to 0)."""
    rng = np.random.default_rng(23)
    h = rng.normal(size=(9, 32))
    t = rng.integers(0, 32, 9)
    t[0] = -100
    g = rng.normal(size=9)
    dh, dw = oracle.linear_logp_bwd(h, np.eye(32), t, g)
    dz = oracle.logp_bwd(h, t, g)
    np.testing.assert_allclose(dh, dz, rtol=0, atol=1e-15)
    np.testing.assert_allclose(dw, dz.T @ h, rtol=1e-14, atol=1e-14)
    w = np.tile(rng.normal(size=(1, 32)), (50, 1))
    t2 = rng.integers(0, 50, 9)
    dh2, _ = oracle.linear_logp_bwd(h, w, t2, g)
    assert np.all(np.abs(dh2) <= 1e-12)


def test_linear_bwd_ignored_rows_add_nothing():
    """Appending ignored rows changes neither dW nor the other rows' dh; the
    given lse is used (a shifted lse scales the softmax part)."""
    rng = np.random.default_rng(24)
    h = rng.normal(size=(6, 8))
    w = rng.normal(size=(20, 8))
    t = rng.integers(0, 20, 6)
    g = rng.normal(size=6)
    dh, dw = oracle.linear_logp_bwd(h, w, t, g)
    h2 = np.vstack([h, rng.normal(size=(3, 8))])
    t2 = np.concatenate([t, [-100, -100, -100]])
    g2 = np.concatenate([g, [5.0, 6.0, 7.0]])
    dh2, dw2 = oracle.linear_logp_bwd(h2, w, t2, g2)
    np.testing.assert_allclose(dh2[:6], dh, rtol=0, atol=1e-15)
    assert np.all(dh2[6:] == 0.0)
    np.testing.assert_allclose(dw2, dw, rtol=1e-14, atol=1e-15)
    _, lse = oracle.linear_logp_fwd(h, w, t)
    dh3, _ = oracle.linear_logp_bwd(h, w, t, g, lse=lse + math.log(2.0))
    z = h @ w.T
    p = np.exp(z - lse[:, None])
    want = dh - (-(g[:, None] * p * 0.5)) @ w
    np.testing.assert_allclose(dh3, want, rtol=1e-12, atol=1e-13)


def test_linear_bwd_weight_rows_matches_full():
    """The sampled-row dW equals the full dW rows (and its own lse path)."""
    rng = np.random.default_rng(25)
    h = rng.normal(size=(20, 16))
    w = rng.normal(size=(70, 16)) * 0.3
    t = rng.integers(0, 70, 20)
    t[[2, 7]] = -100
    t[3] = 11
    g = rng.normal(size=20)
    _, dw = oracle.linear_logp_bwd(h, w, t, g)
    rows = [0, 11, 69, 11, 35]
    got = oracle.linear_logp_bwd_weight_rows(h, w, t, g, rows)
    np.testing.assert_allclose(got, dw[rows], rtol=1e-12, atol=1e-14)
    _, lse = oracle.linear_logp_fwd(h, w, t)
    got2 = oracle.linear_logp_bwd_weight_rows(h, w, t, g, rows, lse=lse)
    np.testing.assert_array_equal(got, got2)


# ----- entropy and temperature -------------------------------------------------

def test_entropy_closed_forms():
    """Uniform row: H = log V.  Two-level row (k entries a, V-k entries b):
    H = -k q_a log q_a - (V-k) q_b log q_b with q = e^x / (k e^a + (V-k) e^b),
    written out with math.  Ignored rows: 0."""
    v = 1000
    x = np.zeros((2, v))
    x[1, :7] = 3.0
    x[1, 7:] = -1.5
    h = oracle.entropy(x, [3, -100])
    assert abs(h[0] - math.log(v)) <= 1e-12
    assert h[1] == 0.0
    h2 = oracle.entropy(x[1:], [0])[0]
    k, a, b = 7, 3.0, -1.5
    zsum = k * math.exp(a) + (v - k) * math.exp(b)
    qa, qb = math.exp(a) / zsum, math.exp(b) / zsum
    want = -k * qa * math.log(qa) - (v - k) * qb * math.log(qb)
    assert abs(h2 - want) <= 1e-12


def test_entropy_library_and_bounds():
    """torch.distributions.Categorical(logits).entropy() in float64; 0 <= H
    <= log V; shift invariance."""
    rng = np.random.default_rng(31)
    x = rng.normal(scale=3.0, size=(20, 500))
    t = rng.integers(0, 500, 20)
    h = oracle.entropy(x, t)
    ref = torch.distributions.Categorical(logits=torch.tensor(x)).entropy().numpy()
    np.testing.assert_allclose(h, ref, rtol=1e-12, atol=1e-12)
    assert (h >= 0).all() and (h <= math.log(500) + 1e-12).all()
    np.testing.assert_allclose(oracle.entropy(x + 7.25, t), h, rtol=1e-12, atol=1e-12)


def test_entropy_bwd_finite_difference():
    rng = np.random.default_rng(32)
    x = rng.normal(size=(3, 6))
    t = [1, -100, 5]
    gh = np.array([0.4, 2.0, -1.3])
    d = oracle.entropy_bwd(x, t, gh)
    eps = 1e-6
    for idx in np.ndindex(x.shape):
        a = x.copy(); a[idx] += eps
        b = x.copy(); b[idx] -= eps
        num = (np.dot(gh, oracle.entropy(a, t)) - np.dot(gh, oracle.entropy(b, t))) / (2 * eps)
        assert abs(num - d[idx]) <= 1e-8, (idx, num, d[idx])
    assert np.all(d[1] == 0.0)


def test_linear_temperature_and_entropy_autograd():
    """torch float64 autograd of g * logp + gH * entropy of softmax(h W^T / T)
    gives the oracle's dh, dW; the oracle's forward matches too."""
    rng = np.random.default_rng(33)
    n, hd, v, temp = 10, 12, 30, 0.7
    h = rng.normal(size=(n, hd))
    w = rng.normal(size=(v, hd)) * 0.5
    t = rng.integers(0, v, n)
    t[4] = -100
    g = rng.normal(size=n)
    gh = rng.normal(size=n)
    logp, lse = oracle.linear_logp_fwd(h, w, t, temperature=temp)
    ent = oracle.linear_entropy(h, w, t, temperature=temp)
    dh, dw = oracle.linear_logp_bwd(h, w, t, g, temperature=temp, grad_entropy=gh)
    th = torch.tensor(h, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    lp = torch.log_softmax((th @ tw.T) / temp, dim=-1)
    tt = torch.tensor(t)
    mask = tt != -100
    sel = lp[mask].gather(1, tt[mask].unsqueeze(1)).squeeze(1)
    ent_t = -(lp.exp() * lp).sum(-1)[mask]
    np.testing.assert_allclose(logp[mask.numpy()], sel.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ent[mask.numpy()], ent_t.detach().numpy(), rtol=1e-12, atol=1e-12)
    assert ent[4] == 0.0
    ((sel * torch.tensor(g)[mask]).sum() + (ent_t * torch.tensor(gh)[mask]).sum()).backward()
    np.testing.assert_allclose(dh, th.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-11, atol=1e-12)
    rows = [0, 7, 29]
    got = oracle.linear_logp_bwd_weight_rows(h, w, t, g, rows, temperature=temp,
                                             grad_entropy=gh)
    np.testing.assert_allclose(got, dw[rows], rtol=1e-11, atol=1e-13)


def test_linear_temperature_limits():
    """T -> large makes every row uniform (logp -> -log V, H -> log V); T = 1
    is the plain fused operator."""
    rng = np.random.default_rng(34)
    h = rng.normal(size=(4, 8))
    w = rng.normal(size=(50, 8))
    t = [0, 1, 2, 49]
    lp, _ = oracle.linear_logp_fwd(h, w, t, temperature=1e9)
    np.testing.assert_allclose(lp, -math.log(50), atol=1e-7)
    np.testing.assert_allclose(oracle.linear_entropy(h, w, t, temperature=1e9), math.log(50),
                               atol=1e-7)
    a = oracle.linear_logp_fwd(h, w, t)
    b = oracle.linear_logp_fwd(h, w, t, temperature=1.0)
    assert np.array_equal(a[0], b[0])


# ----- bf16-rounded-logits variant ---------------------------------------------

def _torch_bf16(x32):
    """float32 -> bfloat16 -> float64 by torch's conversion (round to nearest
    even), the library routine the oracle's rounding is pinned against."""
    return torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def test_round_bf16_matches_library():
    """round_bf16 equals torch's float32 -> bfloat16 conversion on float32
    values across the exponent range, on exact ties (even neighbour wins),
    on subnormals and at the overflow threshold."""
    rng = np.random.default_rng(40)
    mant = rng.uniform(1.0, 2.0, 20000)
    expo = rng.integers(-140, 128, 20000)
    x = (np.where(rng.random(20000) < 0.5, -1.0, 1.0) * np.ldexp(mant, expo)).astype(np.float32)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    y = bits.view(np.float32)
    y = y[np.isfinite(y)]
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -126 * (1 + 2 ** -8),
                     3 * 2 ** -135, 2 ** -134, 2 ** -133, 5 * 2 ** -135,
                     255.5 * 2.0 ** 120, 255.25 * 2.0 ** 120, 65504.0, 0.0, -0.0],
                    dtype=np.float32)
    for v in (x, y, ties):
        got = oracle.round_bf16(v.astype(np.float64))
        want = _torch_bf16(v)
        assert np.array_equal(got, want), v[got != want][:5]
    assert oracle.round_bf16(1 + 2 ** -8) == 1.0
    assert oracle.round_bf16(1 + 3 * 2 ** -8) == 1 + 2 ** -6
    assert oracle.round_bf16(255.5 * 2.0 ** 120) == math.inf
    assert np.isnan(oracle.round_bf16(np.nan))


def test_round_bf16_idempotent_on_bf16_values():
    """Values that are already bfloat16 come back unchanged."""
    rng = np.random.default_rng(41)
    v = _torch_bf16(rng.normal(size=5000).astype(np.float32) * 100)
    assert np.array_equal(oracle.round_bf16(v), v)


def test_linear_round_logits_exact_when_representable():
    """When every logit is already a bf16 value (small integers here), the
    rounded variant gives the plain fused operator's results exactly."""
    rng = np.random.default_rng(42)
    h = rng.integers(-2, 3, size=(7, 16)).astype(np.float64)
    w = rng.integers(-2, 3, size=(40, 16)).astype(np.float64)
    t = rng.integers(0, 40, 7)
    t[3] = -100
    g = rng.normal(size=7)
    a = oracle.linear_logp_fwd(h, w, t, temperature=1.3)
    b = oracle.linear_logp_fwd(h, w, t, temperature=1.3, round_logits=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    da = oracle.linear_logp_bwd(h, w, t, g)
    db = oracle.linear_logp_bwd(h, w, t, g, round_logits=True)
    assert np.array_equal(da[0], db[0]) and np.array_equal(da[1], db[1])


def test_linear_round_logits_closed_form():
    """h = [1, 1], W = [[1, 2^-9], [0, 0], [-1, 2^-7 + 2^-9]]: z = [1 + 2^-9,
    0, -1 + 5 * 2^-9] rounds to [1, 0, -1 + 2^-7].  Above 1 the spacing is
    2^-7, so 1 + 2^-9 goes down to 1; below 1 it is 2^-8, and
    -1 + 5 * 2^-9 = -253.5 / 256 is a tie between -253 / 256 and -254 / 256,
    which goes to the even -254 / 256.  logp, lse, entropy and the gradients
    then follow from the rounded row in closed form; the plain operator uses
    the unrounded row."""
    h = np.array([[1.0, 1.0]])
    w = np.array([[1.0, 2.0 ** -9], [0.0, 0.0], [-1.0, 2.0 ** -7 + 2.0 ** -9]])
    zr = np.array([1.0, 0.0, -1.0 + 2.0 ** -7])
    z = np.array([1.0 + 2.0 ** -9, 0.0, -1.0 + 5 * 2.0 ** -9])
    assert np.array_equal(oracle.round_bf16(z), zr)
    for t in range(3):
        for rnd, row in ((True, zr), (False, z)):
            lse = math.log(sum(math.exp(c) for c in row))
            lp, ls = oracle.linear_logp_fwd(h, w, [t], round_logits=rnd)
            assert abs(ls[0] - lse) < 1e-15 and abs(lp[0] - (row[t] - lse)) < 1e-15
            p = np.exp(row - lse)
            ent = -(p * (row - lse)).sum()
            assert abs(oracle.linear_entropy(h, w, [t], round_logits=rnd)[0] - ent) < 1e-15
            g = 0.75
            dz = g * ((np.arange(3) == t) - p)
            dh, dw = oracle.linear_logp_bwd(h, w, [t], [g], round_logits=rnd)
            np.testing.assert_allclose(dh[0], dz @ w, rtol=0, atol=1e-15)
            np.testing.assert_allclose(dw, np.outer(dz, h[0]), rtol=0, atol=1e-15)
            got = oracle.linear_logp_bwd_weight_rows(h, w, [t], [g], [2, 0], round_logits=rnd)
            np.testing.assert_allclose(got, np.outer(dz, h[0])[[2, 0]], rtol=0, atol=1e-15)
