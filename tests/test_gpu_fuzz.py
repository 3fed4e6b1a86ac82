"""Randomised GPU parity and invariance (hypothesis, fixed derivation so runs
repeat): random small shapes, dtypes, tile widths, shard counts, row
strides, target index types, ignored and out-of-range-free targets, logit
scales, entropy and temperature, each checked against the float64 oracle
with the bounds of the targeted tests, plus bitwise invariance of a row
computed alone and of sharded against unsharded forwards.

ITL_FUZZ_EXAMPLES=N (N > 0) replaces the fixed derivation by N fresh random
examples per test, a deeper search for a one-off run."""

import os

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, example, given, settings
from hypothesis import strategies as st

import invariant_token_log_amd as itl
import oracle
import synth
from gpu_helpers import assert_grad_parity, assert_logp_parity, bits, dev, to_np
from test_gpu_entropy import _ent_ok, _grad_ent_ok

pytestmark = pytest.mark.gpu

_DEEP = int(os.environ.get("ITL_FUZZ_EXAMPLES", "0"))


def _settings(n):
    """n derandomized examples, or ITL_FUZZ_EXAMPLES fresh random ones."""
    return settings(max_examples=_DEEP if _DEEP > 0 else n, deadline=None,
                    derandomize=_DEEP <= 0, database=None,
                    suppress_health_check=list(HealthCheck))


SETTINGS = _settings(40)


@st.composite
def stream_cases(draw):
    dtype = draw(st.sampled_from([torch.float32, torch.bfloat16, torch.float16]))
    unit = 256 if dtype == torch.float32 else 512  # widths: unit x 1, 2, 4, 8, 16
    w = draw(st.sampled_from([unit * k for k in (1, 2, 4, 8, 16)]))
    v = draw(st.integers(1, 6000))
    n = draw(st.integers(1, 48))
    shards = draw(st.sampled_from([s for s in (1, 2, 3, 4) if v % s == 0]))
    pad = draw(st.sampled_from([0, 0, 8, 13]))
    scale = draw(st.sampled_from([0.1, 3.0, 20.0]))
    n_ign = draw(st.integers(0, n))
    tdt = draw(st.sampled_from([torch.int64, torch.int32]))
    ent = draw(st.booleans())
    seed = draw(st.integers(0, 2 ** 30))
    return dict(dtype=dtype, w=w, v=v, n=n, shards=shards, pad=pad, scale=scale, n_ign=n_ign,
                tdt=tdt, ent=ent, seed=seed)


@SETTINGS
@given(stream_cases())
# bf16 dlogits that fall among the bf16 subnormals (|g| = 0.002, large logits)
@example(c=dict(dtype=torch.bfloat16, w=512, v=125, n=6, shards=1, pad=0, scale=20.0, n_ign=0,
                tdt=torch.int64, ent=False, seed=2160))
def test_fuzz_streaming(c):
    n, v, dtype = c["n"], c["v"], c["dtype"]
    base = synth.normal_matrix(n, v + c["pad"], c["scale"], dtype, seed=c["seed"]).to(dev())
    x = base[:, :v]  # row stride v + pad
    ign = torch.randperm(n, generator=torch.Generator().manual_seed(c["seed"]))[:c["n_ign"]]
    t = synth.uniform_targets(n, v, seed=c["seed"] + 1, ignore_rows=ign).to(dev()).to(c["tdt"])
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=c["seed"] + 2)[0].to(dev())
    what = str({k: (str(val) if k in ("dtype", "tdt") else val) for k, val in c.items()})
    out = itl.logp_fwd(x, t, -100, c["w"], num_shards=c["shards"], return_entropy=c["ent"])
    x64 = to_np(x)
    tn = t.cpu().numpy().astype(np.int64)
    ref_logp, ref_lse = oracle.logp_fwd(x64, tn)
    assert_logp_parity(out[0], out[1], ref_logp, ref_lse, t, what=what)
    if c["ent"]:
        _ent_ok(out[2], x64, tn, what)
    # sharded and unsharded forwards agree bit for bit; a row alone too
    one = itl.logp_fwd(x, t, -100, c["w"], return_entropy=c["ent"])
    for a, b in zip(out, one):
        assert torch.equal(bits(a), bits(b)), what
    r = n // 2
    alone = itl.logp_fwd(x[r:r + 1], t[r:r + 1], -100, c["w"], return_entropy=c["ent"])
    for a, b in zip(one, alone):
        assert torch.equal(bits(a)[r:r + 1], bits(b)), what
    # backward against the oracle's gradient at the oracle's lse
    if c["ent"]:
        gh = synth.normal_matrix(1, n, 1.0, torch.float32, seed=c["seed"] + 3)[0].to(dev())
        d = itl.logp_bwd(x, t, one[1], g, -100, c["w"], entropy=one[2], grad_entropy=gh)
    else:
        d = itl.logp_bwd(x, t, one[1], g, -100, c["w"])
        d64 = oracle.logp_bwd(x64, tn, to_np(g), lse=ref_lse)
    if c["ent"]:
        _grad_ent_ok(d, x64, tn, to_np(g), to_np(gh), what)
    else:
        assert_grad_parity(d, d64, x64, ref_lse, to_np(g), t, what=what)
    dalone = itl.logp_bwd(x[r:r + 1], t[r:r + 1], one[1][r:r + 1], g[r:r + 1], -100, c["w"],
                          entropy=one[2][r:r + 1] if c["ent"] else None,
                          grad_entropy=gh[r:r + 1] if c["ent"] else None)
    assert torch.equal(d[r:r + 1].contiguous().view(torch.int16 if dtype != torch.float32
                                                    else torch.int32),
                       dalone.view(torch.int16 if dtype != torch.float32 else torch.int32)), what


@st.composite
def linear_cases(draw):
    return dict(n=draw(st.integers(1, 300)),
                h=draw(st.sampled_from([64, 128, 256, 320, 448, 512])),
                v=draw(st.integers(1, 3000)), temp=draw(st.sampled_from([1.0, 0.7, 2.0])),
                ent=draw(st.booleans()), n_ign=draw(st.integers(0, 5)),
                chunk=draw(st.sampled_from([256, 512, 768, 1024])),
                seed=draw(st.integers(0, 2 ** 30)))


@SETTINGS
@given(linear_cases())
def test_fuzz_linear(c):
    n, h, v = c["n"], c["h"], c["v"]
    hid = synth.normal_matrix(n, h, 1.0, torch.bfloat16, seed=c["seed"]).to(dev())
    w = synth.normal_matrix(v, h, 0.05, torch.bfloat16, seed=c["seed"] + 1).to(dev())
    ign = torch.randperm(n, generator=torch.Generator().manual_seed(c["seed"]))[:min(c["n_ign"], n)]
    t = synth.uniform_targets(n, v, seed=c["seed"] + 2, ignore_rows=ign).to(dev())
    what = str(c)
    out = itl.linear_logp_fwd(hid, w, t, temperature=c["temp"], return_entropy=c["ent"])
    hn, wn, tn = to_np(hid), to_np(w), t.cpu().numpy()
    ref = oracle.linear_logp_fwd(hn, wn, tn, temperature=c["temp"])
    assert_logp_parity(out[0], out[1], *ref, t, what=what)
    if c["ent"]:
        _ent_ok(out[2], (hn @ wn.T) / c["temp"], tn, what)
    r = n // 2
    alone = itl.linear_logp_fwd(hid[r:r + 1].contiguous(), w, t[r:r + 1].contiguous(),
                                temperature=c["temp"], return_entropy=c["ent"])
    for a, b in zip(out, alone):
        assert torch.equal(bits(a)[r:r + 1], bits(b)), what
    # the prepared weight gives the same bits (every tile shape reads it)
    prep = itl.linear_logp_fwd(hid, w, t, temperature=c["temp"], return_entropy=c["ent"],
                               prepared_weight=itl.prepare_weight(w))
    for a, b in zip(out, prep):
        assert torch.equal(bits(a), bits(b)), what


@_settings(20)
@given(linear_cases())
def test_fuzz_linear_bwd(c):
    """dh and dW against the float64 oracle by the fused backward's bound, and
    the saved-logits, prepared-weight and chunked paths with the same bits."""
    from test_gpu_linear_bwd import _bounds

    n, h, v = c["n"], c["h"], c["v"]
    hid = synth.normal_matrix(n, h, 1.0, torch.bfloat16, seed=c["seed"]).to(dev())
    w = synth.normal_matrix(v, h, 0.05, torch.bfloat16, seed=c["seed"] + 1).to(dev())
    ign = torch.randperm(n, generator=torch.Generator().manual_seed(c["seed"]))[:min(c["n_ign"], n)]
    t = synth.uniform_targets(n, v, seed=c["seed"] + 2, ignore_rows=ign).to(dev())
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=c["seed"] + 3)[0].to(dev())
    what = str(c)
    zbuf = torch.empty(n, (v + 3) // 4 * 4, dtype=torch.float32, device=dev())[:, :v]
    _, lse, z = itl.linear_logp_fwd(hid, w, t, return_logits=True, logits_dtype=torch.float32,
                                    logits_out=zbuf)
    dh, dw = itl.linear_logp_bwd(hid, w, t, lse, g)
    dh2, dw2 = itl.linear_logp_bwd(hid, w, t, lse, g, saved_logits=z)
    assert torch.equal(dh, dh2) and torch.equal(dw, dw2), what
    dh3, dw3 = itl.linear_logp_bwd(hid, w, t, lse, g, prepared_weight=itl.prepare_weight(w))
    assert torch.equal(dh, dh3) and torch.equal(dw, dw3), what
    # several vocabulary chunks (a partial last chunk, whose weight lines past
    # v read zeros): the same bits
    dh4, dw4 = itl.linear_logp_bwd(hid, w, t, lse, g, vocab_chunk=c["chunk"])
    assert torch.equal(dh, dh4) and torch.equal(dw, dw4), what
    # bf16 outputs (dh carried in fp32 between chunks, rounded once)
    b1 = itl.linear_logp_bwd(hid, w, t, lse, g, out_dtype=torch.bfloat16)
    b2 = itl.linear_logp_bwd(hid, w, t, lse, g, out_dtype=torch.bfloat16, vocab_chunk=c["chunk"])
    for x32, x1, x2 in zip((dh, dw), b1, b2):
        assert torch.equal(bits(x1), bits(x2)), what
        assert torch.equal(x1, x32.to(torch.bfloat16)), what
    hn, wn, tn, gn = to_np(hid), to_np(w), t.cpu().numpy(), to_np(g)
    dh64, dw64 = oracle.linear_logp_bwd(hn, wn, tn, gn)
    _, lse64 = oracle.linear_logp_fwd(hn, wn, tn)
    bh, bw = _bounds(hn, wn, tn, gn, lse64)
    assert (np.abs(to_np(dh) - dh64) <= bh).all(), what
    assert (np.abs(to_np(dw) - dw64) <= bw).all(), what


@st.composite
def linear_grid_cases(draw):
    return dict(n=draw(st.integers(129, 1100)), h=draw(st.sampled_from([64, 128])),
                v=draw(st.integers(20000, 70000)), ent=draw(st.booleans()),
                n_ign=draw(st.integers(0, 40)), seed=draw(st.integers(0, 2 ** 30)))


@_settings(12)
@given(linear_grid_cases())
def test_fuzz_linear_grids(c):
    """The 256-row kernel on grids of several hundred to about 1400 tiles:
    XCD ranges of unequal length, tiles handed out at run time, and (when the
    final round would be at most a quarter full) the last vocabulary blocks
    on the 64-row tile.  Sampled rows against the oracle; every row's bits
    equal to the row alone, and to the prepared-weight call."""
    n, h, v = c["n"], c["h"], c["v"]
    hid = synth.normal_matrix(n, h, 1.0, torch.bfloat16, seed=c["seed"]).to(dev())
    w = synth.normal_matrix(v, h, 0.05, torch.bfloat16, seed=c["seed"] + 1).to(dev())
    ign = torch.randperm(n, generator=torch.Generator().manual_seed(c["seed"]))[:c["n_ign"]]
    t = synth.uniform_targets(n, v, seed=c["seed"] + 2, ignore_rows=ign).to(dev())
    what = str(c)
    out = itl.linear_logp_fwd(hid, w, t, return_entropy=c["ent"])
    rows = torch.tensor(sorted({0, n // 3, n // 2, n - 1}), device=dev())
    ref = oracle.linear_logp_fwd(to_np(hid[rows]), to_np(w), t[rows].cpu().numpy())
    assert_logp_parity(out[0][rows], out[1][rows], *ref, t[rows], what=what)
    for r in (0, n - 1):
        alone = itl.linear_logp_fwd(hid[r:r + 1].contiguous(), w, t[r:r + 1].contiguous(),
                                    return_entropy=c["ent"])
        for a, b in zip(out, alone):
            assert torch.equal(bits(a)[r:r + 1], bits(b)), what
    prep = itl.linear_logp_fwd(hid, w, t, return_entropy=c["ent"],
                               prepared_weight=itl.prepare_weight(w))
    for a, b in zip(out, prep):
        assert torch.equal(bits(a), bits(b)), what
