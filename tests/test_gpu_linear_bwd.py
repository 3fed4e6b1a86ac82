"""GPU parity and invariance of the fused LM-head backward (linear_logp_bwd)
against the float64 oracle ("[RFC][ROCm] End-to-end optimization of bitwise
VIME R/R beyond native P/P", Workstream 3: the backward recomputes the fixed
logit tiles from the saved LSE; "Batch-Invariant LogP", Batch-Invariance).

Tolerance (derived, elementwise).  The kernel rounds dz = g (onehot - p) to
bf16 once (at most 2^-9 relative), its z and lse differ from float64 by far
less than EPS_Z, and the fp32 K walks add at most K/32 roundings.  So
    |dh - dh64| <= 2^-8 sum_j |dz64[r, j]| |W[j, k]| + |g| p_t EPS_Z |W[t, k]| + 1e-6
and the same with (tokens, h) in place of (vocabulary, W) for dW; the second
term covers the target column, where 1 - p may cancel."""

import numpy as np
import pytest
import torch

import invariant_token_log_amd as itl
import oracle
import synth
from gpu_helpers import assert_logp_parity, bits, dev

pytestmark = pytest.mark.gpu

REL = 2.0 ** -8
EPS_Z = 1e-3
ABS = 1e-6


def _f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _dz64(h, w, t, g, lse64):
    z = h @ w.T
    p = np.exp(z - lse64[:, None])
    active = t != -100
    onehot = np.zeros_like(p)
    onehot[np.flatnonzero(active), t[active]] = 1.0
    dz = g[:, None] * (onehot - p)
    dz[~active] = 0.0
    return dz, p


def _bounds(h, w, t, g, lse64, need_dweight=True):
    """Elementwise bounds for dh [N, H] and dW [V, H] (comparison rule only)."""
    dz, p = _dz64(h, w, t, g, lse64)
    active = t != -100
    pt = np.zeros(len(t))
    pt[active] = p[np.flatnonzero(active), t[active]]
    tgt = np.zeros_like(dz)
    tgt[np.flatnonzero(active), t[active]] = np.abs(g[active]) * pt[active] * EPS_Z
    bh = REL * (np.abs(dz) @ np.abs(w)) + tgt @ np.abs(w) + ABS
    if not need_dweight:
        return bh, None
    bw = REL * (np.abs(dz).T @ np.abs(h)) + tgt.T @ np.abs(h) + ABS
    return bh, bw


def _case(n, hd, v, seed, ignore_frac=0.05):
    c = synth.qwen3_linear(seed=seed, n=n, h=hd, v=v, device=dev(), ignore_frac=ignore_frac)
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=seed + 50)[0].to(dev())
    return c["hidden"], c["weight"], c["targets"], g


@pytest.mark.parametrize("n,hd,v", [(64, 256, 4096), (200, 128, 1000), (1, 64, 256),
                                    (129, 512, 529), (300, 512, 4096), (257, 64, 300),
                                    # H past a whole 256-row tile: the weight rows read
                                    # K-outer for dh end inside the last tile
                                    (100, 320, 700), (70, 576, 1300)])
def test_parity_small(n, hd, v):
    h, w, t, g = _case(n, hd, v, seed=n * 7 + v)
    _, lse = itl.linear_logp_fwd(h, w, t)
    dh, dw = itl.linear_logp_bwd(h, w, t, lse, g)
    hn, wn, tn, gn = _f64(h), _f64(w), t.cpu().numpy(), _f64(g)
    dh64, dw64 = oracle.linear_logp_bwd(hn, wn, tn, gn)
    _, lse64 = oracle.linear_logp_fwd(hn, wn, tn)
    bh, bw = _bounds(hn, wn, tn, gn, lse64)
    eh = np.abs(_f64(dh) - dh64)
    ew = np.abs(_f64(dw) - dw64)
    assert (eh <= bh).all(), (np.argwhere(eh > bh)[:5], eh.max())
    assert (ew <= bw).all(), (np.argwhere(ew > bw)[:5], ew.max())
    ign = torch.from_numpy(tn == -100).to(dev())
    assert (bits(dh[ign]) == 0).all()


def test_bf16_output_is_rne_of_fp32():
    h, w, t, g = _case(130, 256, 1000, seed=3)
    _, lse = itl.linear_logp_fwd(h, w, t)
    dh, dw = itl.linear_logp_bwd(h, w, t, lse, g)
    bh, bw = itl.linear_logp_bwd(h, w, t, lse, g, out_dtype=torch.bfloat16)
    assert torch.equal(bh.view(torch.int16), dh.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(bw.view(torch.int16), dw.to(torch.bfloat16).view(torch.int16))


def test_dh_rows_batch_invariant():
    """dh[r] depends only on row r: alone, permuted, among other rows."""
    h, w, t, g = _case(300, 256, 2000, seed=5)
    _, lse = itl.linear_logp_fwd(h, w, t)
    dh, _ = itl.linear_logp_bwd(h, w, t, lse, g, need_dweight=False)
    b0 = bits(dh)
    for r in [0, 5, 255, 256, 299]:
        d1, _ = itl.linear_logp_bwd(h[r:r + 1].contiguous(), w, t[r:r + 1].contiguous(),
                                    lse[r:r + 1].contiguous(), g[r:r + 1].contiguous(),
                                    need_dweight=False)
        assert torch.equal(bits(d1), b0[r:r + 1]), r
    perm = torch.randperm(300, generator=torch.Generator().manual_seed(2)).to(dev())
    dp, _ = itl.linear_logp_bwd(h[perm].contiguous(), w, t[perm].contiguous(),
                                lse[perm].contiguous(), g[perm].contiguous(), need_dweight=False)
    assert torch.equal(bits(dp), b0[perm.cpu()])


def test_dw_deterministic_and_ignored_rows_neutral():
    """dW repeats bit for bit; appending ignored rows (zero dz rows at the end
    of the token walk) leaves it unchanged; each product alone equals the pair."""
    h, w, t, g = _case(200, 128, 1500, seed=9)
    _, lse = itl.linear_logp_fwd(h, w, t)
    dh, dw = itl.linear_logp_bwd(h, w, t, lse, g)
    dh2, dw2 = itl.linear_logp_bwd(h, w, t, lse, g)
    assert torch.equal(bits(dw), bits(dw2)) and torch.equal(bits(dh), bits(dh2))
    _, dw_only = itl.linear_logp_bwd(h, w, t, lse, g, need_dhidden=False)
    dh_only, _ = itl.linear_logp_bwd(h, w, t, lse, g, need_dweight=False)
    assert torch.equal(bits(dw_only), bits(dw)) and torch.equal(bits(dh_only), bits(dh))
    extra = synth.normal_matrix(100, 128, 1.0, torch.bfloat16, seed=10).to(dev())
    h3 = torch.cat([h, extra])
    t3 = torch.cat([t, torch.full((100,), -100, device=dev())])
    g3 = torch.cat([g, torch.ones(100, device=dev())])
    l3 = torch.cat([lse, torch.zeros(100, device=dev())])
    dh3, dw3 = itl.linear_logp_bwd(h3, w, t3, l3, g3)
    assert torch.equal(bits(dw3), bits(dw))
    assert torch.equal(bits(dh3[:200]), bits(dh)) and (bits(dh3[200:]) == 0).all()


def test_zero_rows_give_zero_dweight():
    w = synth.normal_matrix(300, 64, 0.02, torch.bfloat16, seed=1).to(dev())
    h = torch.empty(0, 64, dtype=torch.bfloat16, device=dev())
    t = torch.empty(0, dtype=torch.int64, device=dev())
    e = torch.empty(0, dtype=torch.float32, device=dev())
    dwo = torch.full((300, 64), 7.0, device=dev())
    _, dw = itl.linear_logp_bwd(h, w, t, e, e, need_dhidden=False, dweight_out=dwo)
    assert (bits(dw) == 0).all()


def test_autograd_matches_direct_call():
    """linear_logp(...).sum().backward() gives the bf16 gradients of a direct
    call with g = 1."""
    h, w, t, _ = _case(96, 128, 700, seed=11)
    hh = h.clone().requires_grad_(True)
    ww = w.clone().requires_grad_(True)
    out = itl.linear_logp(hh, ww, t)
    out.sum().backward()
    _, lse = itl.linear_logp_fwd(h, w, t)
    dh, dw = itl.linear_logp_bwd(h, w, t, lse, torch.ones(96, device=dev()),
                                 out_dtype=torch.bfloat16)
    assert hh.grad.dtype == torch.bfloat16 and ww.grad.dtype == torch.bfloat16
    assert torch.equal(hh.grad.view(torch.int16), dh.view(torch.int16))
    assert torch.equal(ww.grad.view(torch.int16), dw.view(torch.int16))


def test_full_size_sampled():
    """Qwen3-8B LM head (N = 4096, H = 4096, V = 151936) at the benchmarked
    launch: sampled rows of dh and sampled vocabulary rows of dW against the
    float64 oracle (the full-row LSE comes from the oracle's own forward)."""
    h, w, t, g = _case(4096, synth.QWEN3_HIDDEN, synth.QWEN3_VOCAB, seed=1005, ignore_frac=0.05)
    _, lse = itl.linear_logp_fwd(h, w, t)
    dh, dw = itl.linear_logp_bwd(h, w, t, lse, g)
    # the prepared weight gives the same bits at full size
    dh2, dw2 = itl.linear_logp_bwd(h, w, t, lse, g, prepared_weight=itl.prepare_weight(w))
    assert torch.equal(bits(dh2), bits(dh)) and torch.equal(bits(dw2), bits(dw))
    del dh2, dw2
    torch.cuda.synchronize()
    hn, wn, tn, gn = _f64(h), _f64(w), t.cpu().numpy(), _f64(g)
    rows = np.array(list(range(0, 4096, 293)) + [4095])
    dh64, _ = oracle.linear_logp_bwd(hn[rows], wn, tn[rows], gn[rows], need_dweight=False)
    _, lse_rows = oracle.linear_logp_fwd(hn[rows], wn, tn[rows])
    bh, _ = _bounds(hn[rows], wn, tn[rows], gn[rows], lse_rows, need_dweight=False)
    eh = np.abs(_f64(dh)[rows] - dh64)
    assert (eh <= bh).all(), (np.argwhere(eh > bh)[:5], eh.max())
    _, lse64 = oracle.linear_logp_fwd(hn, wn, tn)
    active_targets = np.unique(tn[tn != -100])
    vr = np.unique(np.concatenate([[0, 1, 4095, 151935], active_targets[::400]]))
    dw64 = oracle.linear_logp_bwd_weight_rows(hn, wn, tn, gn, vr, lse=lse64)
    # bound of the sampled rows (comparison rule only): dz of columns vr
    act = tn != -100
    pp = np.exp(hn @ wn[vr].T - lse64[:, None])
    hit = (tn[:, None] == vr[None, :]) & act[:, None]
    dzz = gn[:, None] * (hit.astype(np.float64) - pp)
    dzz[~act] = 0.0
    tgt = np.where(hit, np.abs(gn)[:, None] * pp * EPS_Z, 0.0)
    bw = REL * (np.abs(dzz).T @ np.abs(hn)) + tgt.T @ np.abs(hn) + ABS
    ew = np.abs(_f64(dw)[vr] - dw64)
    assert (ew <= bw).all(), (np.argwhere(ew > bw)[:5], ew.max())
    assert torch.isfinite(dh).all() and torch.isfinite(dw).all()


def test_large_n_sampled():
    """N = 20000 rows on the Qwen3-8B head (79 row blocks: a long tile queue in
    the forward, 10112 dz tiles per chunk and a 20224-token K walk for dW):
    sampled forward rows and dh rows against the float64 oracle, and sampled
    vocabulary rows of dW against the oracle given the forward's LSE (the
    full-row LSE of 20000 rows is too much float64 work here; its fp32 error
    is far inside the bf16 bound of dz)."""
    n = 20000
    h, w, t, g = _case(n, synth.QWEN3_HIDDEN, synth.QWEN3_VOCAB, seed=2024, ignore_frac=0.05)
    logp, lse = itl.linear_logp_fwd(h, w, t)
    dh, dw = itl.linear_logp_bwd(h, w, t, lse, g)
    torch.cuda.synchronize()
    assert torch.isfinite(dh).all() and torch.isfinite(dw).all()
    hn, wn, tn, gn = _f64(h), _f64(w), t.cpu().numpy(), _f64(g)
    rows = np.array([0, 1, 4999, 10007, 15000, 19998, n - 1])
    lp64, lse_rows = oracle.linear_logp_fwd(hn[rows], wn, tn[rows])
    assert_logp_parity(logp[rows], lse[rows], lp64, lse_rows, t[rows], what="linear large n")
    dh64, _ = oracle.linear_logp_bwd(hn[rows], wn, tn[rows], gn[rows], need_dweight=False)
    bh, _ = _bounds(hn[rows], wn, tn[rows], gn[rows], lse_rows, need_dweight=False)
    eh = np.abs(_f64(dh)[rows] - dh64)
    assert (eh <= bh).all(), (np.argwhere(eh > bh)[:5], eh.max())
    lse_gpu = _f64(lse)
    active_targets = np.unique(tn[tn != -100])
    vr = np.unique(np.concatenate([[0, 151935], active_targets[::997]]))
    dw64 = oracle.linear_logp_bwd_weight_rows(hn, wn, tn, gn, vr, lse=lse_gpu)
    act = tn != -100
    pp = np.exp(hn @ wn[vr].T - lse_gpu[:, None])
    hit = (tn[:, None] == vr[None, :]) & act[:, None]
    dzz = gn[:, None] * (hit.astype(np.float64) - pp)
    dzz[~act] = 0.0
    tgt = np.where(hit, np.abs(gn)[:, None] * pp * EPS_Z, 0.0)
    bw = REL * (np.abs(dzz).T @ np.abs(hn)) + tgt.T @ np.abs(hn) + ABS
    ew = np.abs(_f64(dw)[vr] - dw64)
    assert (ew <= bw).all(), (np.argwhere(ew > bw)[:5], ew.max())


def test_int32_targets_same_bits():
    h, w, t, g = _case(140, 128, 900, seed=41)
    _, lse = itl.linear_logp_fwd(h, w, t)
    dh, dw = itl.linear_logp_bwd(h, w, t, lse, g)
    dh2, dw2 = itl.linear_logp_bwd(h, w, t.to(torch.int32), lse, g)
    assert torch.equal(bits(dh), bits(dh2)) and torch.equal(bits(dw), bits(dw2))


@pytest.mark.parametrize("n,hd,v", [(64, 256, 4096), (257, 64, 300), (129, 512, 529)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_saved_logits_same_bits(n, hd, v, out_dtype):
    """Reading the forward's saved fp32 logits instead of recomputing h W^T
    gives dh and dW with the same bits (with temperature and entropy too).
    Unpadded rows of a ragged V are refused (16-byte rows are required)."""
    h, w, t, g = _case(n, hd, v, seed=n + 3 * v)
    gh = synth.normal_matrix(1, n, 1.0, torch.float32, seed=n + 9)[0].to(dev())
    for temp, with_ent in ((1.0, False), (0.8, True)):
        # rows of the saved logits padded to 16 bytes (a ragged V would not be)
        zbuf = torch.empty(n, (v + 3) // 4 * 4, dtype=torch.float32, device=dev())[:, :v]
        out = itl.linear_logp_fwd(h, w, t, temperature=temp, return_entropy=with_ent,
                                  return_logits=True, logits_dtype=torch.float32,
                                  logits_out=zbuf)
        lse, z = out[1], out[-1]
        ent = out[2] if with_ent else None
        kw = dict(out_dtype=out_dtype, temperature=temp, entropy=ent,
                  grad_entropy=gh if with_ent else None)
        dh0, dw0 = itl.linear_logp_bwd(h, w, t, lse, g, **kw)
        dh1, dw1 = itl.linear_logp_bwd(h, w, t, lse, g, saved_logits=z, **kw)
        assert torch.equal(dh0, dh1) and torch.equal(dw0, dw1), (temp, with_ent)
    if v % 4:
        _, lse, z = itl.linear_logp_fwd(h, w, t, return_logits=True, logits_dtype=torch.float32)
        with pytest.raises(itl.LogpError):
            itl.linear_logp_bwd(h, w, t, lse, g, saved_logits=z)


def test_logits_past_two_to_the_31_elements():
    """N = 14200 rows of the Qwen3-8B head: the forward's fp32 logits output
    holds 2.16e9 values, past 2^31.  The last rows get the same logits, logp
    and lse bits as when computed alone, and the backward that reads the saved
    logits gives the recomputing backward's dh and dW bits, so no logits
    offset wraps at 32 bits."""
    n = 14200
    c = synth.qwen3_linear(seed=95, n=n, device=dev(), ignore_frac=0.05)
    h, w, t = c["hidden"], c["weight"], c["targets"]
    assert n * w.shape[0] > 2 ** 31
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=96, device=dev())[0]
    logp, lse, z = itl.linear_logp_fwd(h, w, t, return_logits=True, logits_dtype=torch.float32)
    tail = slice(n - 16, n)
    lp_a, lse_a, z_a = itl.linear_logp_fwd(h[tail].contiguous(), w, t[tail].contiguous(),
                                           return_logits=True, logits_dtype=torch.float32)
    assert torch.equal(bits(z_a), bits(z[tail]))
    assert torch.equal(bits(lp_a), bits(logp[tail])) and torch.equal(bits(lse_a), bits(lse[tail]))
    dh0, dw0 = itl.linear_logp_bwd(h, w, t, lse, g)
    dh1, dw1 = itl.linear_logp_bwd(h, w, t, lse, g, saved_logits=z)
    assert torch.equal(bits(dh0), bits(dh1)) and torch.equal(bits(dw0), bits(dw1))


def test_saved_bf16_logits_rounded_variant():
    """In the bf16-rounded contract the bf16 logits output is exactly z, so
    reading it gives the recomputed gradient's bits; the autograd function
    with save_logits matches the default one."""
    c = synth.lattice_linear(seed=93, n=200, h=256, v=1000, device=dev(), ignore_frac=0.05)
    h, w, t = c["hidden"], c["weight"], c["targets"]
    g = synth.normal_matrix(1, 200, 1.0, torch.float32, seed=94)[0].to(dev())
    _, lse, z = itl.linear_logp_fwd(h, w, t, round_logits=True, return_logits=True)
    assert z.dtype == torch.bfloat16
    dh0, dw0 = itl.linear_logp_bwd(h, w, t, lse, g, round_logits=True)
    dh1, dw1 = itl.linear_logp_bwd(h, w, t, lse, g, round_logits=True, saved_logits=z)
    assert torch.equal(dh0, dh1) and torch.equal(dw0, dw1)
    for rnd in (False, True):
        grads = []
        for save in (False, True):
            hh = h.clone().requires_grad_(True)
            ww = w.clone().requires_grad_(True)
            (itl.linear_logp(hh, ww, t, round_logits=rnd, save_logits=save) * g).sum().backward()
            grads.append((hh.grad, ww.grad))
        assert torch.equal(grads[0][0], grads[1][0]) and torch.equal(grads[0][1], grads[1][1])


def _blocked(x, rows_p, k):
    """x [rows, k] (bf16 bits as uint16) padded with zero rows to rows_p, in
    the K32-blocked order of the product loads: element (r, c) at
    ((r // 16) * (k // 32) + c // 32) * 512 + (r % 16) * 32 + c % 32."""
    out = np.zeros((rows_p, k), dtype=np.uint16)
    out[: x.shape[0]] = x
    return out.reshape(rows_p // 16, 16, k // 32, 32).transpose(0, 2, 1, 3).reshape(-1)


@pytest.mark.parametrize("n,hd,v", [(64, 256, 4096), (257, 64, 300), (1, 128, 529),
                                    (300, 128, 1000), (90, 320, 800)])
def test_prepared_weight_same_bits(n, hd, v):
    """prepare_weight writes the weight [Vp, H] and its transpose [H, Vp]
    (zero vocabulary padding up to Vp = round_up(V, 256)) in the blocked
    order; the forward and the backward reading it give the same bits as the
    calls without it, also through autograd, into a larger buffer and after
    the buffer held other values."""
    h, w, t, g = _case(n, hd, v, seed=7 * n + v)
    vp = (v + 255) // 256 * 256
    need = itl.lib().linear_logp_prepared_bytes(v, hd)
    assert need == 2 * hd * vp * 2
    pw = itl.prepare_weight(w)
    assert pw.buffer.dtype == torch.uint8 and pw.buffer.numel() == need
    got = pw.buffer.view(torch.int16).cpu().numpy().astype(np.uint16)
    wn = w.view(torch.int16).cpu().numpy().astype(np.uint16)
    assert np.array_equal(got[: hd * vp], _blocked(wn, vp, hd))
    wt = np.zeros((hd, vp), dtype=np.uint16)
    wt[:, :v] = wn.T
    assert np.array_equal(got[hd * vp:], _blocked(wt, hd, vp))
    big = torch.full((need + 4096,), 7, dtype=torch.uint8, device=dev())
    pw2 = itl.prepare_weight(w, out=big)
    assert torch.equal(pw2.buffer[:need], pw.buffer) and bool((pw2.buffer[need:] == 7).all())
    for temp, with_ent in ((1.0, False), (0.7, True)):
        ref = itl.linear_logp_fwd(h, w, t, temperature=temp, return_entropy=with_ent,
                                  return_logits=True, logits_dtype=torch.float32)
        for prep in (pw, pw2):
            got_f = itl.linear_logp_fwd(h, w, t, temperature=temp, return_entropy=with_ent,
                                        return_logits=True, logits_dtype=torch.float32,
                                        prepared_weight=prep)
            for a, b in zip(ref, got_f):
                assert torch.equal(bits(a), bits(b))
    _, lse = itl.linear_logp_fwd(h, w, t)
    for out_dtype in (torch.float32, torch.bfloat16):
        dh0, dw0 = itl.linear_logp_bwd(h, w, t, lse, g, out_dtype=out_dtype)
        for prep in (pw, pw2):
            dh1, dw1 = itl.linear_logp_bwd(h, w, t, lse, g, out_dtype=out_dtype,
                                           prepared_weight=prep)
            assert torch.equal(dh0, dh1) and torch.equal(dw0, dw1)
    short = itl.PreparedWeight(pw.buffer[: need - 256], w)
    with pytest.raises(ValueError):
        itl.linear_logp_bwd(h, w, t, lse, g, prepared_weight=short)
    with pytest.raises(ValueError):
        itl.linear_logp_fwd(h, w, t, prepared_weight=short)
    grads = []
    for prepare in (False, True):
        hh = h.clone().requires_grad_(True)
        ww = w.clone().requires_grad_(True)
        prep = itl.prepare_weight(ww) if prepare else None
        (itl.linear_logp(hh, ww, t, prepared_weight=prep) * g).sum().backward()
        grads.append((hh.grad, ww.grad))
    assert torch.equal(grads[0][0], grads[1][0]) and torch.equal(grads[0][1], grads[1][1])


def _bits_any(x):
    return x.view(torch.int32 if x.dtype == torch.float32 else torch.int16)


@pytest.mark.parametrize("n,hd,v", [(300, 128, 1000), (64, 256, 4096), (257, 64, 5000)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_vocab_chunk_same_bits(n, hd, v, out_dtype):
    """The vocabulary chunk changes the workspace, not a bit: dh and dW from
    chunks of 256, 512 and 768 columns and the default equal those of one
    chunk over the whole vocabulary, with the logits recomputed, read from a
    prepared weight or from the forward's saved logits, with the options on
    (temperature, entropy term, bf16-rounded logits), and with only one of
    the two outputs requested."""
    h, w, t, g = _case(n, hd, v, seed=5 * n + v)
    vp = (v + 255) // 256 * 256
    pw = itl.prepare_weight(w)
    gh = synth.normal_matrix(1, n, 0.5, torch.float32, seed=n + 3)[0].to(dev())
    cases = [dict(), dict(prepared_weight=pw)]
    for temp, ent, rnd in ((1.0, False, False), (0.7, True, False), (1.3, False, True)):
        _, lse, *rest = itl.linear_logp_fwd(h, w, t, temperature=temp, return_entropy=ent,
                                            round_logits=rnd, return_logits=True,
                                            logits_dtype=torch.bfloat16 if rnd else torch.float32)
        ent_t = rest[0] if ent else None
        z = rest[-1]
        opts = dict(temperature=temp, round_logits=rnd, entropy=ent_t,
                    grad_entropy=gh if ent else None)
        for extra in cases + [dict(saved_logits=z)]:
            kw = dict(opts, **extra, out_dtype=out_dtype)
            ref = itl.linear_logp_bwd(h, w, t, lse, g, vocab_chunk=vp, **kw)
            for vc in (256, 512, 768, 0):
                got = itl.linear_logp_bwd(h, w, t, lse, g, vocab_chunk=vc, **kw)
                for a, b in zip(ref, got):
                    assert torch.equal(_bits_any(a), _bits_any(b)), (vc, temp, ent, rnd,
                                                                    list(extra))
            dh_only, none_w = itl.linear_logp_bwd(h, w, t, lse, g, vocab_chunk=256,
                                                  need_dweight=False, **kw)
            none_h, dw_only = itl.linear_logp_bwd(h, w, t, lse, g, vocab_chunk=512,
                                                  need_dhidden=False, **kw)
            assert none_w is None and none_h is None
            assert torch.equal(_bits_any(dh_only), _bits_any(ref[0]))
            assert torch.equal(_bits_any(dw_only), _bits_any(ref[1]))


def test_vocab_chunk_full_size_same_bits():
    """The Qwen3-8B head (H = 4096, V = 151936) at N = 512: the default chunk
    (the benchmarked launch sequence, 5 chunks) against one chunk over the
    whole vocabulary, fp32 and bf16 outputs; and the default workspace stays
    far below the one-chunk workspace."""
    h, w, t, g = _case(512, synth.QWEN3_HIDDEN, synth.QWEN3_VOCAB, seed=77)
    _, lse = itl.linear_logp_fwd(h, w, t)
    vp = (synth.QWEN3_VOCAB + 255) // 256 * 256
    for out_dtype in (torch.float32, torch.bfloat16):
        one = itl.linear_logp_bwd(h, w, t, lse, g, vocab_chunk=vp, out_dtype=out_dtype)
        dflt = itl.linear_logp_bwd(h, w, t, lse, g, out_dtype=out_dtype)
        for a, b in zip(one, dflt):
            assert torch.equal(_bits_any(a), _bits_any(b)), out_dtype
    big = itl.linear_logp_bwd_workspace_bytes(512, 4096, synth.QWEN3_VOCAB, vocab_chunk=vp)
    small = itl.linear_logp_bwd_workspace_bytes(512, 4096, synth.QWEN3_VOCAB)
    assert small * 3 < big
