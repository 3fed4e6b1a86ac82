"""GPU parity and invariance of logp_fwd against the float64 oracle.

Sources: "Batch-Invariant LogP" (opening definition, Reference Semantics,
Tensor Parallel, Batch-Invariance, Minimal Example)."""

import math

import numpy as np
import pytest
import torch

import invariant_token_log_amd as itl
import oracle
import synth
from gpu_helpers import assert_grad_parity, assert_logp_parity, bits, dev, to_np

pytestmark = pytest.mark.gpu

V = synth.QWEN3_VOCAB


def _oracle(logits, targets, ignore_index=-100):
    x = logits.detach().float().cpu().numpy()
    return oracle.logp_fwd(x, targets.cpu().numpy(), ignore_index)


def test_tiny_fp32_w512():
    """fp32 [64, 4096], tile width 512, 4 ignored rows."""
    c = synth.tiny_fp32()
    x = c["logits"].to(dev())
    t = c["targets"].to(dev())
    logp, lse = itl.logp_fwd(x, t, -100, 512)
    ref = _oracle(c["logits"], c["targets"])
    assert_logp_parity(logp, lse, *ref, t, what="tiny fp32")
    a = (c["targets"] != -100).numpy()
    assert (to_np(logp)[a] <= 0.0).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_v8_rows_one_padded_tile(dtype):
    """V = 8: one tile of 512 columns, 504 of them padding (T = 1)."""
    c = synth.tiny_v8(n=16)
    x = c["logits"].to(dtype)
    logp, lse = itl.logp_fwd(x.to(dev()), c["targets"].to(dev()), -100, 512)
    assert_logp_parity(logp, lse, *_oracle(x, c["targets"]), c["targets"], what=f"v8 {dtype}")


@pytest.mark.parametrize("v", [8, 300, 4096, V])
@pytest.mark.parametrize("value", [0.0, 1.7, -3.25])
def test_constant_rows_closed_form(v, value):
    """All-equal row: every s_k and the merged sum are exact integers (the
    sum is exactly V), so logp is -log V up to the rounding of the device
    log and of the final add/subtract: 2 ulp for c = 0, 4 ulp otherwise.  A
    sum off by even one unit would miss by about 1/V, far outside."""
    w = 512 if v < 4096 else 4096
    x = synth.constant_rows(v, [value] * 3).to(dev())
    t = torch.tensor([0, v // 2, v - 1], device=dev())
    logp, lse = itl.logp_fwd(x, t, -100, w)
    want = np.float32(-math.log(v))
    got = logp.cpu().numpy()
    assert (got == got[0]).all()
    ulp = float(np.spacing(np.float32(abs(want))))
    k = 2 if value == 0.0 else 4
    assert abs(float(got[0]) - float(want)) <= k * ulp, (got[0], want)


_RAGGED = [(300, 512), (4099, 512), (4096 + 8, 1024), (151936, 4096), (12345, 2048)]


# fp32 tiles stop at 4096 columns, so the 8192-wide tile runs on bf16 only.
@pytest.mark.parametrize("v,w,dtype",
                         [(v, w, d) for v, w in _RAGGED for d in (torch.float32, torch.bfloat16)]
                         + [(151936 - 8, 8192, torch.bfloat16)])
def test_ragged_shapes(v, w, dtype):
    """Ragged vocabularies (last tile partly padding), unaligned rows
    (v * size not a multiple of 16 takes the element-wise load path)."""
    n = 37
    x = synth.normal_matrix(n, v, 3.0, dtype, seed=v + w).to(dev())
    t = synth.uniform_targets(n, v, seed=v, ignore_rows=torch.tensor([3, 17])).to(dev())
    logp, lse = itl.logp_fwd(x, t, -100, w)
    assert_logp_parity(logp, lse, *_oracle(x, t), t, what=f"ragged {v} {w} {dtype}")


def test_minimal_example_shape():
    """[2, 4, 300] bf16 with target[0, 0] = -100 ("Batch-Invariant LogP",
    Minimal Example): output shaped like the targets, float32, 0 at [0, 0]."""
    g = torch.Generator().manual_seed(0)
    x = torch.randn(2, 4, 300, generator=g).to(torch.bfloat16).to(dev())
    t = torch.randint(0, 300, (2, 4), generator=g).to(dev())
    t[0, 0] = -100
    out = itl.batch_invariant_logp(x, t, -100, 512)
    assert out.shape == t.shape and out.dtype == torch.float32
    assert out[0, 0].item() == 0.0
    ref, _ = _oracle(x, t)
    np.testing.assert_allclose(to_np(out).reshape(-1), ref, atol=1e-5, rtol=1e-5)


@pytest.fixture(scope="module")
def qwen_small():
    """512 rows of the Qwen3-vocab forward workload (spikes, ignored rows)."""
    c = synth.qwen3_fwd(n=512, device=dev())
    return c


def test_qwen_vocab_parity(qwen_small):
    c = qwen_small
    logp, lse = itl.logp_fwd(c["logits"], c["targets"], -100, 4096)
    err = assert_logp_parity(logp, lse, *_oracle(c["logits"], c["targets"]), c["targets"],
                             what="qwen 512")
    assert err < 1e-4
    a = (c["targets"] != -100).cpu().numpy()
    assert (to_np(logp)[a] <= 0.0).all(), "logp <= 0 must hold bitwise"


def test_spike_on_target():
    """Target on a +40 spike: logp is ~0 and never positive."""
    x = synth.normal_matrix(8, V, 3.0, torch.float32, seed=77)
    cols = torch.tensor([0, 1, 4095, 4096, 77777, V - 385, V - 384, V - 1])
    x[torch.arange(8), cols] += 40.0
    x = x.to(torch.bfloat16).to(dev())
    t = cols.to(dev())
    logp, lse = itl.logp_fwd(x, t, -100, 4096)
    assert_logp_parity(logp, lse, *_oracle(x, t), t, what="spike")
    assert (to_np(logp) <= 0.0).all()


@pytest.mark.parametrize("shards", [2, 4])
def test_shards_bitwise_equal(qwen_small, shards):
    """S = 2 and 4 emulated vocabulary shards give the same bits as S = 1
    ("Batch-Invariant LogP", Tensor Parallel)."""
    c = qwen_small
    l1, s1 = itl.logp_fwd(c["logits"], c["targets"], -100, 4096, 1)
    l2, s2 = itl.logp_fwd(c["logits"], c["targets"], -100, 4096, shards)
    assert torch.equal(bits(l1), bits(l2))
    assert torch.equal(bits(s1), bits(s2))


@pytest.mark.parametrize("shards", [2, 8])
def test_shards_small_tiles(shards):
    """Shard emulation with one-tile shards and a padded last tile."""
    v = 4096 + 512 * 3 + 256  # 5888, divisible by 2 and 8? 5888 = 2^8 * 23
    x = synth.normal_matrix(40, v, 2.0, torch.float32, seed=5).to(dev())
    t = synth.uniform_targets(40, v, seed=6, ignore_rows=torch.tensor([0])).to(dev())
    l1, s1 = itl.logp_fwd(x, t, -100, 256, 1)
    l2, s2 = itl.logp_fwd(x, t, -100, 256, shards)
    assert torch.equal(bits(l1), bits(l2)) and torch.equal(bits(s1), bits(s2))
    assert_logp_parity(l2, s2, *_oracle(x, t), t, what="small shards")


def test_many_tiles_merge_groups():
    """More than 1024 tiles per row (fp32, 256-wide tiles, V = 300000: 1172
    tiles): the merge holds at most 1024 tiles per lane group in registers
    (64 in the single-launch forward), so every path folds several groups.
    S = 1, 2 and 4 give the same bits (entropy included) and match the
    oracle."""
    v, n = 300000, 6
    x = synth.normal_matrix(n, v, 3.0, torch.float32, seed=31).to(dev())
    x[2, 299999] = 45.0  # a spike in the last, ragged tile
    t = synth.uniform_targets(n, v, seed=32, ignore_rows=torch.tensor([4])).to(dev())
    t[2] = 299999
    l1, s1, e1 = itl.logp_fwd(x, t, -100, 256, 1, return_entropy=True)
    for shards in (2, 4):
        ls, ss, es = itl.logp_fwd(x, t, -100, 256, shards, return_entropy=True)
        assert torch.equal(bits(ls), bits(l1)) and torch.equal(bits(ss), bits(s1)), shards
        assert torch.equal(bits(es), bits(e1)), shards
    assert_logp_parity(l1, s1, *_oracle(x, t), t, what="1172 tiles")


def test_row_invariance(qwen_small):
    """A row's bits do not depend on the batch: alone, reversed, permuted,
    packed among random neighbours, repeated, on another stream."""
    c = qwen_small
    x, t = c["logits"], c["targets"]
    base, base_lse = itl.logp_fwd(x, t, -100, 4096)
    b0 = bits(base)
    # alone, one row per call, from a fresh buffer: 16-byte aligned (offset
    # 8 elements) and unaligned (offset 1, element-wise loads)
    for r in [0, 1, 7, 100, 255, 511]:
        for off in (8, 1):
            xr = torch.empty(1, V + 8, dtype=x.dtype, device=dev())[:, off:off + V]
            xr.copy_(x[r:r + 1])
            lr, _ = itl.logp_fwd(xr, t[r:r + 1].clone(), -100, 4096)
            assert torch.equal(bits(lr), b0[r:r + 1]), (r, off)
    # reversed
    rev = torch.arange(x.shape[0] - 1, -1, -1, device=dev())
    lr, _ = itl.logp_fwd(x[rev].contiguous(), t[rev].contiguous(), -100, 4096)
    assert torch.equal(bits(lr), b0[rev.cpu()])
    # permuted
    perm = torch.randperm(x.shape[0], generator=torch.Generator().manual_seed(3)).to(dev())
    lp, _ = itl.logp_fwd(x[perm].contiguous(), t[perm].contiguous(), -100, 4096)
    assert torch.equal(bits(lp), b0[perm.cpu()])
    # packed among neighbours at an odd offset
    nb_x, nb_t = synth.random_rows(1000, V, seed=11, device=dev())
    packed = torch.cat([nb_x[:333], x, nb_x[333:]])
    packed_t = torch.cat([nb_t[:333], t, nb_t[333:]])
    lk, _ = itl.logp_fwd(packed, packed_t, -100, 4096)
    assert torch.equal(bits(lk)[333:333 + x.shape[0]], b0)
    # repeat and another stream
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        l2, _ = itl.logp_fwd(x, t, -100, 4096)
    s.synchronize()
    assert torch.equal(bits(l2), b0)


def test_replicated_row_all_targets():
    """One row replicated V times with targets 0..V-1: every replica has the
    same lse bits and logp_j = fl32(x_j - lse)."""
    v = 4096
    row = synth.normal_matrix(1, v, 2.0, torch.float32, seed=9)
    x = row.expand(v, v).contiguous().to(dev())
    t = torch.arange(v, device=dev())
    logp, lse = itl.logp_fwd(x, t, -100, 512)
    lb = bits(lse)
    assert (lb == lb[0]).all()
    want = (row[0].to(dev()) - lse[0]).cpu()
    assert torch.equal(bits(logp), bits(want))
    assert abs(math.fsum(np.exp(to_np(logp))) - 1.0) < 1e-5


def test_ignore_index_minus_one():
    """target -1 is an ignored row only when ignore_index is -1."""
    x = synth.normal_matrix(4, 1000, 1.0, torch.float32, seed=1).to(dev())
    t = torch.tensor([5, -1, 999, 0], device=dev())
    logp, lse = itl.logp_fwd(x, t, -1, 512)
    assert logp[1].item() == 0.0
    assert_logp_parity(logp, lse, *_oracle(x, t, -1), t, ignore_index=-1, what="ignore -1")


def test_invalid_targets():
    """validate=1 reports an active target outside [0, V); both modes give
    NaN on that row and leave the other rows exact."""
    x = synth.normal_matrix(6, 5000, 1.0, torch.bfloat16, seed=2).to(dev())
    t = torch.tensor([1, 5000, -100, -1, 4999, 123456789], device=dev())
    logp, lse = itl.logp_fwd(x, t, -100, 512, validate=False)
    got = logp.cpu()
    assert torch.isnan(got[[1, 3, 5]]).all()
    assert got[2].item() == 0.0
    with pytest.raises(itl.LogpError) as ei:
        itl.logp_fwd(x, t, -100, 512, validate=True)
    assert ei.value.status == 8
    for s in (1, 2, 4):
        ok_t = torch.tensor([1, 4, -100, 7, 4999, 0], device=dev())
        itl.logp_fwd(x, ok_t, -100, 512, num_shards=s, validate=True)
    ref, _ = _oracle(x[[0, 4]], t[[0, 4]])
    np.testing.assert_allclose(to_np(logp)[[0, 4]], ref, atol=1e-5, rtol=1e-5)


@pytest.mark.parametrize("shards", [1, 2, 4])
def test_validate_invalid_targets_under_shards(shards):
    """validate=1 under S = 1, 2, 4 shards: LOGP_ERR_TARGET after the sync;
    rows with an active target outside [0, V) hold NaN and only those, the
    ignored row +0, and every other output has the bits of the call without
    validation (whose merge took the same path)."""
    x = synth.normal_matrix(6, 5000, 1.0, torch.bfloat16, seed=2).to(dev())
    t = torch.tensor([1, 5000, -100, -1, 4999, 123456789], device=dev())
    ref_logp, ref_lse = itl.logp_fwd(x, t, -100, 512, num_shards=1, validate=False)
    logp = torch.full((6,), 7.0, device=dev())
    lse = torch.full((6,), 7.0, device=dev())
    with pytest.raises(itl.LogpError) as ei:
        itl.logp_fwd(x, t, -100, 512, num_shards=shards, validate=True, logp_out=logp,
                     lse_out=lse)
    assert ei.value.status == 8
    got = logp.cpu()
    assert torch.isnan(got[[1, 3, 5]]).all()
    assert not torch.isnan(got[[0, 2, 4]]).any()
    assert bits(logp)[2].item() == 0 and bits(lse)[2].item() == 0
    ok = torch.tensor([0, 4])
    assert torch.equal(bits(logp)[ok], bits(ref_logp)[ok])
    # the LSE of a row does not depend on its target
    assert torch.equal(bits(lse)[[0, 1, 3, 4, 5]], bits(ref_lse)[[0, 1, 3, 4, 5]])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_masked_and_huge_logits(dtype):
    """Masked vocabulary entries (-inf): half a row, whole leading tiles, every
    other column, a row whose only finite logit is its target (logp exactly
    +0); and logits of magnitude 1e37.  logp, lse and dlogits against the
    oracle, and the 2-shard forward with the same bits."""
    v, w, n = 5000, 512, 8
    inf = float("inf")
    x = synth.normal_matrix(n, v, 3.0, torch.float32, seed=91)
    t = torch.tensor([10, 2600, 4999, 8, 100, 3000, 1, 4000])
    x[0, 2500:] = -inf
    x[1, :2560] = -inf
    x[2, :] = -inf
    x[2, 4999] = 1.5
    x[3, 1::2] = -inf
    x[4, 50], x[4, 60] = 1e37, -1e37
    x[6, 1] = 1e37
    x[7, :] = -1e37
    x[7, 4000] = 0.0
    x = x.to(dtype).to(dev())
    t = t.to(dev())
    logp, lse = itl.logp_fwd(x, t, -100, w)
    x64, tn = to_np(x), t.cpu().numpy()
    ref_logp, ref_lse = oracle.logp_fwd(x64, tn)
    assert_logp_parity(logp, lse, ref_logp, ref_lse, t, what=f"masked {dtype}")
    assert bits(logp)[2] == 0 and bits(logp)[7] == 0
    lp2, lse2 = itl.logp_fwd(x, t, -100, w, num_shards=2)
    assert torch.equal(bits(lp2), bits(logp)) and torch.equal(bits(lse2), bits(lse))
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=92)[0].to(dev())
    d = itl.logp_bwd(x, t, lse, g, -100, w)
    d64 = oracle.logp_bwd(x64, tn, to_np(g), lse=ref_lse)
    assert_grad_parity(d, d64, x64, ref_lse, to_np(g), t, what=f"masked bwd {dtype}")


def test_empty_batch():
    x = torch.empty(0, V, dtype=torch.bfloat16, device=dev())
    t = torch.empty(0, dtype=torch.int64, device=dev())
    logp, lse = itl.logp_fwd(x, t, -100, 4096)
    assert logp.numel() == 0 and lse.numel() == 0


def test_all_ignored():
    x = synth.normal_matrix(16, 4096, 1.0, torch.bfloat16, seed=4).to(dev())
    t = torch.full((16,), -100, device=dev())
    for s in (1, 2):
        logp, lse = itl.logp_fwd(x, t, -100, 512, s)
        assert (bits(logp) == 0).all() and (bits(lse) == 0).all()


def test_full_size_sampled():
    """N = 4096 Qwen3-vocab workload at the benchmarked launch: sampled rows
    (every spike row, every 37th row, some ignored) against the oracle."""
    c = synth.qwen3_fwd(device=dev())
    logp, lse = itl.logp_fwd(c["logits"], c["targets"], -100, 4096)
    rows = sorted(set(c["spike_rows"].tolist()) | set(range(0, 4096, 37)))
    idx = torch.tensor(rows, device=dev())
    ref = _oracle(c["logits"][idx], c["targets"][idx])
    assert_logp_parity(logp[idx], lse[idx], *ref, c["targets"][idx], what="full sample")
    a = (c["targets"] != -100)
    assert (logp[a] <= 0).all()
    assert (bits(logp[~a]) == 0).all()


@pytest.mark.parametrize("v,w", [(300, 512), (4099, 1024), (151936, 4096)])
def test_fp16_logits(v, w):
    """fp16 logits ("Batch-Invariant LogP", Tensor Contract: fp32 / fp16 /
    bf16) widen exactly; parity with the oracle on the same fp16 values."""
    n = 33
    x = synth.normal_matrix(n, v, 3.0, torch.float16, seed=v + 1).to(dev())
    t = synth.uniform_targets(n, v, seed=v + 2, ignore_rows=torch.tensor([4])).to(dev())
    logp, lse = itl.logp_fwd(x, t, -100, w)
    assert_logp_parity(logp, lse, *_oracle(x, t), t, what=f"fp16 {v}")
    a = (t != -100)
    assert (logp[a] <= 0).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_int32_targets_same_bits(dtype):
    """int32 targets give the same bits as int64 targets (all S)."""
    x = synth.normal_matrix(40, 5000, 2.0, dtype, seed=12).to(dev())
    t = synth.uniform_targets(40, 5000, seed=13, ignore_rows=torch.tensor([0, 39])).to(dev())
    for s in (1, 2):
        a, la = itl.logp_fwd(x, t, -100, 512, s)
        b, lb = itl.logp_fwd(x, t.to(torch.int32), -100, 512, s)
        assert torch.equal(bits(a), bits(b)) and torch.equal(bits(la), bits(lb))
