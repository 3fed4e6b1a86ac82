"""The fused LM-head forward's entry point that takes no workspace
(linear_logp_fwd_noalloc, for callers that cannot allocate device memory)
gives the same bits as linear_logp_fwd with a caller workspace, called through
the C ABI twice in a row (the second call smaller, so it runs on scratch the
first one left behind), and refuses a problem larger than its static scratch
array with LOGP_ERR_SCRATCH before enqueuing anything."""

import ctypes

import pytest
import torch

import invariant_token_log_amd as itl
import synth
from invariant_token_log_amd import _lib
from gpu_helpers import bits, dev

pytestmark = pytest.mark.gpu


def _noalloc(hid, wt, t, logp, lse, ent=None, z=None, temperature=1.0):
    """linear_logp_fwd_noalloc through ctypes, on the current stream."""
    n, h = hid.shape
    v = wt.shape[0]
    with torch.cuda.device(hid.device):
        return itl.lib().linear_logp_fwd_noalloc(
            hid.data_ptr(), h, wt.data_ptr(), h, n, h, v, t.data_ptr(), _lib.LOGP_I64, -100,
            256, ctypes.c_float(temperature), _lib.LOGP_ROUND_NONE, logp.data_ptr(),
            lse.data_ptr(), ent.data_ptr() if ent is not None else None,
            z.data_ptr() if z is not None else None, _lib.LOGP_F32, v if z is not None else 0,
            None, 0, torch.cuda.current_stream(hid.device).cuda_stream)


def _case(seed, n, h, v):
    c = synth.qwen3_linear(seed=seed, n=n, h=h, v=v, device=dev(), ignore_frac=0.05)
    return c["hidden"], c["weight"], c["targets"]


def _outputs(n, v, with_logits):
    f = dict(dtype=torch.float32, device=dev())
    logp = torch.full((n,), 7.0, **f)  # sentinels: every element must be overwritten
    lse = torch.full((n,), 7.0, **f)
    ent = torch.full((n,), 7.0, **f)
    z = torch.full((n, v), 7.0, **f) if with_logits else None
    return logp, lse, ent, z


def _check_same_bits(hid, wt, t, temperature, with_logits):
    n, v = hid.shape[0], wt.shape[0]
    logp, lse, ent, z = _outputs(n, v, with_logits)
    st = _noalloc(hid, wt, t, logp, lse, ent, z, temperature)
    assert st == _lib.LOGP_OK, itl.status_str(st)
    ref = itl.linear_logp_fwd(hid, wt, t, temperature=temperature, return_entropy=True,
                              return_logits=with_logits, logits_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(bits(logp), bits(ref[0]))
    assert torch.equal(bits(lse), bits(ref[1]))
    assert torch.equal(bits(ent), bits(ref[2]))
    if with_logits:
        assert torch.equal(bits(z), bits(ref[3]))


def test_two_calls_in_a_row_same_bits_as_workspace_entry_point():
    # First call at the benchmarked LM-head size (N = H = 4096, V = 151936):
    # partial tables and the re-laid hidden rows fill ~60 MiB of the scratch.
    n, h, v = 4096, synth.QWEN3_HIDDEN, synth.QWEN3_VOCAB
    need = itl.lib().linear_logp_fwd_workspace_bytes(n, h, v, 256)
    assert 0 < need <= itl.NOALLOC_SCRATCH_BYTES
    print(f"noalloc: N={n} H={h} V={v} (scratch use {need} B)", flush=True)
    _check_same_bits(*_case(901, n, h, v), temperature=1.0, with_logits=False)
    # Second call, smaller (the 256-row tile over a ragged V, with the
    # temperature, entropy and logits output): it runs on what the first left.
    print("noalloc: N=300 H=512 V=5000", flush=True)
    _check_same_bits(*_case(902, 300, 512, 5000), temperature=0.7, with_logits=True)
    # Third, smaller again: the narrow 64-row tile.
    print("noalloc: N=40 H=256 V=4096", flush=True)
    _check_same_bits(*_case(903, 40, 256, 4096), temperature=1.0, with_logits=False)


def test_too_large_for_scratch_is_refused_untouched():
    n, h, v = 8192, synth.QWEN3_HIDDEN, synth.QWEN3_VOCAB
    assert itl.lib().linear_logp_fwd_workspace_bytes(n, h, v, 256) > itl.NOALLOC_SCRATCH_BYTES
    hid = torch.zeros(n, h, dtype=torch.bfloat16, device=dev())
    wt = torch.zeros(v, h, dtype=torch.bfloat16, device=dev())
    t = torch.zeros(n, dtype=torch.int64, device=dev())
    logp, lse, _, _ = _outputs(n, 1, False)
    st = _noalloc(hid, wt, t, logp, lse)
    torch.cuda.synchronize()
    assert st == _lib.LOGP_ERR_SCRATCH
    assert (logp == 7.0).all() and (lse == 7.0).all()  # nothing was enqueued
    with pytest.raises(itl.LogpError) as e:
        itl.linear_logp_fwd_noalloc(hid, wt, t, logp_out=logp, lse_out=lse)
    assert e.value.status == _lib.LOGP_ERR_SCRATCH
