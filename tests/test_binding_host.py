"""Checks of the PyTorch binding that need no GPU: a prepared LM-head weight
is tied to the weight tensor it was made from and refused, before any device
work, once that weight changed in place or when another tensor is passed."""

import pytest
import torch

import invariant_token_log_amd as itl


def _case():
    n, h, v = 4, 64, 300
    hidden = torch.zeros(n, h, dtype=torch.bfloat16)
    weight = torch.zeros(v, h, dtype=torch.bfloat16)
    targets = torch.zeros(n, dtype=torch.int64)
    lse = torch.zeros(n)
    g = torch.ones(n)
    return hidden, weight, targets, lse, g


def test_prepared_weight_refused_after_in_place_update():
    hidden, weight, targets, lse, g = _case()
    pw = itl.PreparedWeight(torch.zeros(16, dtype=torch.uint8), weight)
    pw.check(weight)  # unchanged: accepted
    weight.add_(1.0)  # an optimiser-style in-place update bumps the version
    with pytest.raises(ValueError, match="stale"):
        itl.linear_logp_fwd(hidden, weight, targets, prepared_weight=pw)
    with pytest.raises(ValueError, match="stale"):
        itl.linear_logp_bwd(hidden, weight, targets, lse, g, prepared_weight=pw)
    with pytest.raises(ValueError, match="stale"):
        itl.linear_logp_fwd_noalloc(hidden, weight, targets, prepared_weight=pw)


def test_prepared_weight_refused_for_another_tensor():
    hidden, weight, targets, lse, g = _case()
    pw = itl.PreparedWeight(torch.zeros(16, dtype=torch.uint8), weight)
    other = weight.clone()  # same values, another tensor
    with pytest.raises(ValueError, match="another weight"):
        itl.linear_logp_fwd(hidden, other, targets, prepared_weight=pw)
    with pytest.raises(ValueError, match="another weight"):
        itl.linear_logp_bwd(hidden, weight[:200], targets, lse, g, prepared_weight=pw)
    with pytest.raises(TypeError):
        itl.linear_logp_fwd(hidden, weight, targets, prepared_weight=pw.buffer)
