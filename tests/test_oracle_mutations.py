"""The oracle's pins catch planted mistakes (CPU only).

Each case below plants one plausible slip in the float64 oracle (a wrong
sign, a dropped term, a shifted column, a transposed operand, a lost padding
or ownership rule, a temperature applied the wrong way), then runs every pin
of tests/test_oracle_pins.py against the planted version and requires that at
least one pin fails.  The planted versions are wrappers or small rewrites of
the oracle's own functions, patched into the oracle module so that the
oracle's internal calls see them too, exactly as a real slip would spread.

Sources of the arithmetic being mutated: "Batch-Invariant LogP" (opening
definition, Reference Semantics, Tensor Parallel, Batch-Invariance, VIME CP=2
runtime provider) and the fused LM-head operator of "[RFC][ROCm] End-to-end
optimization of bitwise VIME R/R beyond native P/P" (Workstream 3).
"""

import importlib.util
import inspect
import itertools
import math
import os

import numpy as np
import pytest

import oracle
from oracle import logp_oracle as lo

_HERE = os.path.dirname(os.path.abspath(__file__))


def _load_pins():
    spec = importlib.util.spec_from_file_location(
        "_oracle_pins_for_mutation", os.path.join(_HERE, "test_oracle_pins.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _pin_calls(mod):
    """(id, function, kwargs) for every pin and every parameter set."""
    out = []
    for name in sorted(dir(mod)):
        f = getattr(mod, name)
        if not name.startswith("test_") or not callable(f):
            continue
        grids = []
        for mark in getattr(f, "pytestmark", []):
            if mark.name != "parametrize":
                continue
            names, values = mark.args[0], mark.args[1]
            names = [a.strip() for a in names.split(",")] if isinstance(names, str) else list(names)
            sets = []
            for val in values:
                tup = tuple(val) if len(names) > 1 else (val,)
                sets.append(dict(zip(names, tup)))
            grids.append(sets)
        for combo in itertools.product(*grids) if grids else [()]:
            kwargs = {}
            for part in combo:
                kwargs.update(part)
            params = set(inspect.signature(f).parameters)
            assert params <= set(kwargs), f"{name} needs fixtures {params - set(kwargs)}"
            out.append((f"{name}{sorted(kwargs) if kwargs else ''}", f, kwargs))
    return out


PINS = _pin_calls(_load_pins())


def _first_failure():
    for pid, f, kwargs in PINS:
        try:
            f(**kwargs)
        except Exception as e:  # an assertion, or the planted oracle failing loudly
            return pid, type(e).__name__
    return None


# ---------------------------------------------------------------------------
# Planted mistakes.  Each returns {oracle function name: planted version}.
# ---------------------------------------------------------------------------
_orig = {name: getattr(lo, name) for name in (
    "logp_fwd", "logp_bwd", "entropy", "entropy_bwd", "linear_logits", "_lm_logits",
    "linear_logp_bwd", "linear_logp_bwd_weight_rows", "tile_partials", "merge_partials",
    "shard_tile_ranges", "round_bf16")}


def _rows_and_targets(logits, targets, ignore_index):
    x2 = lo._as_2d(logits).astype(np.float64)
    active, t = lo._active_mask(targets, ignore_index, x2.shape[1])
    return x2, active, t


def _fwd_from(lse_fn, target_col=lambda t, v: t, ignored_value=None):
    """logp_fwd rebuilt with a planted lse, target column or ignored-row rule."""
    def fwd(logits, targets, ignore_index=-100):
        x2, active, t = _rows_and_targets(logits, targets, ignore_index)
        n, v = x2.shape
        logp = np.zeros(n)
        lse = np.zeros(n)
        for r in range(n):
            if not active[r]:
                if ignored_value is not None:
                    lse[r] = lse_fn(x2[r])
                    logp[r] = x2[r, 0] - lse[r]
                continue
            lse[r] = lse_fn(x2[r])
            logp[r] = x2[r, target_col(int(t[r]), v)] - lse[r]
        return logp, lse
    return fwd


def _lse_true(x):
    m = x.max()
    return m + math.log(np.exp(x - m).sum())


def m_logp_sign():
    f = _orig["logp_fwd"]
    return {"logp_fwd": lambda *a, **k: tuple(np.negative(o) if i == 0 else o
                                              for i, o in enumerate(f(*a, **k)))}


def m_no_max_shift():
    return {"logp_fwd": _fwd_from(lambda x: math.log(np.exp(x).sum()))}


def m_log_mean_exp():
    return {"logp_fwd": _fwd_from(lambda x: _lse_true(x) - math.log(x.shape[0]))}


def m_target_off_by_one():
    return {"logp_fwd": _fwd_from(_lse_true, target_col=lambda t, v: (t + 1) % v)}


def m_target_term_dropped():
    def lse_wo_max(x):  # the sum skips the largest entry
        m = x.max()
        e = np.exp(x - m)
        e[np.argmax(x)] = 0.0
        return m + math.log(e.sum() + 1e-300)
    return {"logp_fwd": _fwd_from(lse_wo_max)}


def m_ignored_not_zero():
    return {"logp_fwd": _fwd_from(_lse_true, ignored_value=True)}


def m_bwd_sign():
    f = _orig["logp_bwd"]
    return {"logp_bwd": lambda *a, **k: -f(*a, **k)}


def m_bwd_no_onehot():
    f = _orig["logp_bwd"]

    def bwd(logits, targets, grad_logp, ignore_index=-100, lse=None):
        d = f(logits, targets, grad_logp, ignore_index, lse)
        x2, active, t = _rows_and_targets(logits, targets, ignore_index)
        g = np.asarray(grad_logp, dtype=np.float64).reshape(-1)
        rows = np.flatnonzero(active)
        d[rows, t[rows]] -= g[rows]
        return d
    return {"logp_bwd": bwd}


def m_bwd_unnormalised():
    def bwd(logits, targets, grad_logp, ignore_index=-100, lse=None):
        x2, active, t = _rows_and_targets(logits, targets, ignore_index)
        g = np.asarray(grad_logp, dtype=np.float64).reshape(-1)
        d = np.zeros_like(x2)
        for r in np.flatnonzero(active):
            p = np.exp(x2[r] - x2[r].max())  # softmax numerator only
            d[r] = -g[r] * p
            d[r, t[r]] += g[r]
        return d
    return {"logp_bwd": bwd}


def m_bwd_no_grad_scale():
    f = _orig["logp_bwd"]

    def bwd(logits, targets, grad_logp, ignore_index=-100, lse=None):
        return f(logits, targets, np.ones(np.asarray(grad_logp).size), ignore_index, lse)
    return {"logp_bwd": bwd}


def m_entropy_sign():
    f = _orig["entropy"]
    return {"entropy": lambda *a, **k: -f(*a, **k)}


def m_entropy_bwd_no_h():
    def ebwd(logits, targets, grad_entropy, ignore_index=-100):
        x2, active, t = _rows_and_targets(logits, targets, ignore_index)
        gh = np.asarray(grad_entropy, dtype=np.float64).reshape(-1)
        d = np.zeros_like(x2)
        for r in np.flatnonzero(active):
            lp = x2[r] - _lse_true(x2[r])
            d[r] = -gh[r] * np.exp(lp) * lp
        return d
    return {"entropy_bwd": ebwd}


def m_weight_not_transposed():
    def logits(hidden, weight):
        h = np.asarray(hidden, dtype=np.float64)
        w = np.asarray(weight, dtype=np.float64)
        if w.shape[0] == w.shape[1]:
            return h @ w
        return (h @ w.reshape(w.shape[1], w.shape[0])).astype(np.float64)
    return {"linear_logits": logits}


def m_temperature_multiplies():
    def lm(h, w, temperature, round_logits):
        z = lo.linear_logits(h, w)
        if round_logits:
            z = lo.round_bf16(z)
        return z * float(temperature)
    return {"_lm_logits": lm}


def m_bwd_dz_not_scaled():
    f = _orig["linear_logp_bwd"]

    def bwd(hidden, weight, targets, grad_logp, ignore_index=-100, lse=None, need_dweight=True,
            temperature=1.0, grad_entropy=None, round_logits=False):
        dh, dw = f(hidden, weight, targets, grad_logp, ignore_index, lse, need_dweight,
                   temperature, grad_entropy, round_logits)
        t = float(temperature)
        return dh * t, (None if dw is None else dw * t)
    return {"linear_logp_bwd": bwd}


def m_dweight_last_block_only():
    def bwd(hidden, weight, targets, grad_logp, ignore_index=-100, lse=None, need_dweight=True,
            temperature=1.0, grad_entropy=None, round_logits=False):
        dh, dw = _orig["linear_logp_bwd"](hidden, weight, targets, grad_logp, ignore_index, lse,
                                          need_dweight, temperature, grad_entropy, round_logits)
        if dw is None:
            return dh, dw
        n = np.asarray(hidden).shape[0]
        last = (n - 1) // 2 * 2  # the sum over rows loses all but the last two
        if last > 0:
            keep = np.zeros(n, dtype=bool)
            keep[last:] = True
            g = np.where(keep, np.asarray(grad_logp, dtype=np.float64).reshape(-1), 0.0)
            gh = None if grad_entropy is None else np.where(
                keep, np.asarray(grad_entropy, dtype=np.float64).reshape(-1), 0.0)
            _, dw = _orig["linear_logp_bwd"](hidden, weight, targets, g, ignore_index, lse,
                                             True, temperature, gh, round_logits)
        return dh, dw
    return {"linear_logp_bwd": bwd}


def m_merge_exponent_sign():
    def merge(m, s, dtype=np.float64):
        m = np.asarray(m, dtype=dtype)
        s = np.asarray(s, dtype=dtype)
        big_m = m.max()
        acc = dtype(0.0)
        for k in range(m.shape[0]):
            if not np.isneginf(m[k]):
                acc = dtype(acc + s[k] * np.exp(dtype(big_m - m[k])))
        return dtype(big_m + np.log(acc))
    return {"merge_partials": merge}


def m_padding_zero():
    def partials(x_row, tile_width, dtype=np.float64):
        x = np.asarray(x_row, dtype=dtype).reshape(-1)
        t_count = lo.num_tiles(x.shape[0], tile_width)
        padded = np.zeros(t_count * tile_width, dtype=dtype)  # should be -inf
        padded[:x.shape[0]] = x
        tiles = padded.reshape(t_count, tile_width)
        m = tiles.max(axis=1)
        s = np.array([np.exp(tiles[k] - m[k]).sum(dtype=dtype) for k in range(t_count)],
                     dtype=dtype)
        return m, s
    return {"tile_partials": partials}


def m_shard_ownership_shifted():
    f = _orig["shard_tile_ranges"]

    def ranges(v, tile_width, num_shards):
        out = f(v, tile_width, num_shards)
        if len(out) > 1:
            (a0, b0), (a1, b1) = out[0], out[1]
            out = [(a0, b0 - 1), (a1, b1)] + list(out[2:])  # one tile owned by nobody
        return out
    return {"shard_tile_ranges": ranges}


def m_round_truncates():
    def rnd(x):
        x = np.asarray(x, dtype=np.float64)
        b = x.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
        r = b.view(np.float32).astype(np.float64)
        return np.where(np.isfinite(x), r, x)
    return {"round_bf16": rnd}


MUTANTS = [m_logp_sign, m_no_max_shift, m_log_mean_exp, m_target_off_by_one,
           m_target_term_dropped, m_ignored_not_zero, m_bwd_sign, m_bwd_no_onehot,
           m_bwd_unnormalised, m_bwd_no_grad_scale, m_entropy_sign, m_entropy_bwd_no_h,
           m_weight_not_transposed, m_temperature_multiplies, m_bwd_dz_not_scaled,
           m_dweight_last_block_only, m_merge_exponent_sign, m_padding_zero,
           m_shard_ownership_shifted, m_round_truncates]


def test_pins_pass_unmutated():
    assert _first_failure() is None


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__[2:])
def test_planted_mistake_is_caught(mutant, monkeypatch):
    for name, fn in mutant().items():
        monkeypatch.setattr(lo, name, fn)
        if hasattr(oracle, name):
            monkeypatch.setattr(oracle, name, fn)
    caught = _first_failure()
    assert caught is not None, f"no pin fails when the oracle has the slip '{mutant.__name__}'"
