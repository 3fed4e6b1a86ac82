"""Plain, slow CPU oracle for the batch-invariant selected-token log-probability.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constants).

Everything here is numpy in float64.  Inputs arrive as numpy arrays of float32
or float64 (a bf16 tensor is widened to float32 by the caller, which is exact).

Sources (page title -- section):

* "Batch-Invariant LogP" -- opening definition: the selected log-probability of
  a row is the logit at the row's target id minus the log-sum-exp of the whole
  row.
* "Batch-Invariant LogP" -- Reference Semantics: rows are flattened to [N, V],
  the log-softmax of the float row is gathered at the target; a row whose
  target equals ignore_index outputs 0 and gets a zero gradient; any other
  target outside [0, V) is invalid (target -1 is invalid unless ignore_index
  is -1).
* "Batch-Invariant LogP" -- Tensor Parallel: the padded vocabulary is cut into
  fixed tiles, each tile gives a (max, sumexp) pair, the pairs are merged in
  one fixed order as LSE = M + log(sum_t s_t * exp(m_t - M)) with M the
  largest tile max, and the target logit is copied from its owner.
* "Batch-Invariant LogP" -- Batch-Invariance: the backward writes
  g * (onehot - softmax) per row tile from the saved per-row LSE.
* "Batch-Invariant LogP" -- VIME CP=2 runtime provider: full-vocabulary
  entropy is returned on request, merged in the same fixed order as the LSE.
* "[RFC][ROCm] ..." -- Workstream 3, proposed operator: temperature,
  return_entropy and return_logits options of the fused LM head; temperature
  is applied at one contract-defined point (here: the logits are divided by
  it before any statistic).
* "[RFC][ROCm] End-to-end optimization of bitwise VIME R/R beyond native P/P"
  -- Workstream 3 (fused ROCm LM-head and linear logp): the logits are the
  product of the hidden states with the LM-head weight, and the same
  statistics are taken over them without storing them; the backward may
  recompute the fixed logit tiles from the saved LSE.
* "[RFC][ROCm] ..." -- Contract-versioned arithmetic change (the FP32/BF16
  rounding points belong to the contract) and Workstream 1, item 4 (a fused
  epilogue rounds to BF16 explicitly before the next step sees the value):
  the bf16-rounded-logits variant rounds z to bf16 (round to nearest, ties to
  even) before any statistic, as an unfused bf16 LM head would store it.

Parity pins live in tests/test_oracle_pins.py; every function below is pinned
there by closed forms, brute force, a library routine or an invariant.
"""

from __future__ import annotations

import numpy as np

ROW_CHUNK = 256  # rows per block, only to bound host memory


class InvalidTargetError(ValueError):
    """An active row's target lies outside [0, V)."""


def _as_2d(logits):
    x = np.asarray(logits)
    if x.ndim < 1:
        raise ValueError("logits need a vocabulary dimension")
    v = x.shape[-1]
    return x.reshape(-1, v)


def _active_mask(targets, ignore_index, v):
    """Row gate of "Batch-Invariant LogP" -- Reference Semantics.

    Returns (active, t) where active[r] is True for rows that are not
    ignore_index.  Raises InvalidTargetError for an active target outside
    [0, v)."""
    t = np.asarray(targets, dtype=np.int64).reshape(-1)
    active = t != int(ignore_index)
    bad = active & ((t < 0) | (t >= v))
    if np.any(bad):
        r = int(np.flatnonzero(bad)[0])
        raise InvalidTargetError(f"row {r}: target {int(t[r])} not in [0, {v})")
    return active, t


def logp_fwd(logits, targets, ignore_index=-100):
    """Selected-token log-probability and row LSE, in float64.

    Definition ("Batch-Invariant LogP" -- opening definition and Reference
    Semantics), per row r with target t:
        M   = max_j x[r, j]
        S   = sum_j exp(x[r, j] - M)
        lse = M + log(S)
        logp = x[r, t] - lse
    Ignored rows give logp = 0 and lse = 0 (the page fixes the former; the
    latter is this oracle's reading, the lse of an ignored row being
    unspecified).

    Returns (logp [N], lse [N]) as float64 arrays over the flattened rows.
    """
    x2 = _as_2d(logits)
    n, v = x2.shape
    active, t = _active_mask(targets, ignore_index, v)
    if t.shape[0] != n:
        raise ValueError("targets must have one entry per logits row")
    logp = np.zeros(n, dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    for r0 in range(0, n, ROW_CHUNK):
        r1 = min(n, r0 + ROW_CHUNK)
        rows = np.flatnonzero(active[r0:r1]) + r0
        if rows.size == 0:
            continue
        x = x2[rows].astype(np.float64)
        m = x.max(axis=1)
        s = np.exp(x - m[:, None]).sum(axis=1)
        row_lse = m + np.log(s)
        lse[rows] = row_lse
        logp[rows] = x[np.arange(rows.size), t[rows]] - row_lse
    return logp, lse


def logp_bwd(logits, targets, grad_logp, ignore_index=-100, lse=None):
    """Gradient of the selected log-probability with respect to the logits.

    "Batch-Invariant LogP" -- Batch-Invariance / Reference Semantics:
        d[r, j] = g[r] * ([j == t_r] - exp(x[r, j] - lse[r]))
    with lse the forward's float64 row LSE (recomputed here when not given),
    and d[r, :] = 0 for ignored rows.  Returns float64 [N, V].
    Callers that face large N should pass row slices (the [N, V] float64
    result is 8 bytes per logit).
    """
    x2 = _as_2d(logits)
    n, v = x2.shape
    active, t = _active_mask(targets, ignore_index, v)
    g = np.asarray(grad_logp, dtype=np.float64).reshape(-1)
    if g.shape[0] != n:
        raise ValueError("grad_logp must have one entry per logits row")
    if lse is None:
        _, lse = logp_fwd(x2, t, ignore_index)
    lse = np.asarray(lse, dtype=np.float64).reshape(-1)
    d = np.zeros((n, v), dtype=np.float64)
    rows = np.flatnonzero(active)
    for c0 in range(0, rows.size, ROW_CHUNK):
        rr = rows[c0:c0 + ROW_CHUNK]
        x = x2[rr].astype(np.float64)
        p = np.exp(x - lse[rr][:, None])
        onehot = np.zeros_like(p)
        onehot[np.arange(rr.size), t[rr]] = 1.0
        d[rr] = g[rr][:, None] * (onehot - p)
    return d


def entropy(logits, targets, ignore_index=-100):
    """Full-vocabulary entropy of each row's softmax, in float64.

    H = -sum_j p_j log p_j with p_j = exp(x_j - lse) ("Batch-Invariant
    LogP", VIME CP=2 runtime provider: entropy over the whole vocabulary).
    Ignored rows give 0 (reading: like their logp).  Returns H [N]."""
    x2 = _as_2d(logits)
    n, v = x2.shape
    active, t = _active_mask(targets, ignore_index, v)
    ent = np.zeros(n, dtype=np.float64)
    _, lse = logp_fwd(x2, t, ignore_index)
    for r0 in range(0, n, ROW_CHUNK):
        r1 = min(n, r0 + ROW_CHUNK)
        rows = np.flatnonzero(active[r0:r1]) + r0
        if rows.size == 0:
            continue
        logp_all = x2[rows].astype(np.float64) - lse[rows][:, None]
        ent[rows] = -(np.exp(logp_all) * logp_all).sum(axis=1)
    return ent


def entropy_bwd(logits, targets, grad_entropy, ignore_index=-100):
    """Gradient of sum_r gH_r * H_r with respect to the logits, in float64:
    dH/dx_j = -p_j (log p_j + H).  Ignored rows get 0.  Returns [N, V]."""
    x2 = _as_2d(logits)
    n, v = x2.shape
    active, t = _active_mask(targets, ignore_index, v)
    gh = np.asarray(grad_entropy, dtype=np.float64).reshape(-1)
    _, lse = logp_fwd(x2, t, ignore_index)
    ent = entropy(x2, t, ignore_index)
    d = np.zeros((n, v), dtype=np.float64)
    rows = np.flatnonzero(active)
    for c0 in range(0, rows.size, ROW_CHUNK):
        rr = rows[c0:c0 + ROW_CHUNK]
        logp_all = x2[rr].astype(np.float64) - lse[rr][:, None]
        p = np.exp(logp_all)
        d[rr] = -gh[rr][:, None] * p * (logp_all + ent[rr][:, None])
    return d


def linear_logits(hidden, weight):
    """Logits of the LM head: z = h @ W^T in float64.

    "[RFC][ROCm] ..." -- Workstream 3: the fused operator multiplies the
    hidden states [N, H] by the vocabulary-major LM-head weight [V, H].
    Products of bf16 values are exact in float64 and an H-term float64 sum
    has relative error near 1e-16, so z is exact for every purpose here."""
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    if h.ndim != 2 or w.ndim != 2 or h.shape[1] != w.shape[1]:
        raise ValueError("hidden [N,H] and weight [V,H] must share H")
    return h @ w.T


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even, and
    return them as float64.

    bfloat16 keeps 8 significant bits and the float32 exponent range: inside
    a binade [2^(e-1), 2^e) its values are the multiples of 2^(e-8); below
    the smallest normal 2^-126 the spacing stays 2^-133; magnitudes from
    (2 - 2^-8) * 2^127 up round to infinity.  Written from that definition
    (frexp gives the binade, rint rounds half to even); NaN and infinities
    pass through."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    r = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def _lm_logits(h, w, temperature, round_logits):
    """x = z / T with z = h @ W^T, rounded to bf16 first in the variant."""
    z = linear_logits(h, w)
    if round_logits:
        z = round_bf16(z)
    return z / float(temperature)


def linear_logp_fwd(hidden, weight, targets, ignore_index=-100, temperature=1.0,
                    round_logits=False):
    """Fused LM-head + selected log-probability: logp_fwd(h @ W^T / T).

    "[RFC][ROCm] ..." -- Workstream 3.  The fused kernel never stores z; the
    oracle does, a row block at a time.  The temperature T divides the logits
    before any statistic (the proposed operator's temperature option); with
    round_logits, z is rounded to bf16 before that (the variant contract).
    Returns (logp [N], lse [N]) of the scaled logits."""
    h = np.asarray(hidden)
    n = h.shape[0]
    t = np.asarray(targets, dtype=np.int64).reshape(-1)
    logp = np.zeros(n, dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    for r0 in range(0, n, ROW_CHUNK):
        r1 = min(n, r0 + ROW_CHUNK)
        z = _lm_logits(h[r0:r1], weight, temperature, round_logits)
        logp[r0:r1], lse[r0:r1] = logp_fwd(z, t[r0:r1], ignore_index)
    return logp, lse


def linear_entropy(hidden, weight, targets, ignore_index=-100, temperature=1.0,
                   round_logits=False):
    """Entropy of the fused LM head's softmax over h @ W^T / T, per row."""
    h = np.asarray(hidden)
    n = h.shape[0]
    t = np.asarray(targets, dtype=np.int64).reshape(-1)
    ent = np.zeros(n, dtype=np.float64)
    for r0 in range(0, n, ROW_CHUNK):
        r1 = min(n, r0 + ROW_CHUNK)
        z = _lm_logits(h[r0:r1], weight, temperature, round_logits)
        ent[r0:r1] = entropy(z, t[r0:r1], ignore_index)
    return ent


def linear_logp_bwd(hidden, weight, targets, grad_logp, ignore_index=-100, lse=None,
                    need_dweight=True, temperature=1.0, grad_entropy=None, round_logits=False):
    """Gradients of sum_r (g_r logp_r + gH_r H_r) of the fused LM head, in
    float64.

    "[RFC][ROCm] ..." -- Workstream 3 (the backward recomputes the logit
    tiles from the saved LSE) and "Batch-Invariant LogP" -- Batch-Invariance
    (the logit gradient is g * (onehot - softmax), zero on ignored rows):
        x  = h @ W^T / T,  p = exp(x - lse)
        dx = g * (onehot(t) - p) - gH * p * (log p + H)   (rows with t == ignore: 0)
        dz = dx / T,   dh = dz @ W,   dW = dz^T @ h
    lse is the float64 row LSE of x (recomputed when not given); the entropy
    term is present only when grad_entropy is given.  Rows are processed in
    blocks; dW sums the blocks in ascending row order.
    Returns (dh [N, H], dW [V, H]) as float64 (dW is None when not needed)."""
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    n = h.shape[0]
    t = np.asarray(targets, dtype=np.int64).reshape(-1)
    g = np.asarray(grad_logp, dtype=np.float64).reshape(-1)
    if t.shape[0] != n or g.shape[0] != n:
        raise ValueError("targets and grad_logp need one entry per row")
    dh = np.zeros_like(h)
    dw = np.zeros_like(w) if need_dweight else None
    for r0 in range(0, n, ROW_CHUNK):
        r1 = min(n, r0 + ROW_CHUNK)
        x = _lm_logits(h[r0:r1], w, temperature, round_logits)
        row_lse = None if lse is None else np.asarray(lse, dtype=np.float64).reshape(-1)[r0:r1]
        dx = logp_bwd(x, t[r0:r1], g[r0:r1], ignore_index, lse=row_lse)
        if grad_entropy is not None:
            gh = np.asarray(grad_entropy, dtype=np.float64).reshape(-1)[r0:r1]
            dx = dx + entropy_bwd(x, t[r0:r1], gh, ignore_index)
        dz = dx / float(temperature)
        dh[r0:r1] = dz @ w
        if need_dweight:
            dw += dz.T @ h[r0:r1]
    return dh, dw


def linear_logp_bwd_weight_rows(hidden, weight, targets, grad_logp, vocab_rows,
                                ignore_index=-100, lse=None, temperature=1.0,
                                grad_entropy=None, ent=None, round_logits=False):
    """Rows `vocab_rows` of dW from linear_logp_bwd, without forming the other
    vocabulary rows: dW[j] = sum_r dz[r, j] h[r] over active rows, with
    x[:, j] = h W[j]^T / T, p = exp(x - lse) and
    dz[r, j] = (g_r ([t_r == j] - p) - gH_r p (x - lse + H_r)) / T.
    lse and H (float64 [N]) are full-row statistics; they are recomputed from
    all of W when not given (the expensive part).
    Returns float64 [len(vocab_rows), H]."""
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    t = np.asarray(targets, dtype=np.int64).reshape(-1)
    g = np.asarray(grad_logp, dtype=np.float64).reshape(-1)
    active, _ = _active_mask(t, ignore_index, w.shape[0])
    if lse is None:
        _, lse = linear_logp_fwd(h, w, t, ignore_index, temperature, round_logits)
    lse = np.asarray(lse, dtype=np.float64).reshape(-1)
    cols = np.asarray(vocab_rows, dtype=np.int64).reshape(-1)
    x = _lm_logits(h, w[cols], temperature, round_logits)   # [N, J]
    p = np.exp(x - lse[:, None])
    onehot = (t[:, None] == cols[None, :]).astype(np.float64)
    dx = g[:, None] * (onehot - p)
    if grad_entropy is not None:
        if ent is None:
            ent = linear_entropy(h, w, t, ignore_index, temperature, round_logits)
        gh = np.asarray(grad_entropy, dtype=np.float64).reshape(-1)
        dx = dx - gh[:, None] * p * ((x - lse[:, None]) + np.asarray(ent)[:, None])
    dx[~active] = 0.0
    return (dx / float(temperature)).T @ h


# ---------------------------------------------------------------------------
# Tiled construction ("Batch-Invariant LogP" -- Tensor Parallel), written from
# the page's steps.  Diagnostic: it pins the merge identity and the tile /
# shard bookkeeping; it is not used for bit parity with the GPU.
# ---------------------------------------------------------------------------

def num_tiles(v, tile_width):
    """Number of fixed vocabulary tiles: ceil(V / W)."""
    if v < 1 or tile_width < 1:
        raise ValueError("need V >= 1 and W >= 1")
    return -(-v // tile_width)


def shard_tile_ranges(v, tile_width, num_shards):
    """Tiles owned by each of S emulated vocabulary shards.

    Reading of the Tensor Parallel section for shards whose nominal column
    ranges [s*V/S, (s+1)*V/S) are not tile-aligned: there is one global tile
    grid, and shard s owns the tiles whose first column lies in its nominal
    range, i.e. tiles [ceil(s*(V/S)/W), ceil((s+1)*(V/S)/W)).  Every tile then
    has exactly one owner and is reduced whole, on any shard count.
    Returns a list of (first_tile, end_tile) pairs."""
    if num_shards < 1 or v % num_shards:
        raise ValueError("num_shards must divide V")
    per = v // num_shards
    out = []
    for s in range(num_shards):
        lo = -(-(s * per) // tile_width)
        hi = -(-((s + 1) * per) // tile_width)
        out.append((lo, hi))
    return out


def tile_partials(x_row, tile_width, dtype=np.float64):
    """(max, sumexp) of each fixed tile of one row.

    Tensor Parallel, step 2: tile k covers global columns [kW, (k+1)W); the
    padded columns (>= V) hold -inf and add nothing.  m_k is the tile max and
    s_k = sum over the tile of exp(x - m_k), in the given precision.
    Returns (m [T], s [T])."""
    x = np.asarray(x_row, dtype=dtype).reshape(-1)
    v = x.shape[0]
    t_count = num_tiles(v, tile_width)
    padded = np.full(t_count * tile_width, -np.inf, dtype=dtype)
    padded[:v] = x
    tiles = padded.reshape(t_count, tile_width)
    m = tiles.max(axis=1)
    s = np.zeros(t_count, dtype=dtype)
    for k in range(t_count):
        if np.isneginf(m[k]):
            continue
        s[k] = np.exp(tiles[k] - m[k]).sum(dtype=dtype)
    return m, s


def merge_partials(m, s, dtype=np.float64):
    """Fixed-order merge of the Tensor Parallel section, step 4.

    M = max_k m_k, then acc = sum over k = 0..T-1 (ascending) of
    s_k * exp(m_k - M), tiles with m_k = -inf skipped, and
    LSE = M + log(acc)."""
    m = np.asarray(m, dtype=dtype)
    s = np.asarray(s, dtype=dtype)
    big_m = m.max()
    acc = dtype(0.0)
    for k in range(m.shape[0]):
        if np.isneginf(m[k]):
            continue
        acc = dtype(acc + s[k] * np.exp(dtype(m[k] - big_m)))
    return dtype(big_m + np.log(acc))


def tiled_logp_fwd(logits, targets, ignore_index, tile_width, num_shards=1,
                   dtype=np.float64):
    """The Tensor Parallel construction over S emulated shards.

    Each shard writes the partials of the tiles it owns into one [N, T]
    table (the byte-only all-gather), the owner of the target's tile copies
    the target logit, and one fixed-order merge gives LSE and
    logp = target_logit - LSE (steps 1-6).  Returns (logp, lse) in float64,
    computed in `dtype`."""
    x2 = _as_2d(logits)
    n, v = x2.shape
    active, t = _active_mask(targets, ignore_index, v)
    t_count = num_tiles(v, tile_width)
    ranges = shard_tile_ranges(v, tile_width, num_shards)
    logp = np.zeros(n, dtype=np.float64)
    lse = np.zeros(n, dtype=np.float64)
    for r in np.flatnonzero(active):
        m_all = np.full(t_count, -np.inf, dtype=dtype)
        s_all = np.zeros(t_count, dtype=dtype)
        target_logit = None
        m_row, s_row = tile_partials(x2[r], tile_width, dtype)
        for lo, hi in ranges:
            m_all[lo:hi] = m_row[lo:hi]
            s_all[lo:hi] = s_row[lo:hi]
            if lo * tile_width <= t[r] < hi * tile_width:
                target_logit = dtype(x2[r, t[r]])
        row_lse = merge_partials(m_all, s_all, dtype)
        lse[r] = float(row_lse)
        logp[r] = float(dtype(target_logit - row_lse))
    return logp, lse

