"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws random numbers and lays them out; it holds none of the
log-probability arithmetic.  Both the HIP path and the CPU oracle consume
what it returns, so neither depends on the other for inputs.

Distributions follow the workloads the operator is benchmarked on: logits of
a Qwen3-8B-sized vocabulary (V = 151936) drawn N(0, sigma) in float32 and
cast to bf16 with round-to-nearest-even, uniform targets, a fraction of rows
set to ignore_index, optional +40 spikes (added before the cast), and the
LM-head shapes hidden [N, 4096] x weight [151936, 4096].  N(0, s) means a
standard deviation of s.  "p% of rows" means floor(p * N) rows chosen by a
seeded permutation; spikes and ignored rows are drawn independently.
"""

from __future__ import annotations

import torch

QWEN3_VOCAB = 151936
QWEN3_HIDDEN = 4096
IGNORE_INDEX = -100


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_matrix(rows, cols, std, dtype, seed, device="cpu", spike_rows=None,
                  spike_cols=None, spike=40.0, chunk_rows=1024):
    """[rows, cols] drawn N(0, std) in float32 then cast to `dtype`.

    spike_rows / spike_cols (LongTensors of equal length) add `spike` to one
    float32 entry per listed row before the cast.  Generated in row blocks so
    the float32 staging never exceeds chunk_rows * cols values."""
    device = torch.device(device)
    out = torch.empty((rows, cols), dtype=dtype, device=device)
    g = _gen(seed, device)
    spikes = {}
    if spike_rows is not None:
        for r, c in zip(spike_rows.tolist(), spike_cols.tolist()):
            spikes.setdefault(r, []).append(c)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        blk = torch.randn((r1 - r0, cols), generator=g, device=device,
                          dtype=torch.float32)
        blk.mul_(std)
        for r in range(r0, r1):
            for c in spikes.get(r, ()):
                blk[r - r0, c] += spike
        out[r0:r1].copy_(blk)
        del blk
    return out


def choose_rows(n, frac, seed):
    """floor(frac * n) distinct rows from a seeded permutation (CPU)."""
    k = int(frac * n)
    g = _gen(seed, "cpu")
    return torch.randperm(n, generator=g)[:k]


def uniform_targets(n, v, seed, ignore_rows=None, ignore_index=IGNORE_INDEX,
                    device="cpu"):
    """int64 targets uniform in [0, v); listed rows set to ignore_index."""
    g = _gen(seed, "cpu")
    t = torch.randint(0, v, (n,), generator=g, dtype=torch.int64)
    if ignore_rows is not None and len(ignore_rows):
        t[ignore_rows] = ignore_index
    return t.to(device)


# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------

def tiny_fp32(seed=1001):
    """logits [64, 4096] fp32 ~ N(0, 2); 4 rows ignored; tile width 512."""
    n, v = 64, 4096
    logits = normal_matrix(n, v, 2.0, torch.float32, seed)
    ign = choose_rows(n, 4 / n, seed + 1)
    targets = uniform_targets(n, v, seed + 2, ign)
    return dict(logits=logits, targets=targets, ignore_index=IGNORE_INDEX,
                tile_width=512)


def tiny_v8(seed=1001, n=16):
    """n rows of V = 8 fp32 ~ N(0, 2) (one tile, mostly padding)."""
    logits = normal_matrix(n, 8, 2.0, torch.float32, seed + 10)
    targets = uniform_targets(n, 8, seed + 11)
    return dict(logits=logits, targets=targets, ignore_index=IGNORE_INDEX,
                tile_width=512)


def constant_rows(v, values, dtype=torch.float32):
    """One row per value, every entry equal to that value."""
    return torch.stack([torch.full((v,), float(c), dtype=dtype) for c in values])


def qwen3_fwd(seed=1002, n=4096, v=QWEN3_VOCAB, device="cpu"):
    """Forward workload: bf16 [n, v] ~ N(0, 3); 1% of rows get a +40 spike at
    a uniform column; uniform targets; 5% of rows ignored; tile width 4096."""
    spike_rows = choose_rows(n, 0.01, seed + 1)
    g = _gen(seed + 2, "cpu")
    spike_cols = torch.randint(0, v, (spike_rows.numel(),), generator=g)
    logits = normal_matrix(n, v, 3.0, torch.bfloat16, seed, device,
                           spike_rows, spike_cols)
    ign = choose_rows(n, 0.05, seed + 3)
    targets = uniform_targets(n, v, seed + 4, ign, device=device)
    return dict(logits=logits, targets=targets, ignore_index=IGNORE_INDEX,
                tile_width=4096, spike_rows=spike_rows, spike_cols=spike_cols)


def qwen3_fwd_bwd(seed=1004, n=8192, v=QWEN3_VOCAB, device="cpu"):
    """Forward+backward workload: bf16 [n, v] ~ N(0, 3); 10% of rows ignored;
    upstream gradient g ~ N(0, 1) fp32 [n]; tile width 4096."""
    logits = normal_matrix(n, v, 3.0, torch.bfloat16, seed, device)
    ign = choose_rows(n, 0.10, seed + 1)
    targets = uniform_targets(n, v, seed + 2, ign, device=device)
    grad = normal_matrix(1, n, 1.0, torch.float32, seed + 3, device)[0]
    return dict(logits=logits, targets=targets, grad=grad,
                ignore_index=IGNORE_INDEX, tile_width=4096)


def qwen3_invariance(seed=1003, batch=8, seq=2048, v=QWEN3_VOCAB,
                     max_pad=1024, device="cpu"):
    """Batch-invariance workload: bf16 [batch, seq, v] ~ N(0, 3) with a
    right-padding of uniform length 0..max_pad per sequence, masked by
    ignore_index (the padded logits stay random)."""
    logits = normal_matrix(batch * seq, v, 3.0, torch.bfloat16, seed, device)
    g = _gen(seed + 1, "cpu")
    pads = torch.randint(0, max_pad + 1, (batch,), generator=g)
    targets = uniform_targets(batch * seq, v, seed + 2).view(batch, seq)
    for b in range(batch):
        p = int(pads[b])
        if p:
            targets[b, seq - p:] = IGNORE_INDEX
    return dict(logits=logits.view(batch, seq, v), targets=targets.to(device),
                pads=pads, ignore_index=IGNORE_INDEX, tile_width=4096)


def random_rows(n, v, seed, device="cpu", dtype=torch.bfloat16, std=3.0):
    """Fresh neighbour rows and their uniform targets."""
    logits = normal_matrix(n, v, std, dtype, seed, device)
    targets = uniform_targets(n, v, seed + 1, device=device)
    return logits, targets


def qwen3_linear(seed=1005, n=4096, h=QWEN3_HIDDEN, v=QWEN3_VOCAB,
                 device="cpu", ignore_frac=0.0):
    """Fused LM-head workload: hidden bf16 [n, h] ~ N(0, 1), weight bf16
    [v, h] ~ N(0, 0.02), uniform targets (no ignored rows unless asked)."""
    hidden = normal_matrix(n, h, 1.0, torch.bfloat16, seed, device)
    weight = normal_matrix(v, h, 0.02, torch.bfloat16, seed + 1, device)
    ign = choose_rows(n, ignore_frac, seed + 2) if ignore_frac else None
    targets = uniform_targets(n, v, seed + 3, ign, device=device)
    return dict(hidden=hidden, weight=weight, targets=targets,
                ignore_index=IGNORE_INDEX)


def lattice_linear(seed, n, h, v, device="cpu", ignore_frac=0.0, w_den=1024, w_max=127):
    """LM-head operands on small lattices: hidden entries uniform in {-1, 0,
    1}, weight entries k / w_den with k uniform in [-w_max, w_max] (both
    exact in bf16 for w_max < 256), uniform targets.  Every product and
    partial sum of h @ W^T is then a multiple of 1 / w_den below
    h * w_max / w_den in magnitude (19 bits at h = 4096 with the defaults),
    so any float32 accumulation order gives the exact value, while typical
    values carry more significant bits than bf16 keeps."""
    g = _gen(seed, "cpu")
    hidden = (torch.randint(-1, 2, (n, h), generator=g).to(torch.bfloat16)).to(device)
    k = torch.randint(-w_max, w_max + 1, (v, h), generator=g)
    weight = (k.to(torch.float32) / w_den).to(torch.bfloat16).to(device)
    ign = choose_rows(n, ignore_frac, seed + 2) if ignore_frac else None
    targets = uniform_targets(n, v, seed + 3, ign, device=device)
    return dict(hidden=hidden, weight=weight, targets=targets, ignore_index=IGNORE_INDEX)
