"""The C-ABI calls (without validate) only enqueue kernels on the caller's
stream, so a HIP graph can capture them: a captured forward + backward and
a captured fused LM-head forward, replayed several times with new inputs
copied in between (and eager work between the replays), give the eager
results bit for bit on every replay."""

import pytest
import torch

import invariant_token_log_amd as itl
import synth
from gpu_helpers import bits, dev

pytestmark = pytest.mark.gpu


def test_graph_replays_streaming_fwd_bwd():
    n, v = 64, synth.QWEN3_VOCAB
    x = torch.empty(n, v, dtype=torch.bfloat16, device=dev())
    t = torch.empty(n, dtype=torch.int64, device=dev())
    g = torch.empty(n, dtype=torch.float32, device=dev())
    x.copy_(synth.normal_matrix(n, v, 3.0, torch.bfloat16, seed=1).to(dev()))
    t.copy_(synth.uniform_targets(n, v, seed=2, ignore_rows=torch.tensor([5])).to(dev()))
    g.copy_(synth.normal_matrix(1, n, 1.0, torch.float32, seed=3)[0].to(dev()))
    # warm up on a side stream (allocator, library load), as graph capture wants
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            logp, lse = itl.logp_fwd(x, t, -100, 4096)
            d = itl.logp_bwd(x, t, lse, g, -100, 4096)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        logp, lse = itl.logp_fwd(x, t, -100, 4096)
        d = itl.logp_bwd(x, t, lse, g, -100, 4096)
    for seed in (11, 12, 13):
        x.copy_(synth.normal_matrix(n, v, 3.0, torch.bfloat16, seed=seed).to(dev()))
        t.copy_(synth.uniform_targets(n, v, seed=seed + 1,
                                      ignore_rows=torch.tensor([seed % n])).to(dev()))
        g.copy_(synth.normal_matrix(1, n, 1.0, torch.float32, seed=seed + 2)[0].to(dev()))
        graph.replay()
        torch.cuda.synchronize()
        ref_logp, ref_lse = itl.logp_fwd(x, t, -100, 4096)
        ref_d = itl.logp_bwd(x, t, ref_lse, g, -100, 4096)
        torch.cuda.synchronize()
        assert torch.equal(bits(logp), bits(ref_logp)), seed
        assert torch.equal(bits(lse), bits(ref_lse)), seed
        assert torch.equal(d.view(torch.int16), ref_d.view(torch.int16)), seed


def test_graph_replays_fused_lm_head():
    n, h, v = 8, 512, 3000
    hid = torch.empty(n, h, dtype=torch.bfloat16, device=dev())
    w = synth.normal_matrix(v, h, 0.02, torch.bfloat16, seed=20).to(dev())
    t = torch.empty(n, dtype=torch.int64, device=dev())
    hid.copy_(synth.normal_matrix(n, h, 1.0, torch.bfloat16, seed=21).to(dev()))
    t.copy_(synth.uniform_targets(n, v, seed=22).to(dev()))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            out = itl.linear_logp_fwd(hid, w, t, return_entropy=True)
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = itl.linear_logp_fwd(hid, w, t, return_entropy=True)
    for seed in (31, 32, 33):
        hid.copy_(synth.normal_matrix(n, h, 1.0, torch.bfloat16, seed=seed).to(dev()))
        t.copy_(synth.uniform_targets(n, v, seed=seed + 1).to(dev()))
        graph.replay()
        torch.cuda.synchronize()
        ref = itl.linear_logp_fwd(hid, w, t, return_entropy=True)
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(bits(a), bits(b)), seed


@pytest.mark.parametrize("prepared", [False, True])
def test_graph_replays_fused_fwd_bwd_256_tile(prepared):
    """N > 128 (the 256-row tile, which first re-lays the hidden rows): a
    captured fused forward + backward, with or without a prepared weight,
    replayed with new hidden rows and targets, gives the eager bits."""
    n, h, v = 300, 128, 1000
    hid = torch.empty(n, h, dtype=torch.bfloat16, device=dev())
    t = torch.empty(n, dtype=torch.int64, device=dev())
    g = synth.normal_matrix(1, n, 1.0, torch.float32, seed=40)[0].to(dev())
    w = synth.normal_matrix(v, h, 0.05, torch.bfloat16, seed=41).to(dev())
    pw = itl.prepare_weight(w) if prepared else None
    hid.copy_(synth.normal_matrix(n, h, 1.0, torch.bfloat16, seed=42).to(dev()))
    t.copy_(synth.uniform_targets(n, v, seed=43).to(dev()))

    def step():
        logp, lse = itl.linear_logp_fwd(hid, w, t, prepared_weight=pw)
        dh, dw = itl.linear_logp_bwd(hid, w, t, lse, g, prepared_weight=pw)
        return logp, lse, dh, dw

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    for seed in (51, 52, 53):
        hid.copy_(synth.normal_matrix(n, h, 1.0, torch.bfloat16, seed=seed).to(dev()))
        t.copy_(synth.uniform_targets(n, v, seed=seed + 1,
                                      ignore_rows=torch.tensor([seed % n])).to(dev()))
        graph.replay()
        torch.cuda.synchronize()
        ref = step()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(bits(a), bits(b)), seed
