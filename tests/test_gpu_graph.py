"""A round captured in HIP graphs replays identically to eager calls.

The benchmark replays captured graphs of the three ABI calls. Each replay
here is separated by eager work and a synchronisation, and every replay's
outputs are compared with the eager outputs (bitwise).
"""
import numpy as np
import pytest
import torch

from draft_tree_build_amd import api, synth
from gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    w = synth.WORKLOADS["L16_V32000_K8_N64_P2048"]
    x, _ = synth.drafter_logits(w)
    P = synth.prefix_lengths(w)
    offs = synth.kv_offsets(P, w.T)
    q, k, v = synth.qkv(w, P)
    tl = synth.target_logits(w)
    dev = torch.device(DEV)
    x, q, k, v, tl = (t.to(dev) for t in (x, q, k, v, tl))
    roots, P, offs = synth.root_tokens(w).to(dev), P.to(dev), offs.to(dev)
    rnd = api.Round(w.batch, w.L, w.V, w.K, w.N, dev, w.Hq, w.Hkv, w.D, int(w.prefix[1]))
    outs = ("tokens", "parents", "depths", "scores", "num_nodes", "mask", "topk_tokens",
            "topk_logprobs", "out", "accepted", "accept_len", "bonus", "target_argmax")

    def run():
        rnd.build(x, roots, 1.0)
        rnd.verify(q, k, v, offs, P)
        rnd.accept(tl)

    note("graph: eager reference")
    run()
    torch.cuda.synchronize()
    ref = {n: getattr(rnd, n).clone() for n in outs}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for n in outs:
            getattr(rnd, n).fill_(0) if getattr(rnd, n).dtype != torch.float32 else getattr(rnd, n).fill_(float("nan"))
        torch.cuda.synchronize()
        note("graph: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        for n in outs:
            a, b = getattr(rnd, n), ref[n]
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (rep, n)
        _ = (x.float().sum() + 1).item()   # unrelated eager work between replays


def test_graph_replays_sampled_accept_and_commit():
    """Build, verify, sampled acceptance and the in-place KV commit captured in
    one graph: every replay (the caches restored beforehand, outside the
    graph) gives the eager outputs and the eager compacted caches."""
    w = synth.WORKLOADS["L16_V32000_K8_N64_P2048"]
    x, _ = synth.drafter_logits(w)
    P = synth.prefix_lengths(w)
    offs = synth.kv_offsets(P, w.T)
    q, k, v = synth.qkv(w, P)
    tl = synth.target_logits(w)
    dev = torch.device(DEV)
    x, q, k0, v0 = (t.to(dev) for t in (x, q, k, v))
    roots, P, offs = synth.root_tokens(w).to(dev), P.to(dev), offs.to(dev)
    rnd = api.Round(w.batch, w.L, w.V, w.K, w.N, dev, w.Hq, w.Hkv, w.D, int(w.prefix[1]))
    rnd.prepare_commit()
    rnd.build(x, roots, 1.0)
    torch.cuda.synchronize()
    toks, pars, nn = rnd.tokens.cpu(), rnd.parents.cpu(), int(rnd.num_nodes[0])
    seen = set()
    for c in range(1, nn):                       # lead the sampled walk down first children
        p = int(pars[0, c])
        if p not in seen:
            seen.add(p)
            tl[0, p, int(toks[0, c])] = 40.0
    tl = tl.to(dev)
    k, v = k0.clone(), v0.clone()
    outs = ("tokens", "parents", "num_nodes", "mask", "out", "accepted", "accepted_nodes",
            "accept_len", "bonus", "target_argmax", "new_prefix_lens", "next_roots")

    def run():
        rnd.build(x, roots, 1.0)
        rnd.verify(q, k, v, offs, P)
        rnd.accept_sample(tl, 1.0, 1234, 5)
        rnd.commit(k, v, offs, P)

    note("graph sample+commit: eager reference")
    run()
    torch.cuda.synchronize()
    ref = {n: getattr(rnd, n).clone() for n in outs}
    kref, vref = k.clone(), v.clone()
    assert int(ref["accept_len"][0]) >= 2
    assert not torch.equal(kref.view(torch.uint8), k0.view(torch.uint8))   # rows were moved
    k.copy_(k0)
    v.copy_(v0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        k.copy_(k0)
        v.copy_(v0)
        for n in outs:
            getattr(rnd, n).fill_(0)
        torch.cuda.synchronize()
        note("graph sample+commit: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        for n in outs:
            a, b = getattr(rnd, n), ref[n]
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (rep, n)
        assert torch.equal(k.view(torch.uint8), kref.view(torch.uint8)), rep
        assert torch.equal(v.view(torch.uint8), vref.view(torch.uint8)), rep
        _ = (x.float().sum() + 1).item()   # unrelated eager work between replays
