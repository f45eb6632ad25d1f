"""A round captured in a HIP graph: every replay matches the oracle.

The benchmark replays captured graphs of the ABI calls. Each replay here is
separated by eager work and a synchronisation (outputs cleared before it),
and every replay's outputs are compared with the oracle directly: the tree,
its mask, the top-K tables, the accepted path, the bonus and the per-node
target tokens bit for bit, the KV compaction byte for byte, and the
attention rows within the bf16 tolerance (1e-3 + 2e-2 |ref|). Pages:
"Accelerating Speculative Decoding with Block Diffusion Draft Trees", §4.1,
§4.3, App. A, App. B.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_build_amd import api, synth
from gpu_util import DEV, check_attn, note

pytestmark = pytest.mark.gpu

W_NAME = "L16_V32000_K8_N64_P2048"


def _inputs():
    w = synth.WORKLOADS[W_NAME]
    x, _ = synth.drafter_logits(w)
    P = synth.prefix_lengths(w)
    offs = synth.kv_offsets(P, w.T)
    q, k, v = synth.qkv(w, P)
    tl = synth.target_logits(w)
    return w, x, synth.root_tokens(w), P, offs, q, k, v, tl


def _capture(run):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def _check_tree(rnd, o):
    np.testing.assert_array_equal(rnd.num_nodes.cpu().numpy(), o["num_nodes"])
    for n in ("tokens", "parents", "depths"):
        np.testing.assert_array_equal(getattr(rnd, n).cpu().numpy(), o[n], err_msg=n)
    np.testing.assert_array_equal(rnd.scores.cpu().numpy().view(np.uint32),
                                  o["scores"].view(np.uint32))
    np.testing.assert_array_equal(rnd.mask.cpu().numpy().view(np.uint64), o["mask"])
    np.testing.assert_array_equal(rnd.topk_tokens.cpu().numpy(), o["topk_tok"])
    np.testing.assert_array_equal(rnd.topk_logprobs.cpu().numpy().view(np.uint32),
                                  o["topk_lp"].view(np.uint32))
    np.testing.assert_array_equal(rnd.status.cpu().numpy(), o["status"])


def _check_accept(rnd, a, tgt_key):
    for n in ("accepted", "accepted_nodes", "accept_len", "bonus"):
        np.testing.assert_array_equal(getattr(rnd, n).cpu().numpy(), a[n], err_msg=n)
    np.testing.assert_array_equal(rnd.target_argmax.cpu().numpy(), a[tgt_key])


def test_graph_replays_match_oracle():
    w, x, roots, P, offs, q, k, v, tl = _inputs()
    o = oracle.build_tree(x, roots, w.K, w.N, 1.0)
    a = oracle.accept(tl, None, o["tokens"], o["parents"], o["num_nodes"], w.L)
    sel = [(0, i, h) for i in range(w.T) for h in range(w.Hq)]
    with oracle.threads(oracle.host_cores()):
        ref_attn = oracle.attn_rows(q, k, v, offs, P, o["num_nodes"], o["mask"], w.T, w.Hq,
                                    w.Hkv, w.D, 1.0 / np.sqrt(w.D), sel)
    dev = torch.device(DEV)
    xd, qd, kd, vd, tld = (t.to(dev) for t in (x, q, k, v, tl))
    rootsd, Pd, offsd = roots.to(dev), P.to(dev), offs.to(dev)
    rnd = api.Round(w.batch, w.L, w.V, w.K, w.N, dev, w.Hq, w.Hkv, w.D, int(w.prefix[1]))

    def run():
        rnd.build(xd, rootsd, 1.0)
        rnd.verify(qd, kd, vd, offsd, Pd)
        rnd.accept(tld)

    note("graph: eager warm-up")
    run()
    torch.cuda.synchronize()
    g = _capture(run)
    outs = ("tokens", "parents", "depths", "scores", "num_nodes", "mask", "topk_tokens",
            "topk_logprobs", "status", "out", "accepted", "accepted_nodes", "accept_len",
            "bonus", "target_argmax")
    for rep in range(4):
        for n in outs:
            t = getattr(rnd, n)
            t.fill_(float("nan") if t.is_floating_point() else -9)
        torch.cuda.synchronize()
        note("graph: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        _check_tree(rnd, o)
        check_attn(rnd.out.cpu(), ref_attn, sel, torch.bfloat16)
        _check_accept(rnd, a, "target_argmax")
        _ = (xd.float().sum() + 1).item()   # unrelated eager work between replays


def test_graph_replays_sampled_accept_and_commit():
    """Build, verify, sampled acceptance and the in-place KV commit captured in
    one graph: every replay (the caches restored beforehand, outside the
    graph) gives the oracle's tree, sampled path, new prefix lengths, next
    roots and compacted caches."""
    w, x, roots, P, offs, q, k0, v0, tl = _inputs()
    o = oracle.build_tree(x, roots, w.K, w.N, 1.0)
    seen = set()
    for c in range(1, int(o["num_nodes"][0])):     # lead the sampled walk down first children
        p = int(o["parents"][0, c])
        if p not in seen:
            seen.add(p)
            tl[0, p, int(o["tokens"][0, c])] = 40.0
    seed, offset = 1234, 5
    a = oracle.accept_sample(tl, o["tokens"], o["parents"], o["num_nodes"], w.L, 1.0, seed, offset)
    assert int(a["accept_len"][0]) >= 2
    c = oracle.commit_kv(k0, v0, offs, P, a["accept_len"], a["accepted_nodes"], a["bonus"], w.T)
    sel = [(0, i, h) for i in range(w.T) for h in range(w.Hq)]
    with oracle.threads(oracle.host_cores()):
        ref_attn = oracle.attn_rows(q, k0, v0, offs, P, o["num_nodes"], o["mask"], w.T, w.Hq,
                                    w.Hkv, w.D, 1.0 / np.sqrt(w.D), sel)
    dev = torch.device(DEV)
    xd, qd, tld = (t.to(dev) for t in (x, q, tl))
    k0d, v0d = k0.to(dev), v0.to(dev)
    k, v = k0d.clone(), v0d.clone()
    rootsd, Pd, offsd = roots.to(dev), P.to(dev), offs.to(dev)
    rnd = api.Round(w.batch, w.L, w.V, w.K, w.N, dev, w.Hq, w.Hkv, w.D, int(w.prefix[1]))
    rnd.prepare_commit()

    def run():
        rnd.build(xd, rootsd, 1.0)
        rnd.verify(qd, k, v, offsd, Pd)
        rnd.accept_sample(tld, 1.0, seed, offset)
        rnd.commit(k, v, offsd, Pd)

    note("graph sample+commit: eager warm-up")
    run()
    torch.cuda.synchronize()
    k.copy_(k0d)
    v.copy_(v0d)
    g = _capture(run)
    outs = ("tokens", "parents", "num_nodes", "mask", "out", "accepted", "accepted_nodes",
            "accept_len", "bonus", "target_argmax", "new_prefix_lens", "next_roots")
    for rep in range(4):
        k.copy_(k0d)
        v.copy_(v0d)
        for n in outs:
            t = getattr(rnd, n)
            t.fill_(float("nan") if t.is_floating_point() else -9)
        torch.cuda.synchronize()
        note("graph sample+commit: replay %d" % rep)
        g.replay()
        torch.cuda.synchronize()
        _check_tree(rnd, o)
        check_attn(rnd.out.cpu(), ref_attn, sel, torch.bfloat16)
        _check_accept(rnd, a, "target_tokens")
        np.testing.assert_array_equal(rnd.new_prefix_lens.cpu().numpy(), c["new_prefix_lens"])
        np.testing.assert_array_equal(rnd.next_roots.cpu().numpy(), c["next_roots"])
        np.testing.assert_array_equal(oracle.as_raw(k.cpu())[0], c["k"])
        np.testing.assert_array_equal(oracle.as_raw(v.cpu())[0], c["v"])
        _ = (xd.float().sum() + 1).item()   # unrelated eager work between replays
