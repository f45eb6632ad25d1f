"""ddtree_build_noalloc (the build with the library's static scratch, for
callers that cannot allocate) against ddtree_build with a caller workspace:
bit-identical trees, masks, top-K tables and status words, on two calls in a
row, the second on a smaller input (the static scratch keeps the first
call's contents)."""
import numpy as np
import pytest
import torch

from draft_tree_build_amd import api, synth
from gpu_util import DEV, note

pytestmark = pytest.mark.gpu

OUTS = ("tokens", "parents", "depths", "scores", "num_nodes", "mask", "topk_tokens",
        "topk_logprobs", "status")


def _outputs(B, L, K, N):
    dev = torch.device(DEV)
    T, W = N + 1, (N + 64) // 64
    i32 = dict(dtype=torch.int32, device=dev)
    return dict(tokens=torch.full((B, T), -7, **i32), parents=torch.full((B, T), -7, **i32),
                depths=torch.full((B, T), -7, **i32),
                scores=torch.full((B, T), 7.0, dtype=torch.float32, device=dev),
                num_nodes=torch.full((B,), -7, **i32),
                mask=torch.full((B, T, W), 7, dtype=torch.int64, device=dev),
                topk_tokens=torch.full((B, L, K), -7, **i32),
                topk_logprobs=torch.full((B, L, K), 7.0, dtype=torch.float32, device=dev),
                status=torch.full((B,), -7, **i32))


def _build(x, roots, K, N, tau, noalloc):
    B, L, V = x.shape
    o = _outputs(B, L, K, N)
    args = (x, roots, K, N, tau, o["tokens"], o["parents"], o["depths"], o["scores"],
            o["num_nodes"], o["mask"], o["topk_tokens"], o["topk_logprobs"], o["status"])
    if noalloc:
        api.ddtree_build_noalloc(*args)
    else:
        ws = api.new_workspace(api.ddtree_build_workspace_size(B, L, V, K, N), DEV)
        api.ddtree_build(*args, ws)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in o.items()}


def _same(a, b):
    for k in OUTS:
        assert torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8)), k


def test_build_noalloc_matches_build_two_calls():
    cases = [("B32_L16_V151936_K8_N128_P512-16384", 1.0),   # 0.8 MiB of scratch
             ("L16_V32000_K8_N64_P2048", 0.7)]             # then a smaller input
    for name, tau in cases:
        w = synth.WORKLOADS[name]
        x, _ = synth.drafter_logits(w)
        x, roots = x.to(DEV), synth.root_tokens(w).to(DEV)
        note("noalloc build %s tau=%g" % (name, tau))
        got = _build(x, roots, w.K, w.N, tau, noalloc=True)
        ref = _build(x, roots, w.K, w.N, tau, noalloc=False)
        _same(got, ref)
        assert int(got["num_nodes"].min()) == w.T


def test_build_noalloc_rejects_oversized_scratch():
    """A shape whose scratch exceeds the static buffer is rejected before
    anything is enqueued: the outputs keep their contents."""
    B, L, V, K, N = 256, 16, 151936, 8, 4
    x = torch.zeros(B, L, V, dtype=torch.bfloat16, device=DEV)
    roots = torch.zeros(B, dtype=torch.int32, device=DEV)
    o = _outputs(B, L, K, N)
    with pytest.raises(api.DDTreeError) as e:
        api.ddtree_build_noalloc(x, roots, K, N, 1.0, o["tokens"], o["parents"], o["depths"],
                                 o["scores"], o["num_nodes"], o["mask"], o["topk_tokens"],
                                 o["topk_logprobs"], o["status"])
    assert e.value.code == -5
    torch.cuda.synchronize()
    assert torch.all(o["num_nodes"].cpu() == -7)
