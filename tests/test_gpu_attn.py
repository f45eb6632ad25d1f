"""GPU parity of ddtree_verify_attn against the oracle's fp64 tree attention.

Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees",
Abstract / §4.1 (one verify pass, ancestor-only mask), App. B. Tolerance:
|gpu - ref| <= 1e-3 + 2e-2 |ref| for bf16 and 1e-5 + 1e-5 |ref| for f32.
Small shapes compare every output row (ragged prefixes straddling key tiles,
trees with padding rows, GQA group sizes 1/4/8, row tiles with a ragged
tail, the split-KV path with requests of different lengths and with fewer
(request, kv-head) pairs than XCDs); the full-size workloads compare sampled rows in
the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_build_amd import api, synth
from gpu_util import DEV, check_attn, note

pytestmark = pytest.mark.gpu


def _tree(B, L, V, K, N, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, L, V, generator=g) * 2
    return oracle.build_tree(x, list(range(B)), K, N, 1.0)


def _run(q, k, v, P, tree, T, max_prefix=None):
    B, _, Hq, D = q.shape
    offs = synth.kv_offsets(torch.as_tensor(P, dtype=torch.int32), T)
    mp = int(max(P)) if max_prefix is None else max_prefix
    code = 0 if q.dtype == torch.bfloat16 else 1
    ws = api.new_workspace(api.ddtree_verify_workspace_size(code, B, T, Hq, k.shape[1], D, mp), DEV)
    out = torch.full_like(q, 7.0, device=DEV)   # every row must be written
    api.ddtree_verify_attn(q.to(DEV), k.to(DEV), v.to(DEV), offs.to(DEV),
                           torch.as_tensor(P, dtype=torch.int32).to(DEV),
                           torch.from_numpy(tree["num_nodes"]).to(DEV),
                           torch.from_numpy(tree["mask"].view(np.int64)).to(DEV), mp, out, ws)
    torch.cuda.synchronize()
    return out.cpu(), offs


def _ref(q, k, v, offs, P, tree, T, sel):
    Hq, Hkv, D = q.shape[2], k.shape[1], q.shape[3]
    return oracle.attn_rows(q, k, v, offs, P, tree["num_nodes"], tree["mask"], T, Hq, Hkv, D,
                            1.0 / np.sqrt(D), sel)


SMALL = [
    # B, L, V, K, N, Hq, Hkv, prefix lengths
    (3, 4, 30, 3, 8, 8, 2, [0, 65, 130]),
    (1, 6, 40, 4, 64, 4, 4, [63]),
    (2, 8, 50, 5, 100, 32, 8, [64, 1]),
    (2, 2, 20, 2, 20, 8, 1, [200, 7]),          # budget above the restricted set: padding rows
    (1, 16, 80, 8, 64, 32, 8, [2048]),          # split-KV path
    (1, 5, 60, 6, 200, 64, 8, [900]),           # g = 8, many row tiles
    (2, 6, 60, 6, 300, 32, 8, [3000, 1500]),    # split, many row tiles, ragged last row tile
    (3, 6, 60, 6, 100, 32, 8, [700, 3000, 1500]),  # split, requests taken longest first
    (2, 6, 60, 6, 100, 32, 8, [1500, 1500]),    # split, equal lengths (ties by index)
    (1, 16, 80, 8, 64, 32, 4, [4000]),          # 4 (request, kv-head) pairs: splits cut into units
    (2, 4, 40, 4, 40, 16, 2, [2500, 5000]),     # 4 pairs, ragged, longer request second
]


@pytest.mark.parametrize("B,L,V,K,N,Hq,Hkv,P", SMALL)
def test_attn_bf16_all_rows(B, L, V, K, N, Hq, Hkv, P):
    T, D = N + 1, 128
    tree = _tree(B, L, V, K, N, seed=N + Hq)
    g = torch.Generator().manual_seed(B * 1000 + N)
    total = sum(P) + B * T
    q = torch.randn(B, T, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(total, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(total, Hkv, D, generator=g).to(torch.bfloat16)
    note("attn bf16 B=%d T=%d Hq=%d Hkv=%d P=%s" % (B, T, Hq, Hkv, P))
    out, offs = _run(q, k, v, P, tree, T)
    sel = [(b, i, h) for b in range(B) for i in range(T) for h in range(Hq)]
    ref = _ref(q, k, v, offs, P, tree, T, sel)
    check_attn(out, ref, sel, torch.bfloat16)
    for b in range(B):
        assert torch.all(out[b, tree["num_nodes"][b]:] == 0)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_attn_f32_all_rows(D):
    B, L, V, K, N, Hq, Hkv, P = 2, 4, 30, 4, 8, 4, 2, [16, 3]
    T = N + 1
    tree = _tree(B, L, V, K, N, seed=D)
    g = torch.Generator().manual_seed(D)
    total = sum(P) + B * T
    q = torch.randn(B, T, Hq, D, generator=g)
    k = torch.randn(total, Hkv, D, generator=g)
    v = torch.randn(total, Hkv, D, generator=g)
    note("attn f32 D=%d" % D)
    out, offs = _run(q, k, v, P, tree, T)
    sel = [(b, i, h) for b in range(B) for i in range(T) for h in range(Hq)]
    check_attn(out, _ref(q, k, v, offs, P, tree, T, sel), sel, torch.float32)


def test_attn_repeatable_split_counters():
    """Two split-KV calls on one workspace give identical bits (partials rewritten)."""
    B, L, V, K, N, Hq, Hkv, P = 1, 16, 80, 8, 64, 32, 8, [3000]
    T, D = N + 1, 128
    tree = _tree(B, L, V, K, N, seed=1)
    g = torch.Generator().manual_seed(2)
    total = sum(P) + B * T
    q = torch.randn(B, T, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(total, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(total, Hkv, D, generator=g).to(torch.bfloat16)
    note("attn split twice")
    a, _ = _run(q, k, v, P, tree, T)
    b, _ = _run(q, k, v, P, tree, T)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_attn_full_size_workloads_sampled(name):
    w = synth.WORKLOADS[name]
    x, _ = synth.drafter_logits(w)
    roots = synth.root_tokens(w)
    tree = oracle.build_tree(x, roots, w.K, w.N, w.taus[0])
    P = synth.prefix_lengths(w)
    q, k, v = synth.qkv(w, P)
    note("attn workload %s rows=%d" % (name, k.shape[0]))
    out, offs = _run(q, k, v, P.numpy(), tree, w.T, max_prefix=w.prefix[1])
    rng = np.random.default_rng(0)
    nsamp = 4096 if w.prefix[1] <= 2048 else 384
    sel = [(int(rng.integers(w.batch)), int(rng.integers(w.T)), int(rng.integers(w.Hq)))
           for _ in range(nsamp)]
    sel += [(b, int(tree["num_nodes"][b]) - 1, w.Hq - 1) for b in range(w.batch)]
    ref = _ref(q, k, v, offs, P.numpy(), tree, w.T, sel)
    check_attn(out, ref, sel, q.dtype)
