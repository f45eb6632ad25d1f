"""GPU parity of ddtree_accept against the oracle: bit-exact.

Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees",
§4.1: walk with the target's decoding rule (argmax at temperature 0); the
matched path is accepted, the first unmatched target token is the bonus.
Besides the targeted cases, twelve seeded random shapes (requests, block
size, budget, vocabulary, dtype, share of nodes whose target follows a
child) are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_build_amd import api, synth
from gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def _gpu_accept(target_logits, target_ids, tree, L):
    tok = torch.from_numpy(tree["tokens"]).to(DEV)
    B, T = tok.shape
    par = torch.from_numpy(tree["parents"]).to(DEV)
    nn = torch.from_numpy(tree["num_nodes"]).to(DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    acc, accn = torch.empty(B, L, **i32), torch.empty(B, L, **i32)
    alen, bonus, targ = torch.empty(B, **i32), torch.empty(B, **i32), torch.empty(B, T, **i32)
    ws = api.new_workspace(api.ddtree_accept_workspace_size(B, T), DEV)
    tl = None if target_logits is None else target_logits.to(DEV)
    ti = None if target_ids is None else torch.as_tensor(target_ids, dtype=torch.int32).to(DEV)
    api.ddtree_accept(tl, ti, tok, par, nn, L, acc, accn, alen, bonus, targ, ws)
    torch.cuda.synchronize()
    return dict(accepted=acc.cpu().numpy(), accepted_nodes=accn.cpu().numpy(),
                accept_len=alen.cpu().numpy(), bonus=bonus.cpu().numpy(),
                target_argmax=targ.cpu().numpy())


def _same(g, o):
    for k in ("accepted", "accepted_nodes", "accept_len", "bonus", "target_argmax"):
        np.testing.assert_array_equal(g[k], o[k], err_msg=k)


def _planted_logits(tree, V, dtype, seed, follow=0.8):
    """Random target logits, with the top token often set to a child's token."""
    rng = np.random.default_rng(seed)
    B, T = tree["tokens"].shape
    x = torch.from_numpy(rng.standard_normal((B, T, V)).astype(np.float32))
    for b in range(B):
        n = tree["num_nodes"][b]
        for i in range(n):
            kids = [c for c in range(1, n) if tree["parents"][b, c] == i]
            if kids and rng.random() < follow:
                x[b, i, tree["tokens"][b, kids[int(rng.integers(len(kids)))]]] = 9.0
    return x.to(dtype)


@pytest.mark.parametrize("V,dtype", [(64, torch.float32), (1001, torch.bfloat16),
                                     (1001, torch.float32), (32000, torch.bfloat16),
                                     (151936, torch.bfloat16)])
def test_accept_logits_matches_oracle(V, dtype):
    B, L, K, N = 3, 6, 4, 40
    g = torch.Generator().manual_seed(V)
    tree = oracle.build_tree(torch.randn(B, L, V, generator=g) * 2, [0, 1, 2], K, N, 1.0)
    tl = _planted_logits(tree, V, dtype, seed=V)
    tl[0, 3, :] = float("-inf")                     # all -inf row -> token 0
    if dtype == torch.float32:
        tl[1, 2, 5] = float("nan")
    note("accept logits V=%d %s" % (V, dtype))
    g_ = _gpu_accept(tl, None, tree, L)
    o = oracle.accept(tl, None, tree["tokens"], tree["parents"], tree["num_nodes"], L)
    _same(g_, o)
    assert g_["accept_len"].max() >= 2   # the planted paths are followed


def test_accept_ids_full_and_root_miss():
    B, L, V, K, N = 2, 5, 50, 4, 20
    tree = oracle.build_tree(torch.randn(B, L, V) * 2, [0, 1], K, N, 1.0)
    T = N + 1
    ids = np.zeros((B, T), np.int32)
    dep = tree["depths"][0]
    leaf = int(np.argmax(dep))
    path = [leaf]
    while tree["parents"][0, path[-1]] >= 0:
        path.append(int(tree["parents"][0, path[-1]]))
    path = path[::-1]
    for a, b in zip(path[:-1], path[1:]):
        ids[0, a] = tree["tokens"][0, b]
    ids[0, leaf] = 41
    kids = {int(tree["tokens"][1, c]) for c in range(1, T) if tree["parents"][1, c] == 0}
    ids[1, 0] = next(t for t in range(V) if t not in kids)
    note("accept ids")
    g = _gpu_accept(None, ids, tree, L)
    o = oracle.accept(None, ids, tree["tokens"], tree["parents"], tree["num_nodes"], L)
    _same(g, o)
    assert g["accept_len"][0] == dep[leaf] and g["bonus"][0] == 41 and g["accept_len"][1] == 0


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_accept_full_size_workloads(name):
    w = synth.WORKLOADS[name]
    x, _ = synth.drafter_logits(w)
    tree = oracle.build_tree(x, synth.root_tokens(w), w.K, w.N, w.taus[0])
    tl = synth.target_logits(w)
    note("accept workload %s" % name)
    g = _gpu_accept(tl, None, tree, w.L)
    o = oracle.accept(tl, None, tree["tokens"], tree["parents"], tree["num_nodes"], w.L)
    _same(g, o)


def test_accept_optional_outputs_absent():
    """target_argmax and accepted_nodes may be NULL: the walk still runs from
    the per-node target tokens, which then stay in the workgroup."""
    B, L, V, K, N = 4, 7, 3000, 6, 90
    g = torch.Generator().manual_seed(3)
    tree = oracle.build_tree(torch.randn(B, L, V, generator=g) * 2, [0, 1, 2, 3], K, N, 1.0)
    tl = _planted_logits(tree, V, torch.bfloat16, seed=3, follow=0.9)
    o = oracle.accept(tl, None, tree["tokens"], tree["parents"], tree["num_nodes"], L)
    tok = torch.from_numpy(tree["tokens"]).to(DEV)
    par = torch.from_numpy(tree["parents"]).to(DEV)
    nn = torch.from_numpy(tree["num_nodes"]).to(DEV)
    T = tok.shape[1]
    i32 = dict(dtype=torch.int32, device=DEV)
    acc, alen, bonus = torch.empty(B, L, **i32), torch.empty(B, **i32), torch.empty(B, **i32)
    ws = api.new_workspace(api.ddtree_accept_workspace_size(B, T), DEV)
    note("accept without optional outputs")
    api.ddtree_accept(tl.to(DEV), None, tok, par, nn, L, acc, None, alen, bonus, None, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), o["accepted"])
    np.testing.assert_array_equal(alen.cpu().numpy(), o["accept_len"])
    np.testing.assert_array_equal(bonus.cpu().numpy(), o["bonus"])
    assert o["accept_len"].max() >= 2


def _random_accept_case(seed):
    """A seeded shape for the acceptance tests: 1-8 requests, blocks of 1-32
    positions, budgets up to 1,024, vocabularies up to 200,000 (fewer when the
    target logits would pass 1e8 values), bf16 or f32, and target logits whose
    top token follows one child's token at a random share of the nodes."""
    rng = np.random.default_rng(700 + seed)
    B = int(rng.integers(1, 9))
    L = int(rng.integers(1, 33))
    N = int(rng.choice([int(rng.integers(1, 72)), int(rng.integers(72, 300)),
                        int(rng.integers(300, 1025))]))
    V = int(rng.choice([int(rng.integers(2, 300)), int(rng.integers(300, 20000)),
                        int(rng.integers(20000, 200000))]))
    V = max(2, min(V, int(1e8) // (B * (N + 1))))
    K = int(rng.integers(1, min(32, V) + 1))
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    g = torch.Generator().manual_seed(800 + seed)
    roots = [int(r) for r in rng.integers(0, V, size=B)]
    tree = oracle.build_tree(torch.randn(B, L, V, generator=g) * 2, roots, K, N, 1.0)
    T = N + 1
    x = torch.from_numpy(rng.standard_normal((B, T, V)).astype(np.float32))
    follow = float(rng.uniform(0.3, 1.0))
    for b in range(B):
        n = int(tree["num_nodes"][b])
        par = tree["parents"][b, 1:n]
        for i in np.unique(par):
            if rng.random() < follow:
                kids = np.nonzero(par == i)[0] + 1
                x[b, i, int(tree["tokens"][b, kids[int(rng.integers(len(kids)))]])] += 9.0
    return tree, x.to(dtype), L, dict(B=B, L=L, V=V, K=K, N=N, dtype=dtype)


@pytest.mark.parametrize("seed", range(12))
def test_accept_random_shapes(seed):
    tree, tl, L, c = _random_accept_case(seed)
    note("accept random seed=%d %s" % (seed, c))
    g = _gpu_accept(tl, None, tree, L)
    o = oracle.accept(tl, None, tree["tokens"], tree["parents"], tree["num_nodes"], L)
    _same(g, o)
