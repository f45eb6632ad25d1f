"""GPU parity of ddtree_accept_sample against the oracle: bit-exact.

Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees",
§4.1: the tree is walked with the target's own decoding rule; at temperature
> 0 that rule draws from the target's softmax. Both sides draw with
Philox4x32-10 on the same counter and key and an integer CDF, so the sampled
tokens, and the walk that follows them, agree exactly. Twelve seeded random
shapes (those of the greedy acceptance test) run at random temperatures,
seeds and offsets.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_build_amd import api, synth
from gpu_util import DEV, note

pytestmark = pytest.mark.gpu

KEYS = ("accepted", "accepted_nodes", "accept_len", "bonus", "target_tokens")


def _gpu_sample(tl, tree, L, tau, seed, offset, with_targets=True, with_nodes=True):
    tok = torch.from_numpy(tree["tokens"]).to(DEV)
    B, T = tok.shape
    par = torch.from_numpy(tree["parents"]).to(DEV)
    nn = torch.from_numpy(tree["num_nodes"]).to(DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    acc = torch.full((B, L), -7, **i32)
    accn = torch.full((B, L), -7, **i32) if with_nodes else None
    alen, bonus = torch.full((B,), -7, **i32), torch.full((B,), -7, **i32)
    targ = torch.full((B, T), -7, **i32) if with_targets else None
    ws = None if with_targets else api.new_workspace(api.ddtree_accept_workspace_size(B, T), DEV)
    api.ddtree_accept_sample(tl.to(DEV), tok, par, nn, L, tau, seed, offset, acc, accn, alen,
                             bonus, targ, ws)
    torch.cuda.synchronize()
    out = dict(accepted=acc.cpu().numpy(), accept_len=alen.cpu().numpy(),
               bonus=bonus.cpu().numpy())
    if with_nodes:
        out["accepted_nodes"] = accn.cpu().numpy()
    if with_targets:
        out["target_tokens"] = targ.cpu().numpy()
    return out


def _same(g, o):
    for k in KEYS:
        if k in g:
            np.testing.assert_array_equal(g[k], o[k], err_msg=k)


def _tree(B, L, V, K, N, seed):
    g = torch.Generator().manual_seed(seed)
    return oracle.build_tree(torch.randn(B, L, V, generator=g) * 2, list(range(B)), K, N, 1.0)


def _planted(tree, V, dtype, seed, follow=0.8, margin=16.0):
    """Random target logits; at the root and at most other nodes one child's
    token gets a margin large enough that the sample usually follows it
    (deep walks)."""
    rng = np.random.default_rng(seed)
    B, T = tree["tokens"].shape
    x = torch.from_numpy(rng.standard_normal((B, T, V)).astype(np.float32))
    for b in range(B):
        n = tree["num_nodes"][b]
        kids = [[] for _ in range(T)]
        for c in range(1, n):
            kids[tree["parents"][b, c]].append(c)
        for i in range(n):
            if kids[i] and (i == 0 or rng.random() < follow):
                x[b, i, tree["tokens"][b, kids[i][int(rng.integers(len(kids[i])))]]] += margin
    return x.to(dtype)


@pytest.mark.parametrize("tau", [1.0, 0.7, 1.6])
@pytest.mark.parametrize("V,dtype", [(64, torch.float32), (1001, torch.bfloat16),
                                     (1001, torch.float32), (32000, torch.bfloat16),
                                     (151936, torch.bfloat16), (151936, torch.float32)])
def test_accept_sample_matches_oracle(V, dtype, tau):
    B, L, K, N = 3, 6, 4, 40
    tree = _tree(B, L, V, K, N, seed=V)
    # margin tau * (12 + ln V): the planted token outweighs the rest of the
    # row by about e^12 at any temperature
    tl = _planted(tree, V, dtype, seed=V + 1, margin=tau * (12.0 + np.log(V)))
    tl[0, 3, :] = float("-inf")                     # no finite value -> token 0
    tl[1, 1, :] = float("-inf")
    tl[1, 1, V // 2] = 0.5                          # one finite value -> that token
    if dtype == torch.float32:
        tl[1, 2, 5] = float("nan")
        tl[2, 0, 7] = float("inf")                  # +inf counts as -inf
        tl[2, 4, :] = float("nan")
    note("accept_sample V=%d %s tau=%g" % (V, dtype, tau))
    g = _gpu_sample(tl, tree, L, tau, seed=0x1234_5678_9ABC, offset=3)
    o = oracle.accept_sample(tl, tree["tokens"], tree["parents"], tree["num_nodes"], L, tau,
                             0x1234_5678_9ABC, 3)
    _same(g, o)
    assert g["target_tokens"][0, 3] == 0 and g["target_tokens"][1, 1] == V // 2
    assert g["accept_len"].max() >= 2               # the planted paths are followed


@pytest.mark.parametrize("N", [127, 128, 255, 256, 600, 1024])
def test_accept_sample_large_trees(N):
    """T past one wave of the walk's register chase (128) and past one
    workgroup of 256 threads (the 1024-thread walk)."""
    B, L, V, K = 2, 24, 700, 8
    tree = _tree(B, L, V, K, N, seed=N)
    tl = _planted(tree, V, torch.bfloat16, seed=N, follow=0.95, margin=20.0)
    note("accept_sample large tree N=%d" % N)
    g = _gpu_sample(tl, tree, L, 1.0, seed=N, offset=2**40 + 5)
    o = oracle.accept_sample(tl, tree["tokens"], tree["parents"], tree["num_nodes"], L, 1.0, N,
                             2**40 + 5)
    _same(g, o)


def test_accept_sample_seeds_offsets_and_optional_outputs():
    """Key and counter halves above 2^32 reach the generator; NULL target
    tokens (kept in the workspace) and NULL node indices change nothing."""
    B, L, V, K, N = 4, 7, 3000, 6, 90
    tree = _tree(B, L, V, K, N, seed=3)
    tl = _planted(tree, V, torch.bfloat16, seed=3, follow=0.9)
    seen = set()
    for seed, offset in [(0, 0), (2**64 - 1, 2**64 - 1), (2**33 + 1, 7), (7, 2**33 + 1)]:
        note("accept_sample seed=%d offset=%d" % (seed, offset))
        o = oracle.accept_sample(tl, tree["tokens"], tree["parents"], tree["num_nodes"], L, 0.9,
                                 seed, offset)
        _same(_gpu_sample(tl, tree, L, 0.9, seed, offset), o)
        _same(_gpu_sample(tl, tree, L, 0.9, seed, offset, with_targets=False, with_nodes=False), o)
        seen.add(o["target_tokens"].tobytes())
    assert len(seen) == 4                           # every (seed, offset) draws differently


def test_accept_sample_heavy_ties_and_extreme_scale():
    """Rows of equal values (uniform draw over the vocabulary), rows whose
    maximum repeats, and logits scaled far apart by a small temperature."""
    B, L, V, K, N = 2, 5, 5000, 4, 30
    tree = _tree(B, L, V, K, N, seed=8)
    tl = torch.randn(B, N + 1, V) * 0.1
    tl[0] = 2.0                                     # all equal
    tl[1, :, ::97] = 3.0                            # repeated maximum
    for tau in (1.0, 0.05, 20.0):
        note("accept_sample ties tau=%g" % tau)
        g = _gpu_sample(tl, tree, L, tau, 99, 1)
        o = oracle.accept_sample(tl, tree["tokens"], tree["parents"], tree["num_nodes"], L, tau,
                                 99, 1)
        _same(g, o)


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_accept_sample_full_size_workloads(name):
    w = synth.WORKLOADS[name]
    x, _ = synth.drafter_logits(w)
    tree = oracle.build_tree(x, synth.root_tokens(w), w.K, w.N, w.taus[0])
    tl = synth.target_logits(w)
    note("accept_sample workload %s" % name)
    g = _gpu_sample(tl, tree, w.L, 1.0, seed=w.seed, offset=11)
    o = oracle.accept_sample(tl, tree["tokens"], tree["parents"], tree["num_nodes"], w.L, 1.0,
                             w.seed, 11)
    _same(g, o)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_accept_sample_overflowing_products(dtype):
    """Logits whose product with 1/temperature overflows to +inf (ranked as
    -inf, like NaN and +inf logits), next to rows that stay finite; and a
    temperature whose reciprocal is +inf (every value ranked -inf except the
    negative ones' -inf products: token 0)."""
    B, L, V, K, N = 2, 4, 3000, 4, 20
    tree = _tree(B, L, V, K, N, seed=12)
    tl = torch.randn(B, N + 1, V) * 2.0
    tl[0, 0, 10] = 3e37                             # product 3e38 at tau 0.1: finite
    tl[0, 1, 11] = 3.3e37                           # product overflows: -inf
    tl[0, 1, 12] = 1e30
    tl[0, 2, ::5] = 3.39e38                         # many overflowing values
    tl[0, 3, 7] = float("inf")
    tl[0, 3, 8] = float("nan")
    tl[1, 0, :] = 3.39e38                           # every product overflows: token 0
    tl = tl.to(dtype)
    for tau in (0.1, 1.0, 1e-39):
        note("accept_sample overflow %s tau=%g" % (dtype, tau))
        g = _gpu_sample(tl, tree, L, tau, 5, 2)
        o = oracle.accept_sample(tl, tree["tokens"], tree["parents"], tree["num_nodes"], L, tau,
                                 5, 2)
        _same(g, o)


@pytest.mark.parametrize("seed", range(12))
def test_accept_sample_random_shapes(seed):
    """Seeded random shapes (those of the greedy acceptance test), a random
    target temperature in [0.3, 2] and random seed and offset words."""
    from test_gpu_accept import _random_accept_case
    tree, tl, L, c = _random_accept_case(seed)
    rng = np.random.default_rng(950 + seed)
    tau = float(rng.uniform(0.3, 2.0))
    key = int(rng.integers(0, 2**63))
    offset = int(rng.integers(0, 2**40))
    note("accept_sample random seed=%d tau=%g %s" % (seed, tau, c))
    g = _gpu_sample(tl, tree, L, tau, seed=key, offset=offset)
    o = oracle.accept_sample(tl, tree["tokens"], tree["parents"], tree["num_nodes"], L, tau, key,
                             offset)
    _same(g, o)
