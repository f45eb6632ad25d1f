"""GPU parity of ddtree_commit_kv against the oracle: byte-exact caches.

Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees",
§4.1: the matched path is committed and the first unmatched target token is
the next root. Covers bf16 and f32 caches, head slices from 64 to 1024 bytes,
one to eight kv-heads, paths that skip first children (sources that are other
moves' destinations), full-depth paths of 64 nodes, empty acceptance,
malformed requests next to good ones, the full-size workload shapes, and
twelve seeded random shapes.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_build_amd import api, synth
from gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def _walk_ids(tree, rng, follow=1.0, deep=False):
    """Target ids that lead the walk down a random path (to a leaf when
    follow = 1; each step taken with probability follow); deep: always into
    the child with the deepest subtree."""
    B, T = tree["tokens"].shape
    ids = rng.integers(0, 1 << 20, (B, T)).astype(np.int32)
    for b in range(B):
        n = int(tree["num_nodes"][b])
        kids = [[] for _ in range(T)]
        for c in range(1, n):
            kids[int(tree["parents"][b, c])].append(c)
        reach = [0] * T                     # depth of the deepest node below (children follow parents)
        for i in range(n - 1, -1, -1):
            reach[i] = max([reach[c] for c in kids[i]] + [int(tree["depths"][b, i])])
        node = 0
        while kids[node] and rng.random() < follow:
            if deep:
                c = max(kids[node], key=lambda c: reach[c])
            else:
                c = kids[node][int(rng.integers(len(kids[node])))]
            ids[b, node] = tree["tokens"][b, c]
            node = c
    return ids


def _gpu_commit(k, v, offs, P, acc, T):
    kd, vd = k.to(DEV), v.to(DEV)
    i32 = dict(dtype=torch.int32, device=DEV)
    newp = torch.full((len(P),), -7, **i32)
    roots = torch.full((len(P),), -7, **i32)
    api.ddtree_commit_kv(kd, vd, torch.as_tensor(np.asarray(offs, np.int64)).to(DEV),
                         torch.as_tensor(np.asarray(P, np.int32)).to(DEV),
                         torch.as_tensor(acc["accept_len"]).to(DEV),
                         torch.as_tensor(acc["accepted_nodes"]).to(DEV),
                         torch.as_tensor(acc["bonus"]).to(DEV), T, newp, roots)
    torch.cuda.synchronize()
    return kd.cpu(), vd.cpu(), newp.cpu().numpy(), roots.cpu().numpy()


def _check(k, v, offs, P, acc, T):
    gk, gv, newp, roots = _gpu_commit(k, v, offs, P, acc, T)
    o = oracle.commit_kv(k, v, offs, P, acc["accept_len"], acc["accepted_nodes"], acc["bonus"], T)
    np.testing.assert_array_equal(oracle.as_raw(gk)[0], o["k"])
    np.testing.assert_array_equal(oracle.as_raw(gv)[0], o["v"])
    np.testing.assert_array_equal(newp, o["new_prefix_lens"])
    np.testing.assert_array_equal(roots, o["next_roots"])
    return o


def _region_caches(P, T, Hkv, D, dtype, seed, gap=5):
    rng = np.random.default_rng(seed)
    offs, total = [], gap
    for p in P:
        offs.append(total)
        total += int(p) + T + gap
    g = torch.Generator().manual_seed(seed)
    k = torch.randn(total, Hkv, D, generator=g).to(dtype)
    v = torch.randn(total, Hkv, D, generator=g).to(dtype)
    return k, v, np.array(offs, np.int64), rng


@pytest.mark.parametrize("Hkv,D,dtype", [(8, 128, torch.bfloat16), (2, 64, torch.bfloat16),
                                         (1, 8, torch.bfloat16), (8, 128, torch.float32),
                                         (3, 32, torch.float32), (2, 256, torch.float32)])
def test_commit_matches_oracle(Hkv, D, dtype):
    B, L, V, K, N = 5, 12, 60, 3, 80
    g = torch.Generator().manual_seed(Hkv * D)
    tree = oracle.build_tree(torch.randn(B, L, V, generator=g) * 2, list(range(B)), K, N, 1.0)
    T = N + 1
    P = [0, 7, 33, 1, 250]
    k, v, offs, rng = _region_caches(P, T, Hkv, D, dtype, seed=Hkv + D)
    ids = _walk_ids(tree, rng, follow=0.9)
    acc = oracle.accept(None, ids, tree["tokens"], tree["parents"], tree["num_nodes"], L)
    note("commit Hkv=%d D=%d %s lens=%s" % (Hkv, D, dtype, list(acc["accept_len"])))
    _check(k, v, offs, P, acc, T)
    assert acc["accept_len"].max() >= 3


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 256)])
def test_commit_full_depth_chains(dtype, D):
    """L = 64 accepted nodes per request; with D * esize = 1024 bytes every
    thread moves its full share of 16 chunks. One request's path skips the
    first child at every level (each source is the next move's destination)."""
    L, T, Hkv = 64, 200, 4
    B = 3
    tokens = np.full((B, T), -1, np.int32)
    parents = np.full((B, T), -1, np.int32)
    nodes = np.full((B, L), -1, np.int32)
    for b in range(B):
        tokens[b, 0] = 5
        if b == 1:   # node 2k+1 is a dead sibling, node 2k+2 continues the path
            for d in range(L):
                p = 0 if d == 0 else 2 * d
                tokens[b, 2 * d + 1], parents[b, 2 * d + 1] = 1000 + d, p
                tokens[b, 2 * d + 2], parents[b, 2 * d + 2] = 2000 + d, p
                nodes[b, d] = 2 * d + 2
        else:        # a chain 0 - 1 - 2 - ...: every accepted row is already in place
            for d in range(L):
                tokens[b, d + 1], parents[b, d + 1] = 3000 + d, d
                nodes[b, d] = d + 1
    acc = dict(accept_len=np.array([L, L, 17], np.int32), accepted_nodes=nodes,
               bonus=np.array([9, 10, 11], np.int32))
    acc["accepted_nodes"][2, 17:] = -1
    P = [3, 100, 0]
    k, v, offs, _ = _region_caches(P, T, Hkv, D, dtype, seed=D)
    note("commit full depth %s D=%d" % (dtype, D))
    _check(k, v, offs, P, acc, T)


def test_commit_malformed_and_empty_requests():
    L, T, Hkv, D = 8, 20, 2, 128
    P = [4, 4, 4, 4, 4, 4, 4]
    k, v, offs, _ = _region_caches(P, T, Hkv, D, torch.bfloat16, seed=3)
    nodes = np.tile(np.array([[3, 5, 9, 10, -1, -1, -1, -1]], np.int32), (7, 1))
    lens = np.array([4, 0, 9, 4, 4, 4, 4], np.int32)
    nodes[3, 2] = 0          # node 0 cannot be accepted
    nodes[4, 1] = T          # past the tree
    lens[5] = -1             # negative length
    P[6] = 10 ** 6           # region past the cache
    acc = dict(accept_len=lens, accepted_nodes=nodes, bonus=np.arange(7, dtype=np.int32) + 50)
    note("commit malformed")
    o = _check(k, v, offs, P, acc, T)
    assert list(o["new_prefix_lens"]) == [9, 5, -1, -1, -1, -1, -1]


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_commit_full_size_workloads(name):
    w = synth.WORKLOADS[name]
    x, _ = synth.drafter_logits(w)
    tree = oracle.build_tree(x, synth.root_tokens(w), w.K, w.N, w.taus[0])
    P = synth.prefix_lengths(w)
    offs = synth.kv_offsets(P, w.T)
    rows = int(offs[-1]) + int(P[-1]) + w.T
    g = torch.Generator().manual_seed(w.seed + 77)
    k = torch.randn(rows, w.Hkv, w.D, generator=g).to(w.torch_dtype)
    v = torch.randn(rows, w.Hkv, w.D, generator=g).to(w.torch_dtype)
    ids = _walk_ids(tree, np.random.default_rng(w.seed), deep=True)
    acc = oracle.accept(None, ids, tree["tokens"], tree["parents"], tree["num_nodes"], w.L)
    note("commit workload %s (%d rows, accepted %s)" % (name, rows, list(acc["accept_len"][:8])))
    _check(k, v, offs.numpy(), P.numpy(), acc, w.T)


@pytest.mark.parametrize("seed", range(12))
def test_commit_random_shapes(seed):
    """Seeded random shapes: 1-8 requests, blocks of 1-32 positions, budgets
    up to 1,024, 1-8 kv-heads, head slices of 16 to 1,024 bytes in bf16 or
    f32, prefixes of 0-500 rows, and walks that follow the tree at a random
    rate (empty acceptance included)."""
    rng = np.random.default_rng(1100 + seed)
    B = int(rng.integers(1, 9))
    L = int(rng.integers(1, 33))
    N = int(rng.choice([int(rng.integers(1, 72)), int(rng.integers(72, 1025))]))
    K = int(rng.integers(1, 9))
    Hkv = int(rng.integers(1, 9))
    dtype = torch.float32 if rng.random() < 0.4 else torch.bfloat16
    per16 = 4 if dtype == torch.float32 else 8          # values per 16 bytes
    D = per16 * int(rng.integers(1, 65))
    P = [int(x) for x in rng.integers(0, 501, size=B)]
    g = torch.Generator().manual_seed(1200 + seed)
    tree = oracle.build_tree(torch.randn(B, L, 50, generator=g) * 2, list(range(B)), K, N, 1.0)
    T = N + 1
    k, v, offs, rng2 = _region_caches(P, T, Hkv, D, dtype, seed=1300 + seed)
    ids = _walk_ids(tree, rng2, follow=float(rng.uniform(0.0, 1.0)))
    acc = oracle.accept(None, ids, tree["tokens"], tree["parents"], tree["num_nodes"], L)
    note("commit random seed=%d B=%d L=%d N=%d Hkv=%d D=%d %s lens=%s" % (
        seed, B, L, N, Hkv, D, dtype, list(acc["accept_len"])))
    _check(k, v, offs, P, acc, T)
