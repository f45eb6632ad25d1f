"""Pins for the oracle's KV compaction and bonus hand-off (CPU only).

Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees",
§4.1: the matched path is accepted and the first unmatched target token is
the next round's root. After a tree verify the K/V rows of the tree follow
the prefix in node order; committing the accepted path must leave the cache
exactly as a plain left-to-right forward over the committed tokens would:
row j holds the K/V of the token sequence up to position j.

The pin below builds the tree rows the way a causal target produces them
(each row a fixed function of the token sequence from the start of the
request to that node) and checks the compacted cache against that function
evaluated on the committed token sequence -- the accepted tokens, never the
node indices the oracle moves.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle

HKV, D = 2, 8


def kv_of(seq, which):
    """K (which=0) or V (which=1) row of the last token of a sequence."""
    h = zlib.crc32(np.asarray(seq, np.int64).tobytes() + bytes([which]))
    return np.random.default_rng(h).standard_normal((HKV, D)).astype(np.float32)


def _tree(B, L, V, K, N, seed):
    g = torch.Generator().manual_seed(seed)
    return oracle.build_tree(torch.randn(B, L, V, generator=g) * 2, list(range(B)), K, N, 1.0)


def _path(tree, b, node):
    """Token sequence from the root to node (root included)."""
    seq = []
    while node >= 0:
        seq.append(int(tree["tokens"][b, node]))
        node = int(tree["parents"][b, node])
    return seq[::-1]


def _setup(tree, prefix_lens, slack, rng, dtype):
    B, T = tree["tokens"].shape
    prefixes = [list(rng.integers(0, 1000, int(p))) for p in prefix_lens]
    offs = np.zeros(B, np.int64)
    total = 0
    for b in range(B):
        offs[b] = total
        total += int(prefix_lens[b]) + T + slack
    k = rng.standard_normal((total, HKV, D)).astype(np.float32)
    v = rng.standard_normal((total, HKV, D)).astype(np.float32)
    for b in range(B):
        o, P = int(offs[b]), int(prefix_lens[b])
        for j in range(P):
            k[o + j], v[o + j] = kv_of(prefixes[b][:j + 1], 0), kv_of(prefixes[b][:j + 1], 1)
        for i in range(int(tree["num_nodes"][b])):
            seq = prefixes[b] + _path(tree, b, i)
            k[o + P + i], v[o + P + i] = kv_of(seq, 0), kv_of(seq, 1)
    return (torch.from_numpy(k).to(dtype), torch.from_numpy(v).to(dtype), offs, prefixes)


def _walk_ids(tree, rng, stop_at_leaf=True):
    """Target ids that lead the walk down a random root-to-leaf path."""
    B, T = tree["tokens"].shape
    ids = rng.integers(0, 5000, (B, T)).astype(np.int32)
    for b in range(B):
        n = int(tree["num_nodes"][b])
        node = 0
        while True:
            kids = [c for c in range(1, n) if tree["parents"][b, c] == node]
            if not kids:
                break
            c = kids[int(rng.integers(len(kids)))]
            ids[b, node] = tree["tokens"][b, c]
            node = c
    return ids


def _as_f32(raw, dt):
    if dt == oracle.F32:
        return raw
    return (raw.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_compaction_equals_sequential_forward(dtype, seed):
    rng = np.random.default_rng(seed)
    B, L, V, K, N = 3, 6, 40, 3, 30
    tree = _tree(B, L, V, K, N, seed=10 + seed)
    T = N + 1
    P = rng.integers(0, 9, B)
    k, v, offs, prefixes = _setup(tree, P, slack=3, rng=rng, dtype=dtype)
    ids = _walk_ids(tree, rng)
    acc = oracle.accept(None, ids, tree["tokens"], tree["parents"], tree["num_nodes"], L)
    out = oracle.commit_kv(k, v, offs, P, acc["accept_len"], acc["accepted_nodes"], acc["bonus"], T)
    kk, vv = _as_f32(out["k"], out["dtype"]), _as_f32(out["v"], out["dtype"])
    k0, v0 = _as_f32(*oracle.as_raw(k)), _as_f32(*oracle.as_raw(v))
    cast = (lambda x: x) if dtype == torch.float32 else (
        lambda x: torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert acc["accept_len"].max() >= 2
    for b in range(B):
        o, p, n = int(offs[b]), int(P[b]), int(acc["accept_len"][b])
        committed = prefixes[b] + [int(tree["tokens"][b, 0])] + list(acc["accepted"][b, :n])
        for j in range(p + 1 + n):           # every committed position, prefix and root included
            np.testing.assert_array_equal(kk[o + j], cast(kv_of(committed[:j + 1], 0)))
            np.testing.assert_array_equal(vv[o + j], cast(kv_of(committed[:j + 1], 1)))
        # rows of the tree region that received no move keep their values
        for j in range(p + 1 + n, p + T):
            np.testing.assert_array_equal(kk[o + j], k0[o + j])
        assert out["new_prefix_lens"][b] == p + 1 + n
        assert out["next_roots"][b] == acc["bonus"][b]
    # the space after each region is never touched
    for b in range(B):
        end = int(offs[b]) + int(P[b]) + T
        np.testing.assert_array_equal(kk[end:end + 3], k0[end:end + 3])


def test_compaction_of_a_path_skipping_the_first_child():
    """Accepted nodes 2, 3, ...: each source is the next move's destination."""
    T, L = 8, 5
    tokens = np.array([[7, 11, 12, 13, 14, 15, 16, 17]], np.int32)
    parents = np.array([[-1, 0, 0, 2, 3, 4, 5, 6]], np.int32)
    tree = dict(tokens=tokens, parents=parents, num_nodes=np.array([T], np.int32))
    rng = np.random.default_rng(5)
    k, v, offs, prefixes = _setup(tree, np.array([4]), slack=0, rng=rng, dtype=torch.float32)
    ids = np.array([[12, 0, 13, 14, 15, 16, 17, 0]], np.int32)
    acc = oracle.accept(None, ids, tokens, parents, tree["num_nodes"], L)
    assert list(acc["accepted_nodes"][0]) == [2, 3, 4, 5, 6]
    out = oracle.commit_kv(k, v, offs, [4], acc["accept_len"], acc["accepted_nodes"], acc["bonus"], T)
    committed = prefixes[0] + [7, 12, 13, 14, 15, 16]
    for j in range(len(committed)):
        np.testing.assert_array_equal(out["k"][j], kv_of(committed[:j + 1], 0))
    assert out["new_prefix_lens"][0] == 4 + 1 + 5 and out["next_roots"][0] == acc["bonus"][0]


def test_empty_acceptance_keeps_the_root_only():
    T, L = 6, 4
    rng = np.random.default_rng(2)
    k = torch.from_numpy(rng.standard_normal((20, HKV, D)).astype(np.float32))
    v = torch.from_numpy(rng.standard_normal((20, HKV, D)).astype(np.float32))
    out = oracle.commit_kv(k, v, [3], [5], [0], np.full((1, L), -1, np.int32), [42], T)
    np.testing.assert_array_equal(out["k"], k.numpy())
    np.testing.assert_array_equal(out["v"], v.numpy())
    assert out["new_prefix_lens"][0] == 6 and out["next_roots"][0] == 42


@pytest.mark.parametrize("case", ["n_above_L", "n_above_T", "node_zero", "node_T", "past_rows",
                                  "neg_prefix", "neg_offset"])
def test_malformed_requests_are_left_alone(case):
    T, L, rows = 6, 4, 40
    rng = np.random.default_rng(3)
    k = torch.from_numpy(rng.standard_normal((rows, HKV, D)).astype(np.float32))
    v = torch.from_numpy(rng.standard_normal((rows, HKV, D)).astype(np.float32))
    offs, P, n = [0, 20], [4, 4], [2, 2]
    a = np.array([[3, 2, -1, -1], [1, 2, -1, -1]], np.int32)
    if case == "n_above_L":
        n[1] = 5
    elif case == "n_above_T":
        a[1] = [1, 2, 3, 4]
        n[1] = 4
        T = 4                                      # T - 1 = 3 < 4
    elif case == "node_zero":
        a[1, 1] = 0
    elif case == "node_T":
        a[1, 0] = T
    elif case == "past_rows":
        P[1] = rows - 20 - T + 1
    elif case == "neg_prefix":
        P[1] = -1
    elif case == "neg_offset":
        offs[1] = -2
    out = oracle.commit_kv(k, v, offs, P, n, a, [8, 9], T)
    assert out["new_prefix_lens"][1] == -1 and out["next_roots"][1] == -1
    np.testing.assert_array_equal(out["k"][20:], k.numpy()[20:])
    np.testing.assert_array_equal(out["v"][20:], v.numpy()[20:])
    # the well-formed request is still committed
    assert out["new_prefix_lens"][0] == 4 + 1 + 2 and out["next_roots"][0] == 8
    np.testing.assert_array_equal(out["k"][4 + 1], k.numpy()[4 + 3])
    np.testing.assert_array_equal(out["k"][4 + 2], k.numpy()[4 + 2])
