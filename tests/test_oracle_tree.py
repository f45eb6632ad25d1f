"""Pins for the oracle's best-first tree, mask and walk (CPU only).

Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees".
  §4.2 / App. A  the surrogate is additive over prefix probabilities and its
                 optimum under budget B is the B most probable prefixes,
                 which are prefix-closed (Proposition 2)
  §4.3 / App. A  the best-first search (pop the best, push next sibling and
                 best child) returns exactly those B prefixes
  Abstract, §4.1 ancestor-only mask; the walk accepts the matched path and
                 the first unmatched target token is the next bonus
The pins: a brute-force enumeration of the restricted prefix set, a
per-depth selection that reaches the workloads' full sizes, a
hand-worked example, a tree-knapsack DP and an exhaustive search of all
prefix-closed trees (optimality), Monte-Carlo acceptance (additivity),
structural invariants and special cases.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# independent reference: enumerate every restricted prefix, order, cut
# --------------------------------------------------------------------------
def brute_force_tree(tok, lp, L, K, N, root):
    """All prefixes of length 1..L over the per-position candidate lists.

    Within one depth the order is (score desc, parent's order, rank asc);
    across depths (score desc, depth asc, within-depth order). Scores are fp32
    sums accumulated from the root. The first N form the tree, numbered in
    that order (root = 0).
    """
    levels = []
    prev = [dict(score=np.float32(0.0), node=None)]
    for d in range(1, L + 1):
        cands = []
        for ppos, p in enumerate(prev):
            for r in range(K):
                s = np.float32(p["score"] + np.float32(lp[d - 1][r]))
                cands.append(dict(score=s, ppos=ppos, rank=r, parent=p, depth=d,
                                  token=int(tok[d - 1][r])))
        cands.sort(key=lambda c: (-float(c["score"]), c["ppos"], c["rank"]))
        for i, c in enumerate(cands):
            c["pos"] = i
        levels.append(cands)
        prev = cands
    everything = [c for lvl in levels for c in lvl]
    everything.sort(key=lambda c: (-float(c["score"]), c["depth"], c["pos"]))
    chosen = everything[:N]
    index = {id(c): j + 1 for j, c in enumerate(chosen)}
    T = N + 1
    out = dict(tokens=np.full(T, -1, np.int32), parents=np.full(T, -1, np.int32),
               depths=np.full(T, -1, np.int32), scores=np.full(T, -np.inf, np.float32))
    out["tokens"][0], out["depths"][0], out["scores"][0] = root, 0, 0.0
    for j, c in enumerate(chosen):
        n = j + 1
        out["tokens"][n] = c["token"]
        out["depths"][n] = c["depth"]
        out["scores"][n] = c["score"]
        out["parents"][n] = 0 if c["depth"] == 1 else index[id(c["parent"])]
    out["num_nodes"] = len(chosen) + 1
    return out


def level_topn_tree(tok, lp, L, K, N, root):
    """The same tree by per-depth selection, without a priority queue.

    Every depth-d candidate is a depth-(d-1) prefix extended by one of the K
    candidates of position d, and all of them share position d's log-prob
    row; so a depth-d prefix among the N best of its depth has its parent
    among the N best of depth d-1 (the parent's N betters, extended by the
    same rank, would all precede it). Keeping the N best per depth, in the
    within-depth order (score desc, parent's position, rank), and then the
    N best of all depths under (score desc, depth asc, within-depth
    position) gives the node list and numbering without enumerating the
    K^L prefixes, so it runs at the workloads' full sizes.
    """
    levels = []
    prev = np.zeros(1, np.float32)
    for d in range(1, L + 1):
        n = len(prev)
        ppos = np.repeat(np.arange(n), K)
        rank = np.tile(np.arange(K), n)
        score = (prev[ppos] + lp[d - 1][rank]).astype(np.float32)   # fp32 sums from the root
        keep = np.lexsort((rank, ppos, -score.astype(np.float64)))[:N]
        levels.append((score[keep], ppos[keep], rank[keep]))
        prev = score[keep]
    depth = np.concatenate([np.full(len(lv[0]), d + 1) for d, lv in enumerate(levels)])
    pos = np.concatenate([np.arange(len(lv[0])) for lv in levels])
    score = np.concatenate([lv[0] for lv in levels])
    chosen = np.lexsort((pos, depth, -score.astype(np.float64)))[:N]
    node_of = {(int(depth[c]), int(pos[c])): j + 1 for j, c in enumerate(chosen)}
    T = N + 1
    out = dict(tokens=np.full(T, -1, np.int32), parents=np.full(T, -1, np.int32),
               depths=np.full(T, -1, np.int32), scores=np.full(T, -np.inf, np.float32))
    out["tokens"][0], out["depths"][0], out["scores"][0] = root, 0, 0.0
    for j, c in enumerate(chosen):
        d, q = int(depth[c]), int(pos[c])
        sc, pp, rk = levels[d - 1][0][q], levels[d - 1][1][q], levels[d - 1][2][q]
        out["tokens"][j + 1] = tok[d - 1][rk]
        out["depths"][j + 1] = d
        out["scores"][j + 1] = sc
        out["parents"][j + 1] = 0 if d == 1 else node_of[(d - 1, int(pp))]
    out["num_nodes"] = len(chosen) + 1
    return out


def _same_tree(a, b):
    np.testing.assert_array_equal(a["tokens"], b["tokens"])
    np.testing.assert_array_equal(a["parents"], b["parents"])
    np.testing.assert_array_equal(a["depths"], b["depths"])
    np.testing.assert_array_equal(a["scores"].view(np.uint32), b["scores"].view(np.uint32))
    assert a["num_nodes"] == b["num_nodes"]


def _tied_table(rng, L, K, V):
    """Candidate tables whose log-probs come from a tiny set: many exact ties."""
    levels = np.float32([-0.25, -0.5, -1.0, -1.0, -1.5, -2.0, -2.0, -3.0])
    lp = np.sort(rng.choice(levels, size=(L, K)), axis=1)[:, ::-1].astype(np.float32)
    tok = np.stack([rng.permutation(V)[:K] for _ in range(L)]).astype(np.int32)
    return tok, np.ascontiguousarray(lp)


def _oracle_table(rng, L, K, V, sigma, tau=1.0):
    import torch
    g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))
    logits = (torch.randn(1, L, V, generator=g) * sigma)
    res = oracle.build_tree(logits, [0], K, 1, tau)
    return res["topk_tok"][0], res["topk_lp"][0], logits


@pytest.mark.parametrize("L,K,N", [(1, 4, 3), (2, 2, 6), (3, 3, 10), (4, 4, 8), (4, 4, 60),
                                   (5, 3, 40), (3, 8, 100), (4, 2, 30)])
def test_matches_brute_force_enumeration(L, K, N):
    rng = np.random.default_rng(L * 100 + K * 10 + N)
    for trial in range(6):
        if trial % 2 == 0:
            tok, lp = _tied_table(rng, L, K, 50)
        else:
            tok, lp, _ = _oracle_table(rng, L, K, 50, 2.0)
        root = int(rng.integers(50))
        got = oracle.tree(tok, lp, L, K, N, root)
        ref = brute_force_tree(tok, lp, L, K, N, root)
        _same_tree(got, ref)


@pytest.mark.parametrize("L,K,N", [(4, 4, 60), (5, 3, 40), (3, 8, 100)])
def test_level_selection_matches_brute_force(L, K, N):
    """The per-depth selection itself, against full enumeration."""
    rng = np.random.default_rng(7 * L + K + N)
    for trial in range(4):
        tok, lp = _tied_table(rng, L, K, 50) if trial % 2 == 0 else _oracle_table(rng, L, K, 50, 2.0)[:2]
        _same_tree(level_topn_tree(tok, lp, L, K, N, 3), brute_force_tree(tok, lp, L, K, N, 3))


@pytest.mark.parametrize("L,K,N,tied", [(16, 8, 64, True), (16, 16, 256, True), (32, 16, 512, True),
                                        (16, 16, 256, False), (32, 8, 1024, False)])
def test_matches_level_selection_large(L, K, N, tied):
    """The heap's node list at sizes where enumeration is out of reach."""
    rng = np.random.default_rng(L * K + N)
    for trial in range(2):
        tok, lp = _tied_table(rng, L, K, 1000) if tied else _oracle_table(rng, L, K, 1000, 3.0)[:2]
        root = int(rng.integers(1000))
        _same_tree(oracle.tree(tok, lp, L, K, N, root), level_topn_tree(tok, lp, L, K, N, root))


@pytest.mark.parametrize("name", ["L16_V32000_K8_N64_P2048", "L16_V151936_K16_N256_P8192",
                                  "B4_L32_V151936_K16_N512_P65536"])
def test_workload_trees_match_level_selection(name):
    """The trees of the benchmark workloads (seeded inputs, every draft
    temperature they use), node for node."""
    from draft_tree_build_amd import synth
    w = synth.WORKLOADS[name]
    x, _ = synth.drafter_logits(w)
    roots = synth.root_tokens(w)
    for tau in w.taus:
        o = oracle.build_tree(x, roots, w.K, w.N, tau, want_mask=False)
        for b in range(w.batch):
            ref = level_topn_tree(o["topk_tok"][b], o["topk_lp"][b], w.L, w.K, w.N, int(roots[b]))
            got = {k: o[k][b] for k in ("tokens", "parents", "depths", "scores")}
            got["num_nodes"] = int(o["num_nodes"][b])
            _same_tree(got, ref)


def _read_golden(name):
    spec = dict(node=[], walk=[])
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            key, _, rest = line.partition(" ")
            if key in ("node", "walk"):
                spec[key].append(rest)
            else:
                spec[key] = rest
    return spec


def test_golden_hand_worked_tree():
    g = _read_golden("hand_tree_L2_V4.txt")
    L, V, K, N, root = (int(g[k]) for k in ("L", "V", "K", "N", "root"))
    q = np.array([[float(x) for x in g["q1"].split()], [float(x) for x in g["q2"].split()]])
    logits = np.log(q).astype(np.float32)[None]
    res = oracle.build_tree(logits, [root], K, N, 1.0)
    assert res["num_nodes"][0] == N + 1
    for row in g["node"]:
        i, tok, par, dep, prob = row.split()
        i = int(i)
        assert res["tokens"][0, i] == int(tok)
        assert res["parents"][0, i] == int(par)
        assert res["depths"][0, i] == int(dep)
        assert math.isclose(math.exp(res["scores"][0, i]), float(prob), rel_tol=1e-5)
    assert math.isclose(float(np.exp(res["scores"][0, 1:]).sum()), float(g["value"]), rel_tol=1e-5)
    np.testing.assert_array_equal(res["mask"][0, :, 0], [int(x) for x in g["mask"].split()])
    for w in g["walk"]:
        tgt, acc, alen, bonus = (p.split() for p in w.split("|"))
        r = oracle.walk(res["tokens"][0], res["parents"][0], N + 1, [int(x) for x in tgt], L)
        assert r["accept_len"] == int(alen[0])
        assert r["bonus"] == int(bonus[0])
        np.testing.assert_array_equal(r["accepted"][: int(alen[0])], [int(x) for x in acc])
        assert np.all(r["accepted"][int(alen[0]):] == -1)


# --------------------------------------------------------------------------
# optimality of the surrogate (Proposition 2)
# --------------------------------------------------------------------------
def _softmax64(x):
    x = np.asarray(x, np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


def _restricted_tree(logits, K):
    """Candidate tokens per position (numpy order: logit desc, id asc) and fp64 q."""
    L, V = logits.shape
    toks = [np.lexsort((np.arange(V), -logits[i]))[:K] for i in range(L)]
    qs = [_softmax64(logits[i]) for i in range(L)]
    return toks, qs


def _maxplus(a, b):
    c = np.full(len(a), -np.inf)
    for i in range(len(a)):
        if a[i] == -np.inf:
            continue
        m = len(a) - i
        c[i:] = np.maximum(c[i:], a[i] + b[:m])
    return c


def knapsack_best_value(logits, K, N):
    """Max over prefix-closed sets of <= N prefixes of the sum of their Q (tree DP)."""
    toks, qs = _restricted_tree(logits, K)
    L = len(toks)

    def best(depth, prob):
        # f[b]: best value of a subtree rooted at this prefix using <= b nodes
        f = np.zeros(N + 1)
        f[1:] = prob
        if depth < L and N > 1:
            kids = np.zeros(N)  # children combination with <= b nodes
            for t in toks[depth]:
                kids = _maxplus(kids, best(depth + 1, prob * qs[depth][t])[:N])
            f[1:] = prob + kids
        return f

    kids = np.zeros(N + 1)
    for t in toks[0]:
        kids = _maxplus(kids, best(1, qs[0][t]))
    return kids[N]


def tree_value(res, b, logits, tau=1.0):
    toks, qs = _restricted_tree(logits, res["topk_tok"].shape[-1])
    total = 0.0
    n = res["num_nodes"][b]
    prob = np.ones(n)
    for i in range(1, n):
        d = res["depths"][b, i]
        prob[i] = prob[res["parents"][b, i]] * qs[d - 1][res["tokens"][b, i]]
        total += prob[i]
    return total


@pytest.mark.parametrize("L,K,N,sigma", [(4, 3, 10, 2.0), (5, 4, 24, 1.5), (4, 4, 40, 3.0),
                                         (6, 2, 20, 1.0)])
def test_tree_maximises_surrogate_dp(L, K, N, sigma):
    rng = np.random.default_rng(L + K + N)
    for _ in range(3):
        logits = (rng.standard_normal((L, 30)) * sigma).astype(np.float32)
        res = oracle.build_tree(logits[None], [1], K, N, 1.0)
        got = tree_value(res, 0, logits)
        best = knapsack_best_value(logits, K, N)
        assert math.isclose(got, best, rel_tol=1e-6), (got, best)


def test_tree_maximises_surrogate_exhaustive():
    rng = np.random.default_rng(11)
    for L, K, N in [(3, 3, 4), (2, 4, 5), (3, 2, 5)]:
        logits = (rng.standard_normal((L, 12)) * 1.5).astype(np.float32)
        toks, qs = _restricted_tree(logits, K)
        prefixes = [p for d in range(1, L + 1) for p in itertools.product(range(K), repeat=d)]
        prob = {}
        for p in prefixes:
            pr = 1.0
            for i, r in enumerate(p):
                pr *= qs[i][toks[i][r]]
            prob[p] = pr
        best = 0.0
        count = 0
        for size in range(1, N + 1):
            for sub in itertools.combinations(prefixes, size):
                s = set(sub)
                if all(len(p) == 1 or p[:-1] in s for p in sub):
                    count += 1
                    best = max(best, sum(prob[p] for p in sub))
        res = oracle.build_tree(logits[None], [0], K, N, 1.0)
        assert count > 10
        assert math.isclose(tree_value(res, 0, logits), best, rel_tol=1e-6)


def test_surrogate_is_expected_acceptance_monte_carlo():
    """E_Q[accepted length] = sum of the tree's prefix probabilities (additivity)."""
    rng = np.random.default_rng(5)
    L, V, K, N = 4, 12, 3, 10
    logits = (rng.standard_normal((L, V)) * 2.0).astype(np.float32)
    logits[np.arange(L), rng.integers(0, V, L)] += 3.0
    res = oracle.build_tree(logits[None], [0], K, N, 1.0)
    n = res["num_nodes"][0]
    child = np.full((n, V), -1, np.int64)
    for i in range(1, n):
        child[res["parents"][0, i], res["tokens"][0, i]] = i
    M = 400_000
    ys = np.stack([rng.choice(V, size=M, p=_softmax64(logits[i])) for i in range(L)], 1)
    cur = np.zeros(M, np.int64)
    alive = np.ones(M, bool)
    acc = np.zeros(M)
    for i in range(L):
        nxt = child[cur, ys[:, i]]
        alive &= nxt >= 0
        acc += alive
        cur = np.where(alive, nxt, 0)
    expect = float(np.exp(res["scores"][0, 1:n].astype(np.float64)).sum())
    se = acc.std() / math.sqrt(M)
    assert abs(acc.mean() - expect) <= 4 * se + 1e-4, (acc.mean(), expect, se)
    assert expect > 0.3  # the check is not vacuous


# --------------------------------------------------------------------------
# invariants and special cases
# --------------------------------------------------------------------------
@pytest.mark.parametrize("L,V,K,N,tau", [(8, 200, 4, 50, 1.0), (16, 500, 8, 64, 1.0),
                                         (6, 100, 6, 200, 0.8), (4, 64, 4, 8, 1.0)])
def test_structural_invariants(L, V, K, N, tau):
    rng = np.random.default_rng(N)
    logits = (rng.standard_normal((3, L, V)) * 3.0).astype(np.float32)
    res = oracle.build_tree(logits, [1, 2, 3], K, N, tau)
    for b in range(3):
        n = res["num_nodes"][b]
        par, dep, sc, tk = (res[k][b] for k in ("parents", "depths", "scores", "tokens"))
        assert par[0] == -1 and dep[0] == 0 and sc[0] == 0.0
        for i in range(1, n):
            assert 0 <= par[i] < i
            assert dep[i] == dep[par[i]] + 1 <= L
            assert sc[i] <= sc[i - 1]
        rank = np.array([-1] + [list(res["topk_tok"][b, dep[i] - 1]).index(tk[i])
                                for i in range(1, n)])
        for p in range(n):
            kids = sorted(rank[i] for i in range(1, n) if par[i] == p)
            assert kids == list(range(len(kids)))
        assert np.all(tk[n:] == -1) and np.all(np.isneginf(sc[n:]))
        m = res["mask"][b]
        for i in range(n):
            bits = [j for j in range(N + 1) if (int(m[i, j // 64]) >> (j % 64)) & 1]
            chain, j = [], i
            while j >= 0:
                chain.append(j)
                j = par[j]
            assert sorted(chain) == bits
            assert len(bits) == dep[i] + 1
        assert np.all(m[n:] == 0)


def test_k1_is_the_argmax_chain():
    rng = np.random.default_rng(3)
    logits = (rng.standard_normal((1, 10, 300)) * 2).astype(np.float32)
    for N in (4, 10, 25):
        res = oracle.build_tree(logits, [7], 1, N, 1.0)
        n = min(N, 10)
        assert res["num_nodes"][0] == n + 1
        np.testing.assert_array_equal(res["tokens"][0, 1:n + 1], logits[0, :n].argmax(-1))
        np.testing.assert_array_equal(res["parents"][0, 1:n + 1], np.arange(n))


def test_k_at_least_n_is_invariant_in_k():
    rng = np.random.default_rng(4)
    logits = (rng.standard_normal((2, 6, 400)) * 2).astype(np.float32)
    a = oracle.build_tree(logits, [0, 1], 12, 12, 1.0)
    b = oracle.build_tree(logits, [0, 1], 20, 12, 1.0)
    for k in ("tokens", "parents", "depths", "num_nodes"):
        np.testing.assert_array_equal(a[k], b[k])
    np.testing.assert_array_equal(a["scores"].view(np.uint32), b["scores"].view(np.uint32))


def test_temperature_zero_puts_the_argmax_chain_first():
    rng = np.random.default_rng(6)
    L = 8
    logits = (rng.standard_normal((1, L, 500)) * 3).astype(np.float32)
    res = oracle.build_tree(logits, [2], 4, 30, 0.0)
    np.testing.assert_array_equal(res["tokens"][0, 1:L + 1], logits[0].argmax(-1))
    np.testing.assert_array_equal(res["parents"][0, 1:L + 1], np.arange(L))
    assert np.all(res["scores"][0, :L + 1] == 0.0)
    assert np.all(np.isneginf(res["scores"][0, L + 1:]))


def test_budget_larger_than_restricted_set():
    logits = np.random.default_rng(8).standard_normal((1, 2, 16)).astype(np.float32)
    res = oracle.build_tree(logits, [3], 2, 10, 1.0)
    assert res["num_nodes"][0] == 1 + 2 + 4
    assert np.all(res["tokens"][0, 7:] == -1) and np.all(res["parents"][0, 7:] == -1)
    assert np.all(res["depths"][0, 7:] == -1) and np.all(np.isneginf(res["scores"][0, 7:]))
    assert np.all(res["mask"][0, 7:] == 0)
