"""GPU parity of ddtree_build / ddtree_mask against the oracle: bit-exact.

Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees",
§3, §4.1-4.3, App. A. Covers every kernel variant (register-resident rows of
several lengths, streaming rows, unaligned rows), temperature 1 / scaled / 0,
the exact fallback of the top-K selection, non-finite and all -inf rows,
budget and block limits, the full-size workloads, and sixteen seeded random
shapes across the row-kernel variants, the heap and the level selection.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_build_amd import api, synth
from gpu_util import DEV, assert_same_build, gpu_build, note

pytestmark = pytest.mark.gpu


def _logits(B, L, V, seed, sigma=3.0, dtype=torch.bfloat16, boost=8.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, L, V, generator=g) * sigma
    if boost:
        idx = torch.randint(0, V, (B, L), generator=g)
        x.scatter_add_(2, idx[..., None], torch.full((B, L, 1), boost))
    return x.to(dtype)


CASES = [
    # (B, L, V, K, N, dtype) -- V picks the kernel variant
    (1, 4, 64, 4, 8, torch.float32),          # 256 threads, one vector per thread
    (2, 5, 1000, 8, 30, torch.bfloat16),      # 256 threads
    (2, 3, 1001, 6, 20, torch.bfloat16),      # unaligned rows: scalar path
    (1, 6, 1001, 5, 25, torch.float32),       # unaligned f32
    (3, 8, 5000, 8, 64, torch.bfloat16),      # 512 threads, 4 vectors per thread
    (1, 16, 32000, 8, 64, torch.bfloat16),    # 8 vectors per thread
    (2, 7, 60000, 16, 100, torch.bfloat16),   # split rows, 29 chunks
    (1, 5, 60000, 16, 100, torch.float32),
    (2, 4, 151936, 16, 50, torch.bfloat16),   # split rows, 32 chunks
    (16, 16, 151936, 8, 40, torch.bfloat16),  # 256 rows: split, 10 chunks of <= 2048 vectors
    (16, 16, 32768, 8, 70, torch.bfloat16),   # 256 rows of 4096 vectors: whole rows, 8 per thread
    (16, 16, 32776, 8, 70, torch.bfloat16),   # 256 rows of 4097 vectors: split, 3 chunks
    (1, 3, 151936, 8, 20, torch.float32),     # split rows, f32
    (1, 3, 400000, 32, 40, torch.bfloat16),   # streaming
]


@pytest.mark.parametrize("tau", [1.0, 0.7, 0.0])
@pytest.mark.parametrize("B,L,V,K,N,dtype", CASES)
def test_build_matches_oracle(B, L, V, K, N, dtype, tau):
    x = _logits(B, L, V, seed=V + K + N, dtype=dtype)
    roots = torch.arange(B, dtype=torch.int32) * 7 % V
    note("build B=%d L=%d V=%d K=%d N=%d %s tau=%g" % (B, L, V, K, N, dtype, tau))
    g, _ = gpu_build(x, roots, K, N, tau)
    o = oracle.build_tree(x, roots, K, N, tau)
    assert_same_build(g, o)


@pytest.mark.parametrize("B,L,V,K,N", [(1, 16, 32000, 32, 200), (1, 2, 151936, 32, 100),
                                       (1, 4, 9000, 24, 60)])
def test_build_split_rows_fewer_chunks_than_K(B, L, V, K, N):
    """Split rows where S < K chunks: the merge threshold is the K-th largest
    of the first ceil(K/S) words of every chunk."""
    x = _logits(B, L, V, seed=V + K, sigma=1.0, boost=0.0)
    note("build split S<K B=%d L=%d V=%d K=%d N=%d" % (B, L, V, K, N))
    g, _ = gpu_build(x, list(range(B)), K, N, 1.0)
    o = oracle.build_tree(x, list(range(B)), K, N, 1.0)
    assert_same_build(g, o)


def test_build_adversarial_rows():
    B, L, V, K, N = 2, 6, 5000, 16, 120
    x = _logits(B, L, V, seed=5, dtype=torch.float32)
    x[0, 0] = 1.5                                  # all equal: exact fallback (ties > buffer)
    x[0, 1] = torch.randint(-3, 3, (V,)).float()   # heavy ties at the top
    x[0, 2, 17] = float("nan")
    x[0, 2, 99] = float("inf")
    x[1, 0] = float("-inf")                        # no finite logit
    x[1, 1, :4000] = float("-inf")
    x[1, 2] = torch.where(torch.arange(V) % 3 == 0, torch.tensor(2.0), torch.tensor(float("-inf")))
    for tau in (1.0, 0.5, 0.0):
        for dtype in (torch.float32, torch.bfloat16):
            xd = x.to(dtype)
            note("build adversarial dtype=%s tau=%g" % (dtype, tau))
            g, _ = gpu_build(xd, [3, 4], K, N, tau)
            o = oracle.build_tree(xd, [3, 4], K, N, tau)
            assert_same_build(g, o)
            assert g["status"][0] & 1 and g["status"][1] & 2


@pytest.mark.parametrize("L,K,N", [(1, 1, 1), (1, 32, 1024), (64, 1, 64), (64, 2, 1024),
                                   (2, 2, 10), (16, 32, 1024), (33, 3, 700)])
def test_build_limits(L, K, N):
    x = _logits(2, L, 3000, seed=L * K + N, sigma=2.0)
    note("build limits L=%d K=%d N=%d" % (L, K, N))
    g, _ = gpu_build(x, [1, 2], K, N, 1.0)
    o = oracle.build_tree(x, [1, 2], K, N, 1.0)
    assert_same_build(g, o)


def test_build_repeatable_on_one_workspace():
    """Two calls on one workspace give identical results."""
    x = _logits(4, 8, 2000, seed=3)
    ws = api.new_workspace(api.ddtree_build_workspace_size(4, 8, 2000, 8, 40), DEV)
    note("build twice on one workspace")
    g1, _ = gpu_build(x, [0, 1, 2, 3], 8, 40, 1.0, ws=ws)
    g2, _ = gpu_build(x, [0, 1, 2, 3], 8, 40, 1.0, ws=ws)
    for k in g1:
        np.testing.assert_array_equal(g1[k], g2[k])
    o = oracle.build_tree(x, [0, 1, 2, 3], 8, 40, 1.0)
    assert_same_build(g2, o)


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_build_full_size_workloads(name):
    w = synth.WORKLOADS[name]
    x, _ = synth.drafter_logits(w)
    roots = synth.root_tokens(w)
    for tau in w.taus:
        note("build workload %s tau=%g" % (name, tau))
        g, _ = gpu_build(x, roots, w.K, w.N, tau)
        o = oracle.build_tree(x, roots, w.K, w.N, tau)
        assert_same_build(g, o)


def test_mask_matches_oracle():
    rng = np.random.default_rng(0)
    for T in (1, 9, 64, 65, 129, 513, 1025):
        B = 3
        par = np.full((B, T), -1, np.int32)
        nn = np.zeros(B, np.int32)
        for b in range(B):
            n = T if b == 0 else int(rng.integers(1, T + 1))
            nn[b] = n
            for i in range(1, n):
                par[b, i] = int(rng.integers(0, i)) if b != 2 else i - 1
        mask = torch.empty(B, T, (T + 63) // 64, dtype=torch.int64, device=DEV)
        note("mask T=%d" % T)
        api.ddtree_mask(torch.from_numpy(par).to(DEV), torch.from_numpy(nn).to(DEV), mask)
        got = mask.cpu().numpy().view(np.uint64)
        for b in range(B):
            np.testing.assert_array_equal(got[b], oracle.mask(par[b], nn[b], T))


def _lane_refills(lp, L, K, N, lanes=64):
    """How often a 64-entry sorted candidate window runs dry while overflow
    candidates remain, replayed on the oracle's own tables (the test below
    uses it only to make sure its inputs reach that case)."""
    def key(score, d, p, r):
        return (-float(score), d, p, r)
    scores = [np.float32(0)]
    s0 = np.float32(np.float32(0) + lp[0][0])
    head, over, n, refills = [(key(s0, 1, 0, 0), s0, 1, 0, 0)], [], 1, 0
    while n <= N:
        if not head:
            if not over:
                break
            refills += 1
            over.sort()
            head, over = over[:lanes], over[lanes:]
        _, s, d, p, r = head.pop(0)
        scores.append(s)
        new = []
        if r + 1 < K:
            v = np.float32(scores[p] + lp[d - 1][r + 1])
            new.append((key(v, d, p, r + 1), v, d, p, r + 1))
        if d < L:
            v = np.float32(s + lp[d][0])
            new.append((key(v, d + 1, n, 0), v, d + 1, n, 0))
        if len(head) >= N - n:
            over = []
        for c in new:
            if over and c >= min(over):
                over.append(c)
            else:
                head.append(c)
                head.sort()
                if len(head) > lanes:
                    over.append(head.pop())
        if len(head) >= N - n:
            over = []
        n += 1
    return refills


@pytest.mark.parametrize("L,K,spread", [(16, 8, 3.0), (64, 4, 3.0), (4, 32, 3.0), (16, 8, 0.0)])
def test_build_overflow_refills(L, K, spread):
    """Budgets far beyond 64 with widely spread log-probs: the candidate
    window of the tree kernel runs dry and is refilled from its overflow list."""
    B, V, N = 2, 64, 1024
    rng = np.random.default_rng(L * K)
    x = np.full((B, L, V), -60.0, np.float32)
    for b in range(B):
        for i in range(L):
            gaps = rng.exponential(spread, K) if spread else np.zeros(K)
            x[b, i, rng.permutation(V)[:K]] = -np.cumsum(gaps)
    x = torch.from_numpy(x)
    o = oracle.build_tree(x, [5, 6], K, N, 1.0)
    assert sum(_lane_refills(o["topk_lp"][b], L, K, N) for b in range(B)) > 0
    note("build overflow L=%d K=%d spread=%g" % (L, K, spread))
    g, _ = gpu_build(x, [5, 6], K, N, 1.0)
    assert_same_build(g, o)


@pytest.mark.parametrize("B,L,V,K", [(1, 2, 151936, 16), (16, 16, 5000, 8)])
def test_build_all_equal_rows_exact_fallback(B, L, V, K):
    """Rows of one repeated value: more tied candidates than the candidate
    buffer holds, so the exact selection runs -- inside row chunks (few rows,
    long vocabulary) and on whole rows (many rows)."""
    x = torch.full((B, L, V), 0.25, dtype=torch.bfloat16)
    x[0, 0, V // 3] = 1.0                          # one row with a single clear winner
    roots = list(range(B))
    for tau in (1.0, 0.0):
        note("build all-equal B=%d L=%d V=%d K=%d tau=%g" % (B, L, V, K, tau))
        g, _ = gpu_build(x, roots, K, 40, tau)
        o = oracle.build_tree(x, roots, K, 40, tau)
        assert_same_build(g, o)


@pytest.mark.parametrize("B,L,V,K,frac", [(1, 2, 151936, 16, 0.08), (16, 16, 20000, 8, 0.06)])
def test_build_many_tied_candidates(B, L, V, K, frac):
    """Rows whose top value repeats at a random fraction of positions: more
    tied candidates than a workgroup has threads, but few enough per wave to
    stay off the exact fallback, so the full sorting network orders them --
    inside row chunks (few rows) and on whole rows (many rows). Ties resolve
    to the lowest token ids."""
    g = torch.Generator().manual_seed(11)
    x = (torch.randn((B, L, V), generator=g) * 0.5).to(torch.bfloat16)
    x[torch.rand((B, L, V), generator=g) < frac] = 4.0
    roots = list(range(B))
    for tau in (1.0, 0.0):
        note("build tied B=%d L=%d V=%d K=%d frac=%g tau=%g" % (B, L, V, K, frac, tau))
        gb, _ = gpu_build(x, roots, K, 40, tau)
        o = oracle.build_tree(x, roots, K, 40, tau)
        assert_same_build(gb, o)


def _few_values(B, L, V, seed, values):
    """Logits drawn from a handful of values: log-probabilities tie within
    rows, so scores tie across siblings, cousins and depths."""
    g = torch.Generator().manual_seed(seed)
    idx = torch.randint(0, len(values), (B, L, V), generator=g)
    return torch.tensor(values, dtype=torch.float32)[idx].to(torch.bfloat16)


@pytest.mark.parametrize("L,V,K,N,kind", [
    (8, 500, 8, 129, "normal"), (16, 4000, 16, 300, "normal"), (32, 3000, 16, 1024, "normal"),
    (6, 400, 12, 500, "few"), (16, 600, 16, 1024, "few"), (3, 50, 32, 1024, "few"),
    (64, 300, 2, 1000, "few"), (4, 40, 4, 1024, "normal"),   # budget above the restricted set (340)
    (40, 300, 1, 200, "normal"), (12, 700, 8, 257, "peaked"),
    (8, 500, 8, 71, "few"), (8, 500, 8, 72, "few"),   # the two sides of the kernel switch
    (10, 400, 16, 159, "few"), (10, 400, 16, 160, "few"),   # same at temperature 0
    (16, 600, 8, 100, "normal"), (20, 900, 16, 140, "peaked")
])
@pytest.mark.parametrize("tau", [1.0, 0.7, 0.0])
def test_build_level_selection(L, V, K, N, kind, tau):
    """Budgets from 72 (from 160 at temperature 0) run the level-synchronous
    selection, smaller ones the heap's pops; both must give the oracle's
    heap tree: ties at the threshold score (bf16 logits from a handful of
    values, temperature 0's -inf tails), budgets above the restricted set
    (padding rows), K = 1 chains, deep trees under a peaked drafter, and the
    two budgets on either side of the switch."""
    B = 2
    if kind == "few":
        x = _few_values(B, L, V, seed=L * V + N, values=[2.0, 1.0, 1.0, 0.5, 0.0, -1.0])
    elif kind == "peaked":
        x = _logits(B, L, V, seed=L + N, sigma=1.0, boost=12.0)
    else:
        x = _logits(B, L, V, seed=L + N + K, sigma=2.0)
    roots = [3, 4]
    note("build level L=%d V=%d K=%d N=%d %s tau=%g" % (L, V, K, N, kind, tau))
    g, _ = gpu_build(x, roots, K, N, tau)
    o = oracle.build_tree(x, roots, K, N, tau)
    assert_same_build(g, o)


@pytest.mark.parametrize("value", [0.0, float("-inf")])
def test_build_level_selection_degenerate_rows(value):
    """All-equal rows (every prefix of a depth ties) and rows that are -inf
    past position 0 (scores -inf below depth 1), at budgets above 128."""
    B, L, V, K, N = 2, 6, 300, 8, 600
    x = torch.full((B, L, V), value, dtype=torch.bfloat16)
    x[:, 0, :] = torch.linspace(0, 3, V).to(torch.bfloat16)
    for tau in (1.0, 0.0):
        note("build level degenerate value=%g tau=%g" % (value, tau))
        g, _ = gpu_build(x, [1, 2], K, N, tau)
        o = oracle.build_tree(x, [1, 2], K, N, tau)
        assert_same_build(g, o)


@pytest.mark.parametrize("seed", range(16))
def test_build_random_shapes(seed):
    """Seeded random shapes: 1-8 requests, block sizes 1-32, vocabularies
    from 2 to 200,000 (every row-kernel variant, aligned or not), K up to 32,
    budgets up to 1,024 (the heap and the level selection on either side of
    their switch), draft temperatures 0, 1 and others, bf16 or f32 logits,
    some rows quantised to force ties."""
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 9))
    L = int(rng.integers(1, 33))
    V = int(rng.choice([int(rng.integers(2, 300)), int(rng.integers(300, 20000)),
                        int(rng.integers(20000, 200000))]))
    K = int(rng.integers(1, min(32, V) + 1))
    N = int(rng.choice([int(rng.integers(1, 72)), int(rng.integers(72, 160)),
                        int(rng.integers(160, 1025))]))
    tau = float(rng.choice([0.0, 1.0, float(rng.uniform(0.3, 2.0))]))
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    x = _logits(B, L, V, seed=600 + seed, sigma=float(rng.uniform(0.5, 4.0)), dtype=torch.float32,
                boost=float(rng.choice([0.0, 8.0])))
    if rng.random() < 0.3:
        x = torch.round(x)                         # ties
    x = x.to(dtype)
    roots = torch.as_tensor(rng.integers(0, V, size=B), dtype=torch.int32)
    note("build random seed=%d B=%d L=%d V=%d K=%d N=%d tau=%g %s" % (seed, B, L, V, K, N, tau, dtype))
    g, _ = gpu_build(x, roots, K, N, tau)
    o = oracle.build_tree(x, roots, K, N, tau)
    assert_same_build(g, o)
