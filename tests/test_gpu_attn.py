"""GPU parity of ddtree_verify_attn against the oracle's fp64 tree attention.

Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees",
Abstract / §4.1 (one verify pass, ancestor-only mask), App. B (budgets up to
1024). Tolerance: |gpu - ref| <= 1e-3 + 2e-2 |ref| for bf16 and
1e-5 + 1e-5 |ref| for f32.

Small shapes compare every output row (ragged prefixes straddling key tiles,
trees with padding rows, GQA group sizes 1/4/8, row tiles with a ragged tail,
the split-KV path with requests of different lengths and with fewer
(request, kv-head) pairs than XCDs); the largest tree (T = 1025, split keys,
ragged prefixes and a ragged last row tile) and a batch of more requests than
XCDs compare every row as well. The last row tile of a (request, kv-head)
is mostly padding when T = N + 1 (the last node's heads); a tile of at most
32 rows has two waves take its keys by 32-key halves and merge: cases with
its valid rows whole, partly padding and all padding, with one key split
and with several, sit beside a case whose rows fill whole tiles. The full-size
workloads run in the launch configuration the benchmark times and compare
at least one row of every (request, kv-head, 128-row tile) unit of the
kernel, every row of one query head per (request, kv-head) where the
oracle's cost allows it (all but the 65,536-key workload, which compares
every row of one head for one kv-head per request), and each request's
first, last and padding rows.
The fp16 V copy (many row tiles per (request, kv-head)) runs on full trees
and on cut trees whose dropped nodes' K/V rows hold NaN, beside a request
whose prefix exceeds max_prefix_len (it converts its own tiles). Twelve
seeded random shapes (1-4 requests, GQA groups 1-8, budgets up to 399,
prefixes up to 2,500 keys, some above max_prefix_len, trees cut at random
with NaN in the dropped rows) cross the split, V-pass and last-tile cases.
Root-only trees (T = 1) are single-query decode attention; with no prefix
the output is the root's own V row, exactly.
Device-side checks: V values beyond the fp16 range and requests whose K/V
rows are outside the caches are reported in the status words.
"""
import numpy as np
import pytest
import torch

import oracle
from draft_tree_build_amd import api, synth
from gpu_util import DEV, check_attn, note

pytestmark = pytest.mark.gpu

ROWS_PER_TILE = 128   # query rows of one attention workgroup


@pytest.fixture(autouse=True, scope="module")
def _oracle_threads():
    """The oracle's attention rows are spread over the host's cores (the
    results do not depend on the thread count)."""
    with oracle.threads(oracle.host_cores()):
        yield


def _tree(B, L, V, K, N, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, L, V, generator=g) * 2
    return oracle.build_tree(x, list(range(B)), K, N, 1.0)


def _run(q, k, v, P, tree, T, max_prefix=None, offs=None):
    B, _, Hq, D = q.shape
    if offs is None:
        offs = synth.kv_offsets(torch.as_tensor(P, dtype=torch.int32), T)
    mp = int(max(max(P), 0)) if max_prefix is None else max_prefix
    code = 0 if q.dtype == torch.bfloat16 else 1
    ws = api.new_workspace(api.ddtree_verify_workspace_size(code, B, T, Hq, k.shape[1], D, mp), DEV)
    out = torch.full_like(q, 7.0, device=DEV)   # every row must be written
    status = torch.full((B,), -1, dtype=torch.int32, device=DEV)   # every word must be written
    api.ddtree_verify_attn(q.to(DEV), k.to(DEV), v.to(DEV), offs.to(DEV),
                           torch.as_tensor(P, dtype=torch.int32).to(DEV),
                           torch.from_numpy(tree["num_nodes"]).to(DEV),
                           torch.from_numpy(tree["mask"].view(np.int64)).to(DEV), mp, out, ws,
                           status_flags=status)
    torch.cuda.synchronize()
    return out.cpu(), offs, status.cpu().numpy()


def _ref(q, k, v, offs, P, tree, T, sel):
    Hq, Hkv, D = q.shape[2], k.shape[1], q.shape[3]
    return oracle.attn_rows(q, k, v, offs, P, tree["num_nodes"], tree["mask"], T, Hq, Hkv, D,
                            1.0 / np.sqrt(D), sel)


def _qkv(B, T, Hq, Hkv, P, seed, dtype=torch.bfloat16, D=128):
    g = torch.Generator().manual_seed(seed)
    total = sum(P) + B * T
    q = torch.randn(B, T, Hq, D, generator=g).to(dtype)
    k = torch.randn(total, Hkv, D, generator=g).to(dtype)
    v = torch.randn(total, Hkv, D, generator=g).to(dtype)
    return q, k, v


def _all_rows(B, T, Hq):
    return [(b, i, h) for b in range(B) for i in range(T) for h in range(Hq)]


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
    (1, 6, 40, 4, 63, 8, 2, [500]),             # R = 256: two full row tiles, no tail rows
    (2, 2, 20, 2, 32, 8, 2, [300, 40]),         # 4-row last tile, all padding (7-node trees)
    (2, 2, 20, 2, 32, 8, 2, [3000, 40]),        # the same with split keys
]


@pytest.mark.parametrize("B,L,V,K,N,Hq,Hkv,P", SMALL)
def test_attn_bf16_all_rows(B, L, V, K, N, Hq, Hkv, P):
    T = N + 1
    tree = _tree(B, L, V, K, N, seed=N + Hq)
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=B * 1000 + N)
    note("attn bf16 B=%d T=%d Hq=%d Hkv=%d P=%s" % (B, T, Hq, Hkv, P))
    out, offs, st = _run(q, k, v, P, tree, T)
    sel = _all_rows(B, T, Hq)
    check_attn(out, _ref(q, k, v, offs, P, tree, T, sel), sel, torch.bfloat16)
    for b in range(B):
        assert torch.all(out[b, tree["num_nodes"][b]:] == 0)
    assert np.all(st == 0), st


def test_attn_bf16_largest_tree_all_rows():
    """N = 1024 (T = 1025, 17 mask words): split keys, ragged prefixes that
    straddle key tiles, 33 row tiles with a 4-row last tile."""
    B, L, V, K, N, Hq, Hkv, P = 2, 16, 80, 8, 1024, 32, 8, [3001, 1703]
    T = N + 1
    tree = _tree(B, L, V, K, N, seed=1025)
    assert int(tree["num_nodes"].min()) == T            # full trees
    assert api.ddtree_verify_workspace_size(0, B, T, Hq, Hkv, 128, max(P)) > 256   # keys split
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=1025)
    note("attn bf16 T=1025 all rows P=%s" % P)
    out, offs, st = _run(q, k, v, P, tree, T)
    sel = _all_rows(B, T, Hq)
    check_attn(out, _ref(q, k, v, offs, P, tree, T, sel), sel, torch.bfloat16)
    assert np.all(st == 0), st


def test_attn_bf16_batch_beyond_xcds_all_rows():
    """12 requests (more than the 8 XCDs the grid deals units to) with
    unequal prefixes, some of them short of a key tile, and padded trees."""
    B, L, V, K, N, Hq, Hkv = 12, 6, 40, 4, 64, 32, 8
    T = N + 1
    rng = np.random.default_rng(12)
    P = [int(x) for x in rng.integers(0, 3000, size=B)]
    P[3], P[7] = 0, 33
    tree = _tree(B, L, V, K, N, seed=12)
    tree["num_nodes"][5] = 17            # a short tree: rows 17.. are padding
    tree["mask"][5, 17:] = 0
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=12)
    note("attn bf16 B=12 all rows P=%s" % P)
    out, offs, st = _run(q, k, v, P, tree, T)
    sel = _all_rows(B, T, Hq)
    check_attn(out, _ref(q, k, v, offs, P, tree, T, sel), sel, torch.bfloat16)
    assert torch.all(out[5, 17:] == 0)
    assert np.all(st == 0), st


def test_attn_bf16_last_tile_partly_padding():
    """g = 1 and T = 160: a 32-row last tile past one full row tile, one
    node per row. Request 0's tree is cut to 140 nodes, so 12 of those rows
    are valid and 20 are padding; request 0's keys are split, request 1's
    are not."""
    B, L, V, K, N, Hq, Hkv, P = 2, 7, 40, 2, 159, 4, 4, [3000, 200]
    T = N + 1
    tree = _tree(B, L, V, K, N, seed=160)
    assert int(tree["num_nodes"].min()) == T
    tree["num_nodes"][0] = 140
    tree["mask"][0, 140:] = 0
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=160)
    note("attn bf16 last tile partly padding P=%s" % P)
    out, offs, st = _run(q, k, v, P, tree, T)
    sel = _all_rows(B, T, Hq)
    check_attn(out, _ref(q, k, v, offs, P, tree, T, sel), sel, torch.bfloat16)
    assert torch.all(out[0, 140:] == 0)
    assert np.all(st == 0), st


def test_attn_bf16_reference_moves_all_rows():
    """Scores that rise along the prefix (K rows scaled up to 6x, so the
    exponentials' running reference has to move on many key tiles), one key
    near the end of a prefix far above all others (a late jump of ~50 in
    log2 units), a tree-only request and a split-KV request: every row."""
    B, L, V, K, N, Hq, Hkv, P = 3, 6, 60, 6, 64, 32, 8, [2000, 1300, 0]
    T = N + 1
    tree = _tree(B, L, V, K, N, seed=77)
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=77)
    kf = k.float()
    offs = synth.kv_offsets(torch.as_tensor(P, dtype=torch.int32), T)
    for b in range(2):
        o = int(offs[b])
        ramp = 1.0 + 5.0 * torch.arange(P[b], dtype=torch.float32) / P[b]
        kf[o:o + P[b]] *= ramp[:, None, None]
    g = Hq // Hkv
    qm = q.float()[1].reshape(T, Hkv, g, 128).mean(dim=(0, 2))      # [Hkv, D]
    kf[int(offs[1]) + P[1] - 3] = 3.0 * qm / qm.norm(dim=1, keepdim=True) * 11.0
    kf[int(offs[1]) + P[1] - 5, 0] = 3.0 * q.float()[1, 5, 0]    # row 5, head 0: +~49 (log2)
    k = kf.to(torch.bfloat16)
    note("attn bf16 reference moves P=%s" % P)
    out, offs2, st = _run(q, k, v, P, tree, T, offs=offs)
    sel = _all_rows(B, T, Hq)
    check_attn(out, _ref(q, k, v, offs2, P, tree, T, sel), sel, torch.bfloat16)
    assert np.all(st == 0), st


def test_attn_bf16_preconverted_v():
    """33 row tiles per (request, kv-head) (T = 513, g = 8): V goes to fp16
    in a pass of its own before the main kernel. A request whose prefix
    exceeds max_prefix_len converts its own tiles; a request whose K/V rows
    end past the caches gets zero rows and the BAD_KV bit. Every row of one
    query head per kv-head, and each request's last rows of every head."""
    B, L, V, K, N, Hq, Hkv = 3, 6, 60, 6, 512, 64, 8
    T = N + 1
    P = [1500, 700, 2100]
    max_prefix = 1600                     # request 2 is longer
    tree = _tree(B, L, V, K, N, seed=513)
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=513)
    ws_pre = api.ddtree_verify_workspace_size(0, B, T, Hq, Hkv, 128, max_prefix)
    tiles = -(-max_prefix // 64) + -(-T // 64)
    assert ws_pre >= B * Hkv * tiles * 64 * 128 * 2      # the fp16 copy is planned
    offs = synth.kv_offsets(torch.as_tensor(P, dtype=torch.int32), T)
    total = k.shape[0]
    offs_bad = offs.clone()
    offs_bad[1] = total - P[1] - T + 1    # one row past the end
    note("attn bf16 preconverted V P=%s max_prefix=%d" % (P, max_prefix))
    out, offs2, st = _run(q, k, v, P, tree, T, max_prefix=max_prefix, offs=offs_bad)
    g = Hq // Hkv
    heads = [hk * g + (hk * 3) % g for hk in range(Hkv)]
    sel = [(b, i, h) for b in range(B) for i in range(T) for h in heads]
    sel += [(b, i, h) for b in range(B) for i in range(T - 3, T) for h in range(Hq)]
    sel = sorted(set(sel))
    check_attn(out, _ref(q, k, v, offs2, P, tree, T, sel), sel, torch.bfloat16)
    assert torch.all(out[1] == 0)
    assert st.tolist() == [0, 8, 0], st


def test_attn_bf16_preconverted_v_cut_trees():
    """The fp16 V pass on cut trees: 33 row tiles (T = 513, g = 8), a prefix
    that fills its key tiles exactly, a tree-only request, and a ragged
    prefix. Requests 0 and 2 keep 300 and 65 of their nodes, and the K/V
    rows of the dropped nodes hold NaN: no kernel may read them (the pass
    writes zeros for keys a tile does not hold). Every row of one query head
    per kv-head, and each request's rows around num_nodes for every head."""
    B, L, V, K, N, Hq, Hkv = 3, 6, 60, 6, 512, 64, 8
    T = N + 1
    P = [640, 0, 1333]
    max_prefix = 1400
    tree = _tree(B, L, V, K, N, seed=514)
    cut = {0: 300, 2: 65}
    for b, n in cut.items():
        tree["num_nodes"][b] = n
        tree["mask"][b, n:] = 0
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=514)
    offs = synth.kv_offsets(torch.as_tensor(P, dtype=torch.int32), T)
    for b, n in cut.items():
        o = int(offs[b]) + P[b]
        k[o + n:o + T] = float("nan")
        v[o + n:o + T] = float("nan")
    note("attn bf16 preconverted V, cut trees P=%s max_prefix=%d" % (P, max_prefix))
    out, offs2, st = _run(q, k, v, P, tree, T, max_prefix=max_prefix, offs=offs)
    g = Hq // Hkv
    heads = [hk * g + (hk * 5 + 1) % g for hk in range(Hkv)]
    sel = [(b, i, h) for b in range(B) for i in range(T) for h in heads]
    for b in range(B):
        n = int(tree["num_nodes"][b])
        sel += [(b, i, h) for i in range(max(n - 2, 0), min(n + 2, T)) for h in range(Hq)]
    sel = sorted(set(sel))
    check_attn(out, _ref(q, k, v, offs2, P, tree, T, sel), sel, torch.bfloat16)
    for b, n in cut.items():
        assert torch.all(out[b, n:] == 0)
    assert np.all(st == 0), st


def _random_case(seed):
    """One seeded shape: 1-4 requests, GQA group 1-8, a tree budget and
    prefixes that may or may not split keys or reach the fp16 V pass, a
    max_prefix_len that some prefixes may exceed, and trees cut at random
    with NaN in the K/V rows of the dropped nodes."""
    rng = np.random.default_rng(seed)
    big = seed % 3 == 0           # 17 or more row tiles: the fp16 V pass
    B = int(rng.integers(1, 5))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    g = 8 if big else int(rng.choice([1, 2, 4, 8]))
    N = int(rng.integers(256, 400)) if big else int(rng.integers(1, 400))
    L = int(rng.integers(2, 9))
    K = int(rng.integers(2, 7))
    P = [int(x) for x in rng.integers(0, 2500, size=B)]
    mp = max(P)
    if rng.random() < 0.4 and mp > 64:
        mp = int(rng.integers(mp // 2, mp))       # some prefixes exceed it
    cuts = {b: int(rng.integers(0, N + 2)) for b in range(B) if rng.random() < 0.4}
    return dict(B=B, Hkv=Hkv, Hq=Hkv * g, N=N, L=L, K=K, P=P, max_prefix=mp, cuts=cuts)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (32, 8), (64, 8)])
def test_attn_root_only_trees(Hq, Hkv, dtype):
    """T = 1 (no drafted node): single-query decode attention over the prefix
    and the root itself, with prefixes of 0, 1, 63 and 4,100 keys (split
    keys); with no prefix the output is the root's own V row."""
    B, T, P = 4, 1, [0, 1, 63, 4100]
    tree = dict(num_nodes=np.ones(B, np.int32), mask=np.ones((B, 1, 1), np.uint64))
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=Hq + Hkv, dtype=dtype, D=128)
    note("attn root-only Hq=%d Hkv=%d %s" % (Hq, Hkv, dtype))
    out, offs, st = _run(q, k, v, P, tree, T)
    sel = _all_rows(B, T, Hq)
    check_attn(out, _ref(q, k, v, offs, P, tree, T, sel), sel, dtype)
    g = Hq // Hkv
    root = int(offs[0]) + P[0]
    want = v[root].float().repeat_interleave(g, dim=0)          # [Hq, D]
    # one key of weight exactly 1: V itself (bf16 V passes fp16 and back
    # unchanged outside the fp16 subnormal range)
    assert torch.allclose(out[0, 0].float(), want, atol=1e-6, rtol=0)
    assert np.all(st == 0), st


@pytest.mark.parametrize("seed", range(12))
def test_attn_bf16_random_shapes(seed):
    """Seeded random shapes across the plan's branches (splits, the fp16 V
    pass and its fallback, last row tiles of any size, cut trees): every row
    of one query head per (request, kv-head), every head of each request's
    rows around num_nodes, and 256 random rows."""
    c = _random_case(1000 + seed)
    B, Hq, Hkv, N, P = c["B"], c["Hq"], c["Hkv"], c["N"], c["P"]
    T = N + 1
    tree = _tree(B, c["L"], 40, c["K"], N, seed=2000 + seed)
    for b, n in c["cuts"].items():
        n = min(n, int(tree["num_nodes"][b]))
        tree["num_nodes"][b] = n
        tree["mask"][b, n:] = 0
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=3000 + seed)
    offs = synth.kv_offsets(torch.as_tensor(P, dtype=torch.int32), T)
    for b in range(B):
        n = int(tree["num_nodes"][b])
        o = int(offs[b]) + P[b]
        k[o + n:o + T] = float("nan")
        v[o + n:o + T] = float("nan")
    note("attn bf16 random seed=%d B=%d T=%d Hq=%d Hkv=%d P=%s max_prefix=%d num_nodes=%s" % (
        seed, B, T, Hq, Hkv, P, c["max_prefix"], list(tree["num_nodes"])))
    out, offs2, st = _run(q, k, v, P, tree, T, max_prefix=c["max_prefix"], offs=offs)
    g = Hq // Hkv
    rng = np.random.default_rng(seed)
    sel = set()
    for b in range(B):
        for hk in range(Hkv):
            h = hk * g + int(rng.integers(g))
            sel.update((b, i, h) for i in range(T))
        n = int(tree["num_nodes"][b])
        sel.update((b, i, h) for i in range(max(n - 2, 0), min(n + 2, T)) for h in range(Hq))
    for _ in range(256):
        sel.add((int(rng.integers(B)), int(rng.integers(T)), int(rng.integers(Hq))))
    sel = sorted(sel)
    check_attn(out, _ref(q, k, v, offs2, P, tree, T, sel), sel, torch.bfloat16)
    for b in range(B):
        assert torch.all(out[b, int(tree["num_nodes"][b]):] == 0)
    assert np.all(st == 0), st


@pytest.mark.parametrize("D", [32, 64, 128])
def test_attn_f32_all_rows(D):
    B, L, V, K, N, Hq, Hkv, P = 2, 4, 30, 4, 8, 4, 2, [16, 3]
    T = N + 1
    tree = _tree(B, L, V, K, N, seed=D)
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=D, dtype=torch.float32, D=D)
    note("attn f32 D=%d" % D)
    out, offs, st = _run(q, k, v, P, tree, T)
    sel = _all_rows(B, T, Hq)
    check_attn(out, _ref(q, k, v, offs, P, tree, T, sel), sel, torch.float32)
    assert np.all(st == 0), st


def test_attn_repeatable_split_counters():
    """Two split-KV calls on one workspace give identical bits (partials rewritten)."""
    B, L, V, K, N, Hq, Hkv, P = 1, 16, 80, 8, 64, 32, 8, [3000]
    T = N + 1
    tree = _tree(B, L, V, K, N, seed=1)
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=2)
    note("attn split twice")
    a, _, _ = _run(q, k, v, P, tree, T)
    b, _, _ = _run(q, k, v, P, tree, T)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("P", [[2048, 700], [100, 40]])   # split keys / one split
def test_attn_v_range_status(P):
    """bf16 V enters the P.V product as fp16: 65280 (the largest bf16 value
    below the fp16 limit) is exact and matches the oracle; 65536 (which is
    where 65504 rounds in bf16) and 1e5 overflow fp16, and the request that
    holds them is flagged DDTREE_STATUS_OUT_NONFINITE while the other
    request's rows still match."""
    B, L, V, K, N, Hq, Hkv = 2, 4, 30, 4, 20, 32, 8
    T = N + 1
    tree = _tree(B, L, V, K, N, seed=5)
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=5)
    offs = synth.kv_offsets(torch.as_tensor(P, dtype=torch.int32), T)
    v[int(offs[0]) + 3, 2, 7] = 65280.0                  # request 0: in range
    v[int(offs[0]) + P[0] + 1, 5, 100] = -65280.0        # (a tree row, node 1)
    note("attn V range: in range P=%s" % P)
    out, _, st = _run(q, k, v, P, tree, T)
    sel = _all_rows(B, T, Hq)
    check_attn(out, _ref(q, k, v, offs, P, tree, T, sel), sel, torch.bfloat16)
    assert np.all(st == 0), st
    for big in (65504.0, 1e5):
        v2 = v.clone()
        v2[int(offs[1]) + 1, 0, 0] = big                 # request 1, a prefix row of kv-head 0
        assert abs(float(v2[int(offs[1]) + 1, 0, 0])) >= 65536
        note("attn V range: %g P=%s" % (big, P))
        out, _, st = _run(q, k, v2, P, tree, T)
        assert st[0] == 0 and st[1] == api.STATUS_OUT_NONFINITE, st
        sel0 = _all_rows(1, T, Hq)
        check_attn(out, _ref(q, k, v2, offs, P, tree, T, sel0), sel0, torch.bfloat16)


@pytest.mark.parametrize("N", [20, 32])   # one row tile / a full tile and a 4-row one
def test_attn_bad_kv_rows_zero_and_flagged(N):
    """Requests whose K/V rows are not inside the caches (a negative offset, a
    negative prefix, a region past the last row) read nothing: their rows are
    zeros and DDTREE_STATUS_BAD_KV is set; the valid request matches. Every
    buffer is in bounds: the device check keeps the kernel from reading the
    described rows at all."""
    B, L, V, K, Hq, Hkv = 4, 4, 30, 4, 32, 8
    T = N + 1
    P = [300, 300, 300, 300]
    tree = _tree(B, L, V, K, N, seed=6)
    q, k, v = _qkv(B, T, Hq, Hkv, P, seed=6)
    total = k.shape[0]
    offs = synth.kv_offsets(torch.as_tensor(P, dtype=torch.int32), T)
    P_bad = list(P)
    offs[0] = -5                     # negative offset
    P_bad[2] = -1                    # negative prefix
    offs[3] = total - P[3] - T + 1   # one row past the caches
    for dtype in (torch.bfloat16, torch.float32):
        note("attn bad kv rows dtype=%s" % dtype)
        qq, kk, vv = (t.to(dtype) for t in (q, k, v))
        out, _, st = _run(qq, kk, vv, P_bad, tree, T, max_prefix=max(P), offs=offs)
        assert list(st) == [api.STATUS_BAD_KV, 0, api.STATUS_BAD_KV, api.STATUS_BAD_KV], st
        for b in (0, 2, 3):
            assert torch.all(out[b] == 0)
        sel = [(1, i, h) for i in range(T) for h in range(Hq)]
        ref = _ref(qq, kk, vv, offs, P_bad, tree, T, sel)
        check_attn(out, ref, sel, dtype)
        # the oracle reads the same rule: the bad requests' rows are zeros
        sel_bad = [(b, i, 3) for b in (0, 2, 3) for i in (0, T - 1)]
        assert np.all(_ref(qq, kk, vv, offs, P_bad, tree, T, sel_bad) == 0)


def _unit_rows(w, tree, rng):
    """At least one row of every (request, kv-head, 128-row tile) unit, and
    the first, last and (when present) first padding row of every request."""
    g = w.Hq // w.Hkv
    R = w.T * g
    sel = []
    for b in range(w.batch):
        nn = int(tree["num_nodes"][b])
        for hk in range(w.Hkv):
            for t0 in range(0, R, ROWS_PER_TILE):
                r = int(rng.integers(t0, min(t0 + ROWS_PER_TILE, R)))
                node, j = divmod(r, g)
                sel.append((b, node, hk * g + j))
        for i in sorted({0, nn - 1} | ({nn} if nn < w.T else set())):
            sel += [(b, i, 0), (b, i, w.Hq - 1)]
    return sel


def _head_rows(w, tree, pairs):
    """Every node's row of one query head for each (request, kv-head) pair."""
    g = w.Hq // w.Hkv
    return [(b, i, hk * g + (b + hk) % g) for (b, hk) in pairs for i in range(w.T)]


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_attn_full_size_workloads(name):
    w = synth.WORKLOADS[name]
    x, _ = synth.drafter_logits(w)
    roots = synth.root_tokens(w)
    tree = oracle.build_tree(x, roots, w.K, w.N, w.taus[0])
    P = synth.prefix_lengths(w)
    q, k, v = synth.qkv(w, P)
    note("attn workload %s rows=%d" % (name, k.shape[0]))
    out, offs, st = _run(q, k, v, P.numpy(), tree, w.T, max_prefix=w.prefix[1])
    assert np.all(st == 0), st
    rng = np.random.default_rng(0)
    if w.prefix[1] <= 2048:       # small: every row
        sel = _all_rows(w.batch, w.T, w.Hq)
    else:
        sel = _unit_rows(w, tree, rng)
        if w.prefix[1] < 65536:
            pairs = [(b, hk) for b in range(w.batch) for hk in range(w.Hkv)]
        else:
            pairs = [(b, (3 * b + 1) % w.Hkv) for b in range(w.batch)]
        sel += _head_rows(w, tree, pairs)
    ref = _ref(q, k, v, offs, P.numpy(), tree, w.T, sel)
    check_attn(out, ref, sel, q.dtype)
