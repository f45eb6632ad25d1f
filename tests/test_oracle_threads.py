"""The oracle's results do not depend on its thread count (CPU only).

The batch-level oracle calls spread independent units (drafter rows and
requests, query rows, target rows) over OpenMP threads; each unit runs the
same serial code, so one thread and several give the same bits. Also the
attention's reading for requests whose K/V rows are outside the caches:
their rows are zeros, the other requests' rows are unchanged.
"""
import numpy as np
import torch

import oracle


def _inputs(seed=3):
    g = torch.Generator().manual_seed(seed)
    B, L, V, K, N, Hq, Hkv, D = 3, 5, 300, 4, 40, 8, 2, 32
    T = N + 1
    x = (torch.randn(B, L, V, generator=g) * 2).to(torch.bfloat16)
    roots = [1, 2, 3]
    P = np.array([50, 0, 130], np.int32)
    offs = np.array([0, 50 + T, 50 + 2 * T], np.int64)
    total = int(P.sum()) + B * T
    q = torch.randn(B, T, Hq, D, generator=g).to(torch.bfloat16)
    k = torch.randn(total, Hkv, D, generator=g).to(torch.bfloat16)
    v = torch.randn(total, Hkv, D, generator=g).to(torch.bfloat16)
    tl = (torch.randn(B, T, V, generator=g) * 3).to(torch.bfloat16)
    return dict(B=B, L=L, V=V, K=K, N=N, T=T, Hq=Hq, Hkv=Hkv, D=D, x=x, roots=roots, P=P,
                offs=offs, q=q, k=k, v=v, tl=tl)


def _round(a):
    t = oracle.build_tree(a["x"], a["roots"], a["K"], a["N"], 1.0)
    sel = [(b, i, h) for b in range(a["B"]) for i in range(a["T"]) for h in range(a["Hq"])]
    at = oracle.attn_rows(a["q"], a["k"], a["v"], a["offs"], a["P"], t["num_nodes"], t["mask"],
                          a["T"], a["Hq"], a["Hkv"], a["D"], 0.17, sel)
    ac = oracle.accept(a["tl"], None, t["tokens"], t["parents"], t["num_nodes"], a["L"])
    sa = oracle.accept_sample(a["tl"], t["tokens"], t["parents"], t["num_nodes"], a["L"], 0.8,
                              7, 3)
    return t, at, ac, sa


def test_thread_count_does_not_change_results():
    a = _inputs()
    assert oracle.get_threads() == 1
    ref = _round(a)
    for n in (2, 5):
        with oracle.threads(n):
            assert oracle.get_threads() == n
            got = _round(a)
        for r, g in zip(ref, got):
            if isinstance(r, dict):
                for key in r:
                    if r[key] is not None:
                        np.testing.assert_array_equal(np.asarray(r[key]), np.asarray(g[key]),
                                                      err_msg=key)
            else:
                np.testing.assert_array_equal(r.view(np.uint64), g.view(np.uint64))
    assert oracle.get_threads() == 1


def test_attention_rows_of_requests_outside_the_caches_are_zero():
    a = _inputs(5)
    t = oracle.build_tree(a["x"], a["roots"], a["K"], a["N"], 1.0)
    sel = [(b, i, h) for b in range(a["B"]) for i in (0, 3, a["T"] - 1) for h in range(a["Hq"])]
    base = oracle.attn_rows(a["q"], a["k"], a["v"], a["offs"], a["P"], t["num_nodes"], t["mask"],
                            a["T"], a["Hq"], a["Hkv"], a["D"], 0.17, sel)
    assert np.all(np.abs(base).sum(axis=1) > 0)       # every request valid: rows are not zero
    total = a["k"].shape[0]
    for b_bad, offs_b, P_b in ((0, -1, 50), (1, 50 + a["T"], -2),
                               (2, total - 130 - a["T"] + 1, 130)):
        offs, P = a["offs"].copy(), a["P"].copy()
        offs[b_bad], P[b_bad] = offs_b, P_b
        got = oracle.attn_rows(a["q"], a["k"], a["v"], offs, P, t["num_nodes"], t["mask"],
                               a["T"], a["Hq"], a["Hkv"], a["D"], 0.17, sel)
        for s, (b, _, _) in enumerate(sel):
            if b == b_bad:
                assert np.all(got[s] == 0)
            else:
                np.testing.assert_array_equal(got[s], base[s])
