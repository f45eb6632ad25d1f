"""Pins for the oracle's per-position log-softmax and top-K (CPU only).

Each test checks the oracle against something other than itself: libm,
numpy fp64 log-sum-exp, numpy's lexicographic sort, or a closed form.
Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees",
§3 (per-position marginals q_i), §4.3 (log space keeps the order), App. A
(restricted prefix set = per-position candidates).
"""
import math

import numpy as np
import pytest

import oracle

TWO44 = float(2 ** 44)


def _logsumexp64(x):
    x = np.asarray(x, np.float64)
    m = np.max(x)
    return m + math.log(np.sum(np.exp(x - m)))


def test_exp_fixed_special_values():
    assert oracle.exp_fixed(0.0) == 2 ** 44
    assert oracle.exp_fixed(float("-inf")) == 0
    assert oracle.exp_fixed(-50.0) == 0          # 2^44 e^-50 ~ 3e-8
    assert oracle.exp_fixed(-1e30) == 0


def test_exp_fixed_matches_libm():
    # Error budget, relative: degree-5 Taylor truncation of 2^f on |f| <= 1/2
    # ((ln2/2)^6/6! absolute, over 2^f >= 2^-1/2), the fp32 rounding of t = d*log2(e) (half an ulp of t, times
    # ln 2) and a few fp32 ulp of Horner rounding; the integer rounding adds 0.5.
    rng = np.random.default_rng(0)
    ds = np.concatenate([np.linspace(-31.0, 0.0, 4001), -rng.random(4000) * 31.0])
    worst = 0.0
    for d in ds.astype(np.float32):
        true = math.exp(float(d)) * TWO44
        got = oracle.exp_fixed(float(d))
        t = abs(float(d)) * 1.4426950408889634
        ulp_t = 2.0 ** (math.frexp(t)[1] - 24) if t > 0 else 0.0
        taylor = (0.5 * math.log(2)) ** 6 / 720 / math.sqrt(0.5)
        rel = taylor + 0.5 * ulp_t * math.log(2) + t * 2.0 ** -24 + 4 * 2.0 ** -24
        err = abs(got - true) - 0.5
        worst = max(worst, err / true)
        assert err <= rel * true, (d, got, true)
    assert worst > 1e-7  # the approximation is not accidentally libm itself


def test_log64_matches_libm():
    rng = np.random.default_rng(1)
    assert oracle.log64(1.0) == 0.0
    vals = np.concatenate([1.0 + rng.random(2000) * 1e-3, rng.random(2000) * 2.0 ** 20 + 1.0,
                           2.0 ** np.arange(0, 40), [math.sqrt(2.0), 151936.0, 32000.0]])
    for s in vals:
        ref = math.log(float(s))
        got = oracle.log64(float(s))
        assert abs(got - ref) <= 4e-16 * max(1.0, abs(ref)), (s, got, ref)


@pytest.mark.parametrize("V,sigma,dtype", [(64, 2.0, "f32"), (1000, 1.0, "f32"),
                                           (32000, 3.0, "bf16"), (4096, 10.0, "f32"),
                                           (151936, 3.0, "bf16")])
def test_lse_and_logprobs_match_fp64(V, sigma, dtype):
    import torch
    g = torch.Generator().manual_seed(V)
    x = torch.randn(V, generator=g) * sigma
    x[3] += 8.0
    row = x.to(torch.bfloat16) if dtype == "bf16" else x
    r = oracle.row_topk(row, 16, 1.0)
    xf = row.float().numpy().astype(np.float64)
    lse_ref = _logsumexp64(xf)
    assert abs((r["m"] + r["lse"]) - lse_ref) <= 1e-5 * max(1.0, abs(lse_ref))
    lp_ref = xf[r["tok"]] - lse_ref
    np.testing.assert_allclose(r["lp"], lp_ref, rtol=0, atol=1e-5 * max(1.0, abs(lse_ref)))
    assert r["flags"] == 0


def test_topk_order_matches_lexsort_with_ties():
    rng = np.random.default_rng(2)
    for trial in range(40):
        V = int(rng.integers(5, 300))
        x = rng.integers(-4, 4, size=V).astype(np.float32)   # many exact ties
        if trial % 3 == 0:
            x[rng.integers(0, V, size=3)] = -np.inf
        if trial % 5 == 0:
            x[rng.integers(0, V)] = np.nan
        K = int(rng.integers(1, min(V, 32) + 1))
        r = oracle.row_topk(x, K, 1.0)
        xs = np.where(np.isnan(x), -np.inf, x)
        ref = np.lexsort((np.arange(V), -xs))[:K]          # x desc, id asc
        np.testing.assert_array_equal(r["tok"], ref)
        assert r["flags"] == (1 if np.isnan(x).any() else 0)
        assert np.all(np.diff(r["lp"]) <= 0)


@pytest.mark.parametrize("V", [4, 64, 1000, 32000, 151936])
def test_all_equal_row_gives_minus_log_v(V):
    x = np.full(V, 1.25, np.float32)
    r = oracle.row_topk(x, min(V, 8), 1.0)
    assert r["S"] == V * 2 ** 44
    assert r["lse"] == np.float32(math.log(V))
    assert np.all(r["lp"] == -np.float32(math.log(V)))
    np.testing.assert_array_equal(r["tok"], np.arange(min(V, 8)))


def test_dominant_row_gives_zero_logprob():
    x = np.zeros(5000, np.float32)
    x[1234] = 60.0
    r = oracle.row_topk(x, 4, 1.0)
    assert r["S"] == 2 ** 44
    assert r["lp"][0] == 0.0 and r["tok"][0] == 1234
    assert np.all(r["lp"][1:] == np.float32(-60.0))


def test_temperature_scaling_rank_and_values():
    import torch
    g = torch.Generator().manual_seed(7)
    x = (torch.randn(3000, generator=g) * 3).to(torch.bfloat16).float().numpy()
    tau = 0.7
    r = oracle.row_topk(x, 16, tau)
    xs = x * np.float32(np.float32(1.0) / np.float32(tau))   # fp32 product, as specified
    ref = np.lexsort((np.arange(x.size), -xs))[:16]
    np.testing.assert_array_equal(r["tok"], ref)
    lse_ref = _logsumexp64(xs.astype(np.float64))
    np.testing.assert_allclose(r["lp"], xs[ref].astype(np.float64) - lse_ref, atol=1e-5)


def test_temperature_zero_is_argmax_with_tie_mass():
    x = np.zeros(100, np.float32)
    x[[5, 17, 60]] = 3.0          # three tied maxima share the mass equally
    x[40] = 2.9
    r = oracle.row_topk(x, 5, 0.0)
    np.testing.assert_array_equal(r["tok"], [5, 17, 60, 40, 0])
    assert r["S"] == 3 * 2 ** 44
    assert np.all(r["lp"][:3] == -np.float32(math.log(3)))
    assert np.all(np.isneginf(r["lp"][3:]))
    one = oracle.row_topk(np.array([0.0, 7.0, 1.0], np.float32), 3, 0.0)
    assert one["lp"][0] == 0.0 and np.all(np.isneginf(one["lp"][1:]))


def test_nan_and_all_minus_inf_rows():
    x = np.array([np.nan, 1.0, np.inf, -np.inf, 0.5], np.float32)
    r = oracle.row_topk(x, 3, 1.0)
    assert r["flags"] == 1
    np.testing.assert_array_equal(r["tok"], [1, 4, 0])    # NaN and +inf rank as -inf
    np.testing.assert_allclose(r["lp"][:2], np.array([1.0, 0.5]) - _logsumexp64([1.0, 0.5]),
                               atol=1e-6)
    assert np.isneginf(r["lp"][2])
    z = oracle.row_topk(np.full(10, -np.inf, np.float32), 4, 1.0)
    assert z["flags"] == 2
    assert np.all(np.isneginf(z["lp"]))
    np.testing.assert_array_equal(z["tok"], [0, 1, 2, 3])
