"""Pins for the oracle's acceptance at target temperature > 0 (CPU only).

Page: "Accelerating Speculative Decoding with Block Diffusion Draft Trees",
§4.1: the tree is walked with the target's decoding rule; at temperature > 0
that rule is a sample of the target's softmax. The uniform comes from
Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
as 1, 2, 3", SC 2011).
Pins: the published Philox4x32-10 known-answer vectors; the empirical token
frequencies against the float softmax (chi-square); exact special cases
(one finite logit, no finite logit, tokens far below the maximum); the
temperature as a rescaling of the logits; and the losslessness of the walk
(a tree that holds the sampled path is followed to its end).
"""
import numpy as np
import pytest
import torch

import oracle


@pytest.mark.parametrize("ctr,key,want", [
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
])
def test_philox_known_answers(ctr, key, want):
    np.testing.assert_array_equal(oracle.philox4x32_10(ctr, key), np.array(want, np.uint32))


def test_sample_frequencies_follow_softmax():
    x = np.array([1.0, 0.5, -0.25, 2.0, 0.0, -1.5], np.float32)
    p = np.exp(x.astype(np.float64) - x.max())
    p /= p.sum()
    n = 20000
    counts = np.bincount([oracle.sample_row(x, 1.0, seed=11, offset=k) for k in range(n)],
                         minlength=x.size)
    chi2 = float(((counts - n * p) ** 2 / (n * p)).sum())
    assert chi2 < 25.0, (counts, n * p)          # 5 degrees of freedom: p-value ~ 1e-4


def test_sample_special_cases():
    row = np.full(50, -np.inf, np.float32)
    row[17] = 3.0
    assert {oracle.sample_row(row, 1.0, 5, k) for k in range(200)} == {17}
    assert oracle.sample_row(np.full(9, -np.inf, np.float32), 1.0, 5, 0) == 0
    nan_row = row.copy()
    nan_row[3] = np.nan                            # NaN is ranked as -inf
    assert {oracle.sample_row(nan_row, 1.0, 5, k) for k in range(200)} == {17}
    far = np.zeros(8, np.float32)
    far[2] = -40.0                                 # e^-40 < 2^-45: its fixed-point weight is 0
    assert 2 not in {oracle.sample_row(far, 1.0, 9, k) for k in range(3000)}


def test_sample_temperature_rescales_logits():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(300).astype(np.float32)
    for k in range(100):
        assert oracle.sample_row(x, 0.5, 3, k) == oracle.sample_row(2.0 * x, 1.0, 3, k)


def test_sample_counter_layout():
    """Node i of request b uses counter (i, b, offset): the same row drawn as
    another node or request gives another (independent) token sequence."""
    x = np.zeros(1000, np.float32)
    a = [oracle.sample_row(x, 1.0, 7, k, b=0, i=1) for k in range(50)]
    b = [oracle.sample_row(x, 1.0, 7, k, b=1, i=1) for k in range(50)]
    c = [oracle.sample_row(x, 1.0, 7, k, b=0, i=2) for k in range(50)]
    assert a != b and a != c


def test_accept_sample_follows_sampled_path():
    """A chain tree whose every node carries the token the target samples
    after its parent is accepted to its end; the bonus is the sample at the
    leaf (losslessness: the committed tokens are the target's own samples)."""
    rng = np.random.default_rng(4)
    L, V, T = 5, 40, 6
    logits = torch.from_numpy(rng.standard_normal((1, T, V)).astype(np.float32))
    seed, offset = 21, 9
    tokens = np.full((1, T), -1, np.int32)
    parents = np.full((1, T), -1, np.int32)
    tokens[0, 0] = 0
    for i in range(1, T):
        parents[0, i] = i - 1
        tokens[0, i] = oracle.sample_row(logits[0, i - 1].numpy(), 1.0, seed, offset, b=0, i=i - 1)
    out = oracle.accept_sample(logits, tokens, parents, np.array([T], np.int32), L, 1.0, seed, offset)
    assert out["accept_len"][0] == L
    np.testing.assert_array_equal(out["accepted"][0], tokens[0, 1:])
    np.testing.assert_array_equal(out["accepted_nodes"][0], np.arange(1, T))
    assert out["bonus"][0] == oracle.sample_row(logits[0, T - 1].numpy(), 1.0, seed, offset, b=0, i=T - 1)
    # a different draw leaves the chain at the first mismatch
    out2 = oracle.accept_sample(logits, tokens, parents, np.array([T], np.int32), L, 1.0, seed,
                                offset + 1)
    n = out2["accept_len"][0]
    assert out2["bonus"][0] == out2["target_tokens"][0, n]
