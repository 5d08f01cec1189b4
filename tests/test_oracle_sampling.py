"""Pins for the float64 sampling-parameter reference (CPU only).

The processed row is pinned by closed forms (no truncation: the softmax of
logits / T; a hand-worked five-token example), by special cases (top-k 1 is
the lowest-index argmax; equal logits keep the lower index), by brute force
(the top-p set is the shortest rank prefix reaching the mass, found by trying
every prefix) and by an exact scale invariance. The logits-input accept is
pinned by the exact losslessness test of the accept on tiny vocabularies with
truncating parameters: every emitted token is distributed as the processed
target row. A planted top-p mistake must fail the hand-worked example.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import oracle.sampling
from test_oracle_accept import exact_distribution


@pytest.mark.parametrize("T", [1.0, 0.7, 2.0])
def test_no_truncation_is_the_softmax(T):
    rng = np.random.default_rng(1)
    l = rng.normal(0, 3, 600).astype(np.float32)
    p, kept, tie = oracle.sampling_filter(l, T, len(l), 1.0)
    assert len(kept) == len(l) and not tie
    assert np.max(np.abs(p - softmax(l.astype(np.float64) / T))) < 1e-15


def test_hand_worked_five_tokens():
    # logits 2, 1, 0, 0, -1 at temperature 1, top-k 3: ranks 0, 1, 2 (token 2
    # before token 3 on the tie); masses 1 : e^-1 : e^-2. top-p 0.8: the mass
    # before rank 1 is 1 / (1 + e^-1 + e^-2) = 0.665 < 0.8, before rank 2 it
    # is 0.910 >= 0.8, so tokens 0 and 1 are kept: 1/(1+e^-1), e^-1/(1+e^-1)
    l = np.array([2, 1, 0, 0, -1], np.float32)
    p, kept, _ = oracle.sampling_filter(l, 1.0, 3, 0.8)
    assert kept == [0, 1]
    want = np.array([1, math.exp(-1), 0, 0, 0]) / (1 + math.exp(-1))
    assert np.max(np.abs(p - want)) < 1e-15
    # temperature 0.5, top-k 4: masses 1 : e^-2 : e^-4 : e^-4; before rank 2
    # the mass is (1 + e^-2) / (1 + e^-2 + 2 e^-4) = 0.969 >= 0.95
    p, kept, _ = oracle.sampling_filter(l, 0.5, 4, 0.95)
    assert kept == [0, 1]
    want = np.array([1, math.exp(-2), 0, 0, 0]) / (1 + math.exp(-2))
    assert np.max(np.abs(p - want)) < 1e-15
    # top-p 0.97 keeps rank 2 (token 2, the lower index of the tie) as well
    p, kept, _ = oracle.sampling_filter(l, 0.5, 4, 0.97)
    assert kept == [0, 1, 2]
    want = np.array([1, math.exp(-2), math.exp(-4), 0, 0]) / (1 + math.exp(-2) + math.exp(-4))
    assert np.max(np.abs(p - want)) < 1e-15


def test_top_k_one_is_the_lowest_index_argmax():
    rng = np.random.default_rng(2)
    for _ in range(20):
        l = rng.integers(-3, 4, 50).astype(np.float32)   # many equal maxima
        p, kept, _ = oracle.sampling_filter(l, 1.0, 1, 0.9)
        assert kept == [oracle.argmax_lowest(l)] and p[kept[0]] == 1.0 and p.sum() == 1.0


def test_equal_logits_keep_the_lower_index_and_nan_is_never_kept():
    l = np.array([0, 5, 5, 1, 5, 5, np.nan, 9], np.float32)
    _, kept, _ = oracle.sampling_filter(l, 1.0, 3, 1.0)
    assert kept == [7, 1, 2]
    _, kept, _ = oracle.sampling_filter(np.array([0.0, -0.0, 0.0], np.float32), 1.0, 2, 1.0)
    assert kept == [0, 1]


@pytest.mark.parametrize("seed", range(6))
def test_top_p_set_is_the_shortest_prefix_reaching_the_mass(seed):
    rng = np.random.default_rng(10 + seed)
    V, k = 200, 30
    l = rng.normal(0, 2, V).astype(np.float32)
    T, top_p = float(rng.uniform(0.5, 1.5)), float(rng.uniform(0.3, 0.99))
    p, kept, tie = oracle.sampling_filter(l, T, k, top_p)
    order = sorted(range(V), key=lambda v: (-float(l[v]), v))[:k]
    w = [math.exp((float(l[v]) - float(l[order[0]])) / T) for v in order]
    n = next(n for n in range(1, k + 1) if math.fsum(w[:n]) / math.fsum(w) >= top_p)
    assert kept == order[:n]
    assert abs(p.sum() - 1) < 1e-15 and np.all(p[order[n:]] == 0)
    assert np.allclose(p[order[:n]], np.array(w[:n]) / math.fsum(w[:n]), rtol=1e-14, atol=0)


def test_scaling_logits_and_temperature_together_changes_nothing():
    l = np.random.default_rng(3).normal(0, 3, 500).astype(np.float32)
    a = oracle.sampling_filter(l, 0.8, 40, 0.9)
    b = oracle.sampling_filter(2 * l, 1.6, 40, 0.9)
    assert a[1] == b[1] and np.array_equal(a[0], b[0])


def _logit_rows(seed, K, V):
    rng = np.random.default_rng(seed)
    return (rng.normal(0, 1.5, (K + 1, V)).astype(np.float32),
            rng.normal(0, 1.5, (K, V)).astype(np.float32))


@pytest.mark.parametrize("K,V,k,top_p,T,seed", [(2, 5, 3, 0.9, 1.0, 0), (1, 6, 4, 0.8, 0.7, 1),
                                                (3, 4, 3, 0.95, 1.3, 2)])
def test_logits_accept_is_lossless_for_the_processed_target(K, V, k, top_p, T, seed):
    tl, dl = _logit_rows(seed, K, V)
    p = np.stack([oracle.sampling_filter(r, T, k, top_p)[0] for r in tl])
    q = np.stack([oracle.sampling_filter(r, T, k, top_p)[0] for r in dl])
    assert (p == 0).any() and (q == 0).any()  # the parameters do truncate

    def run(d, u):
        return oracle.accept_logits_request(tl, dl, d, u, 0, T, k, top_p)

    dist = exact_distribution(p, q, run)
    assert abs(sum(dist.values()) - 1) < 1e-12
    reach = np.zeros(K + 2)
    emit = np.zeros((K + 1, V))
    for out, w in dist.items():
        for i in range(out[0] + 1):
            reach[i] += w
            emit[i, out[1 + i]] += w
    for i in range(K + 1):
        assert np.max(np.abs(emit[i] - reach[i] * p[i])) < 1e-10
        if i < K:
            assert abs(reach[i + 1] - reach[i] * np.minimum(p[i], q[i]).sum()) < 1e-10


def test_planted_inclusive_top_p_fails_the_hand_worked_example(monkeypatch):
    """Discrimination check: counting rank r's own mass in the top-p test
    (keep r iff sum_{s <= r} P_s < top_p) must fail."""
    monkeypatch.setattr(oracle.sampling, "mass_before",
                        lambda e, r, z_k: math.fsum(e[:r + 1]) / z_k)
    with pytest.raises(AssertionError):
        test_hand_worked_five_tokens()


def test_logits_accept_flags_top_p_ties_only_in_used_rows():
    # target row 1 has a top-p decision exactly at the boundary (masses 1 : 1,
    # top_p 0.5); it is used only when the first draft is accepted
    V = 4
    tl = np.array([[5, 0, 0, 0], [1, 1, -9, -9], [0, 0, 0, 0]], np.float32)
    dl = np.array([[5, 0, 0, 0], [1, 1, -9, -9]], np.float32)
    draft = np.array([0, 0])
    acc = oracle.accept_logits_request(tl, dl, draft, np.array([0.1, 0.2, 0.3], np.float32),
                                       0, 1.0, 2, 0.5)
    assert acc["accept_len"] >= 1 and acc["tie_topp"]
    rej = oracle.accept_logits_request(tl, dl, np.array([1, 0]),
                                       np.array([0.99, 0.2, 0.3], np.float32), 0, 1.0, 2, 0.5)
    assert rej["accept_len"] == 0 and not rej["tie_topp"]
