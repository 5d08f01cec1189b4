"""Pins for the float64 accept reference (CPU only).

The central pin is exact: on a tiny vocabulary the reference is treated as a
black box, every draft sequence is enumerated with its probability, and the
uniforms are integrated exactly (the outputs are piecewise constant in each
uniform, so the pieces are located by scanning and bisection). The resulting
distribution must satisfy the losslessness the pages state for rejection
sampling: the token emitted at a reached position is distributed as the target
row, and the per-position acceptance probability is sum_v min(p, q)
(Leviathan et al., Corollary 3.6, cited by the Uno summary).
"""
import json
import os

import numpy as np
import pytest

import oracle
from verify_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dist(rng, V, floor=0.05):
    w = rng.random(V) + floor
    return w / w.sum()


def _rows(seed, K, V):
    """Full-support p [K+1, V] and q [K, V] whose residual pieces are all
    either empty or wider than 1/200 of their row's mass."""
    rng = np.random.default_rng(seed)
    while True:
        p = np.stack([_dist(rng, V) for _ in range(K + 1)])
        q = np.stack([_dist(rng, V) for _ in range(K)])
        ok = True
        for i in range(K):
            r = np.maximum(p[i] - q[i], 0)
            nz = r[r > 0]
            if len(nz) == 0 or nz.min() / nz.sum() < 5e-3 or np.min(np.abs(p[i] - q[i])) < 1e-3:
                ok = False
        if ok:
            return p, q


def _scan_last_uniform(call, grid=1024):
    """Pieces of [0, 1) on which call(u_last) is constant: (length, output)."""
    us = (np.arange(grid) + 0.5) / grid
    outs = [call(u) for u in us]
    cuts = [0.0]
    for a in range(grid - 1):
        if outs[a] != outs[a + 1]:
            lo, hi = us[a], us[a + 1]
            for _ in range(60):
                mid = 0.5 * (lo + hi)
                if call(mid) == outs[a]:
                    lo = mid
                else:
                    hi = mid
            cuts.append(hi)
    cuts.append(1.0)
    vals = [outs[0]] + [outs[a + 1] for a in range(grid - 1) if outs[a] != outs[a + 1]]
    return [(cuts[n + 1] - cuts[n], vals[n]) for n in range(len(vals))]


def exact_distribution(p, q, run=None):
    """{(accept_len, out_tokens...): probability} of the reference's output
    when d_i ~ q_i independently and every uniform ~ U[0, 1). run(d, u)
    calls the reference under test (default: accept_request on p, q)."""
    K, V = q.shape
    if run is None:
        def run(d, u):
            return oracle.accept_request(p, q, d, u, 0)
    dist = {}
    for d in np.ndindex(*([V] * K)):
        d = np.array(d)
        wd = np.prod([q[i, d[i]] for i in range(K)])
        if wd == 0:
            continue
        a = [min(1.0, p[i, d[i]] / q[i, d[i]]) for i in range(K)]
        # the accept threshold sits exactly at min(1, p/q)
        for i in range(K):
            # (position i is reached with u = 0 before it unless an earlier
            # draft has target probability 0)
            if 0 < a[i] < 1 and all(a[s] > 0 for s in range(i)):
                for u_i, want in ((a[i] * (1 - 1e-9), True), (a[i] * (1 + 1e-9), False)):
                    u = np.zeros(K + 1)
                    u[i] = u_i
                    r = run(d, u)
                    assert (r["accept_len"] > i) == want
        for j in range(K + 1):
            w = wd
            u = np.zeros(K + 1)
            for i in range(j):
                w *= a[i]
                u[i] = a[i] / 2
            if j < K:
                w *= 1 - a[j]
                u[j] = (a[j] + 1) / 2
            if w == 0:
                continue

            def call(ul, u=u):
                uu = u.copy()
                uu[K] = ul
                r = run(d, uu)
                return (r["accept_len"],) + tuple(r["out_tokens"])

            for length, out in _scan_last_uniform(call):
                assert out[0] == j
                dist[out] = dist.get(out, 0.0) + w * length
    return dist


@pytest.mark.parametrize("K,V,seed", [(3, 3, 0), (2, 5, 1), (1, 7, 2)])
def test_exact_losslessness_on_tiny_vocab(K, V, seed):
    p, q = _rows(seed, K, V)
    dist = exact_distribution(p, q)
    assert abs(sum(dist.values()) - 1) < 1e-12
    reach = np.zeros(K + 2)
    emit = np.zeros((K + 1, V))
    for out, w in dist.items():
        n_acc, toks = out[0], out[1:]
        for i in range(n_acc + 1):
            reach[i] += w
            emit[i, toks[i]] += w
        # outputs are the accepted drafts, then one sampled token, then -1
        assert all(t == -1 for t in toks[n_acc + 1:])
    for i in range(K + 1):
        # the token emitted at a reached position is distributed as p_i
        assert np.max(np.abs(emit[i] - reach[i] * p[i])) < 1e-10
        if i < K:
            # acceptance probability at position i is sum_v min(p_i, q_i)
            assert abs(reach[i + 1] - reach[i] * np.minimum(p[i], q[i]).sum()) < 1e-10


def test_planted_residual_sign_error_breaks_losslessness(monkeypatch):
    """Discrimination check: the same exact test fails when the reference's
    residual is max(q - p, 0) instead of max(p - q, 0)."""
    real_max = np.maximum

    def swapped(a, b, *args, **kw):
        if isinstance(a, np.ndarray) and a.ndim == 1 and np.isscalar(b) and b == 0.0:
            return real_max(-a, b)
        return real_max(a, b, *args, **kw)

    p, q = _rows(3, 1, 4)
    monkeypatch.setattr(oracle.accept.np, "maximum", swapped)
    dist = exact_distribution(p, q)
    monkeypatch.undo()
    emit = np.zeros(4)
    for out, w in dist.items():
        emit[out[1]] += w
    assert np.max(np.abs(emit - p[0])) > 1e-3


def test_acceptance_rate_at_full_vocab_is_one_minus_tv():
    """Statistical form of the same corollary at V = 151936: the mean of the
    first test's accept indicator matches the mean of sum_v min(p, q)."""
    cfg = synth.config(2, k_spec=1)
    n = 300
    x = synth.make_accept_inputs(cfg, seed=123, bs=n)
    hits = 0
    expect = 0.0
    var = 0.0
    for b in range(n):
        r = oracle.accept_request(x.p[b], x.q[b], x.draft[b], x.u[b], 0)
        hits += r["accept_len"] >= 1
        a = np.minimum(x.p[b, 0].astype(np.float64), x.q[b, 0]).sum()
        expect += a
        var += a * (1 - a)
    assert abs(hits - expect) < 4.5 * np.sqrt(var) + 1


def test_one_hot_rows_reduce_to_greedy_rule():
    rng = np.random.default_rng(5)
    K, V = 6, 20
    for trial in range(50):
        tgt = rng.integers(0, V, K + 1)
        draft = np.where(rng.random(K) < 0.7, tgt[:K], rng.integers(0, V, K))
        p = np.zeros((K + 1, V), np.float32)
        p[np.arange(K + 1), tgt] = 1
        q = np.zeros((K, V), np.float32)
        q[np.arange(K), draft] = 1
        u = rng.random(K + 1).astype(np.float32)
        s = oracle.accept_request(p, q, draft, u, 50)
        g = oracle.greedy_accept_request(p, draft, 50)
        for key in ("accept_len", "commit_len", "bonus", "new_seq_len"):
            assert s[key] == g[key]
        assert np.array_equal(s["out_tokens"], g["out_tokens"])


def test_greedy_golden_dflash_example():
    fx = json.load(open(os.path.join(GOLDEN, "greedy_accept_dflash.json")))
    V = fx["vocab"]
    for c in fx["cases"]:
        tp = np.array(c["target_predict"])
        p = np.zeros((len(tp), V), np.float32)
        p[np.arange(len(tp)), tp] = 1
        r = oracle.greedy_accept_request(p, np.array(c["drafts"]), c["seq_len"])
        assert r["accept_len"] == c["accept_len"]
        assert r["bonus"] == c["bonus"]
        assert r["commit_len"] == c["commit_len"]
        assert r["new_seq_len"] == c["new_seq_len"]
        assert list(r["out_tokens"]) == c["out_tokens"]


def test_linear_spec_golden_nemotron_loop():
    fx = json.load(open(os.path.join(GOLDEN, "linear_spec_nemotron.json")))
    V = fx["vocab"]
    for c in fx["cases"]:
        ar = np.array(c["ar_tokens"])
        block = np.array(c["block"])
        p = np.zeros((len(ar), V), np.float32)
        p[np.arange(len(ar)), ar] = 1
        r = oracle.greedy_accept_request(p, block[1:], c["cache_len"])
        assert r["commit_len"] == c["accepted"]
        assert r["new_seq_len"] == c["cropped_len"]
        assert r["bonus"] == c["next_token"]
        assert list(r["out_tokens"][:r["commit_len"]]) == c["accepted_toks"]


def test_bounds_and_identity_draft():
    cfg = synth.config(1)
    x = synth.make_accept_inputs(cfg, seed=9, bs=40)
    for b in range(40):
        r = oracle.accept_request(x.p[b], x.q[b], x.draft[b], x.u[b], 17)
        K = cfg.k_spec
        assert 1 <= r["commit_len"] <= K + 1
        assert r["new_seq_len"] == 17 + r["commit_len"]
        n = r["accept_len"]
        assert np.array_equal(r["out_tokens"][:n], x.draft[b, :n])
        assert 0 <= r["bonus"] < cfg.vocab
        # q == p accepts every draft (u < 1)
        pp = x.p[b]
        rr = oracle.accept_request(pp, pp[:K], x.draft[b], x.u[b], 0)
        assert rr["accept_len"] == K


def test_invalid_draft_token_is_rejected_and_flagged():
    cfg = synth.config(1)
    x = synth.make_accept_inputs(cfg, seed=10, bs=1)
    d = x.draft[0].copy()
    d[2] = cfg.vocab + 5
    r = oracle.accept_request(x.p[0], x.q[0], d, np.zeros(cfg.k_spec + 1, np.float32), 0)
    assert r["accept_len"] == 2 and r["err"] & oracle.accept.ERR_TOKEN


def test_argmax_lowest_index_matches_numpy():
    rng = np.random.default_rng(0)
    for _ in range(200):
        x = rng.integers(-5, 5, size=rng.integers(1, 64)).astype(np.float32)
        assert oracle.argmax_lowest(x) == int(np.argmax(x))
    x = np.zeros(10)
    x[[3, 7]] = 1
    assert oracle.argmax_lowest(x) == 3
    # NaN never wins: numpy's nanargmax (first maximum ignoring NaN)
    for _ in range(200):
        x = rng.integers(-5, 5, size=rng.integers(2, 64)).astype(np.float32)
        x[rng.random(len(x)) < 0.3] = np.nan
        x[rng.integers(len(x))] = -np.inf
        if np.isnan(x).all():
            continue
        assert oracle.argmax_lowest(x) == int(np.nanargmax(x))
    assert oracle.argmax_lowest(np.array([np.nan, -np.inf, -np.inf])) == 1
    assert oracle.argmax_lowest(np.full(4, np.nan)) == 0


# ------------------------------------------------------------------ tree walk
def _tree_key(r):
    return tuple(int(n) for n in r["path_nodes"][:r["accept_len"]]), int(r["bonus"])


def exact_tree_distribution(parent, token, p, grid=256):
    """{(accepted nodes, bonus): probability} of the tree walk under
    independent U[0, 1) uniforms, integrated exactly with the reference as a
    black box. Nodes are numbered breadth first, so a decision on u[c] can
    only depend on uniforms of lower-numbered nodes: the uniforms are scanned
    in node order (then u[0], the final draw), each one split into the pieces
    on which the output is constant with the earlier ones fixed inside their
    pieces."""
    N = len(parent)
    order = list(range(1, N)) + [0]
    dist = {}

    def rec(k, u, w):
        if k == len(order):
            key = _tree_key(oracle.tree_accept_request(parent, token, p, u, 0))
            dist[key] = dist.get(key, 0.0) + w
            return
        dim = order[k]

        def call(x):
            uu = u.copy()
            uu[dim] = x
            return _tree_key(oracle.tree_accept_request(parent, token, p, uu, 0))

        pieces = _scan_last_uniform(call, grid)
        lo = 0.0
        for length, _ in pieces:
            uu = u.copy()
            uu[dim] = lo + length / 2
            rec(k + 1, uu, w * length)
            lo += length

    rec(0, np.full(N, 0.5), 1.0)
    return dist


TREES_BFS = [
    # (parent, V, seed): breadth-first numbered trees
    ([-1, 0, 0, 1, 1, 2], 5, 0),
    ([-1, 0, 0, 0, 1, 3], 6, 1),
    ([-1, 0, 1, 2], 4, 2),        # a chain
    ([-1, 0, 0, 0], 5, 3),        # one level, three candidates
]


def _tree_case(parent, V, seed):
    rng = np.random.default_rng(seed)
    N = len(parent)
    token = np.zeros(N, np.int64)
    for x in range(N):
        kids = oracle.tree_children(parent, x)
        token[kids] = rng.choice(V, size=len(kids), replace=False)   # distinct siblings
    p = np.stack([_dist(rng, V) for _ in range(N)])
    return np.array(parent), token, p


@pytest.mark.parametrize("parent,V,seed", TREES_BFS)
def test_tree_walk_is_lossless_exactly(parent, V, seed):
    """Losslessness of the tree walk: every (accepted path, bonus) outcome has
    exactly the target's autoregressive probability of the emitted tokens
    along the tree, prod p[parent(n)](token n) * p[last](bonus), and a bonus is
    never one of the last node's child tokens (those are emitted by
    descending)."""
    parent, token, p = _tree_case(parent, V, seed)
    dist = exact_tree_distribution(parent, token, p)
    assert abs(sum(dist.values()) - 1) < 1e-12
    seen = 0.0
    for (path, bonus), w in dist.items():
        prob, x = 1.0, 0
        for n in path:
            assert parent[n] == x
            prob *= p[x, token[n]]
            x = n
        assert bonus not in [token[c] for c in oracle.tree_children(parent, x)]
        prob *= p[x, bonus]
        assert abs(w - prob) < 1e-10, (path, bonus, w, prob)
        seen += prob
    # every emitted sequence of positive probability occurs
    assert abs(seen - 1) < 1e-10


def test_chain_tree_is_the_linear_accept_with_one_hot_drafts():
    """A chain tree is a linear block whose draft distributions are one-hot at
    the draft tokens: the tree walk must agree with the (separately pinned)
    linear reference fed q = one-hot, test uniforms u[1..K] and final u[0]."""
    rng = np.random.default_rng(7)
    for trial in range(300):
        K, V = int(rng.integers(1, 6)), int(rng.integers(2, 9))
        parent = np.arange(-1, K, dtype=np.int64)
        token = np.concatenate([[0], rng.integers(0, V, size=K)])
        p = np.stack([_dist(rng, V, floor=0.01) for _ in range(K + 1)]).astype(np.float32)
        u = rng.random(K + 1).astype(np.float32)
        q = np.zeros((K, V), np.float32)
        q[np.arange(K), token[1:]] = 1.0
        lin = oracle.accept_request(p, q, token[1:], np.concatenate([u[1:], u[:1]]), 5)
        tr = oracle.tree_accept_request(parent, token, p, u, 5)
        for key in ("accept_len", "commit_len", "bonus", "new_seq_len", "err"):
            assert lin[key] == tr[key], (trial, key)
        assert np.array_equal(lin["out_tokens"], tr["out_tokens"])
        assert np.array_equal(tr["path_nodes"][:tr["accept_len"]], np.arange(1, tr["accept_len"] + 1))


def test_planted_tree_normaliser_mistake_breaks_losslessness(monkeypatch):
    """Discrimination check: testing later siblings against p alone (dropping
    the 1 - T normaliser of the residual) must fail the exact test."""
    parent, token, p = _tree_case([-1, 0, 0, 0], 5, 3)
    real = oracle.accept.np.float64

    class NoRenorm:
        calls = 0

    def fake_tree(parent, token, p, u, seq_len):
        # same walk with T frozen at 0
        N, V = p.shape
        x, path, tried = 0, [], []
        while True:
            nxt = -1
            tried = []
            for c in oracle.tree_children(parent, x):
                d = int(token[c])
                if real(u[c]) < real(p[x, d]) and d not in tried:
                    nxt = c
                    break
                tried.append(d)
            if nxt < 0:
                break
            path.append(nxt)
            x = nxt
        r = p[x].astype(real)
        r[tried] = 0.0
        t = int(np.searchsorted(np.cumsum(r), real(u[0]) * r.sum(), side="right"))
        nodes = np.full(N, -1)
        nodes[:len(path)] = path
        return dict(accept_len=len(path), path_nodes=nodes, bonus=t)

    monkeypatch.setattr(oracle, "tree_accept_request", fake_tree)
    with pytest.raises(AssertionError):
        test_tree_walk_is_lossless_exactly([-1, 0, 0, 0], 5, 3)


def test_tree_walk_flags_bad_tokens_and_parents():
    p = np.full((4, 3), 1 / 3, np.float32)
    r = oracle.tree_accept_request(np.array([-1, 0, 0, 5]), np.array([0, 7, 1, 2]), p,
                                   np.zeros(4, np.float32), 10)
    assert r["err"] & oracle.accept.ERR_TOKEN and r["err"] & oracle.accept.ERR_TREE
    # u = 0 accepts the first valid child (node 2), a leaf; bonus from p[2]
    assert r["accept_len"] == 1 and r["path_nodes"][0] == 2 and r["out_tokens"][0] == 1
    assert r["new_seq_len"] == 12


def test_sample_tie_band_covers_other_summation_orders():
    """oracle.accept.sample_tie_band(V, S) bounds how far two correct float64
    evaluations of the draw's running sums may be apart. On a full-vocabulary
    residual row, the reference's sequential running sum, a blocked order
    (pairwise sums of four entries, a reduction over 256-entry sub-blocks, a
    running sum over the sub-block totals, then a running sum inside the
    sub-block, as a GPU reduction orders it) and a reversed accumulation all
    agree to well inside half the band at every index, and against exactly
    rounded prefix sums (math.fsum) at sampled indices."""
    import math
    rng = np.random.default_rng(7)
    V = 151936
    lp = rng.standard_normal(V) * 3.0
    lq = lp + rng.standard_normal(V) * 0.5
    p = np.exp(lp - lp.max()); p = (p / p.sum()).astype(np.float32)
    q = np.exp(lq - lq.max()); q = (q / q.sum()).astype(np.float32)
    r = np.maximum(p.astype(np.float64) - q.astype(np.float64), 0.0)
    C = np.cumsum(r)
    S = C[-1]
    band = oracle.accept.sample_tie_band(V, S)
    pad = np.zeros(-(-V // 256) * 256)
    pad[:V] = r
    quads = pad.reshape(-1, 4)
    lane = (quads[:, 0] + quads[:, 1]) + (quads[:, 2] + quads[:, 3])
    sub = lane.reshape(-1, 64)
    while sub.shape[1] > 1:          # pairwise tree inside each sub-block
        sub = sub[:, 0::2] + sub[:, 1::2]
    base = np.concatenate([[0.0], np.cumsum(sub[:, 0])[:-1]])
    inner = np.cumsum(pad.reshape(-1, 256), axis=1)
    C_blocked = (base[:, None] + inner).ravel()[:V]
    C_rev = S - np.concatenate([np.cumsum(r[::-1])[::-1][1:], [0.0]])
    assert np.max(np.abs(C_blocked - C)) <= band / 2
    assert np.max(np.abs(C_rev - C)) <= band / 2
    for t in rng.integers(0, V, size=64):
        exact = math.fsum(r[:t + 1])
        assert abs(C[t] - exact) <= band / 4 and abs(C_blocked[t] - exact) <= band / 4
    # the band is a rounding bound, orders of magnitude below the accept-test
    # tie width
    assert band < 1e-9 * S


def test_zero_threshold_is_not_a_tie():
    """u = 0 draws the first entry with mass on both sides exactly (the
    threshold and every earlier running sum are exact zeros): no tie, while a
    threshold a rounding step away from a boundary is one."""
    C = np.cumsum(np.array([0.0, 0.0, 0.25, 0.75]))
    band = oracle.accept.sample_tie_band(4, 1.0)
    assert not oracle.accept.draw_is_tie(0.0, C, 2, band)
    assert oracle.accept.draw_is_tie(0.25 + band / 2, C, 3, band)
    assert not oracle.accept.draw_is_tie(0.5, C, 3, band)
    p = np.array([[0.0, 0.0, 0.25, 0.75], [0.1, 0.2, 0.3, 0.4]], np.float32)
    q = np.array([[0.0, 0.0, 0.25, 0.75]], np.float32)
    r = oracle.accept_request(p, q, np.array([3]), np.array([0.0, 0.0], np.float32), 0)
    assert r["accept_len"] == 1 and r["bonus"] == 0 and not r["tie"]


def test_long_chain_tree_is_the_linear_accept():
    """The same identity for chains longer than one 64-bit mask word (up to
    200 nodes), with targets peaked at the drafts so that deep acceptance
    happens: the tree walk has no node limit of its own."""
    rng = np.random.default_rng(71)
    deepest = 0
    for trial in range(20):
        K, V = int(rng.integers(65, 200)), 7
        parent = np.arange(-1, K, dtype=np.int64)
        token = np.concatenate([[0], rng.integers(0, V, size=K)])
        p = np.stack([_dist(rng, V, floor=0.001) for _ in range(K + 1)])
        p[np.arange(K), token[1:]] += 40.0           # mostly accepted
        p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
        u = rng.random(K + 1).astype(np.float32)
        q = np.zeros((K, V), np.float32)
        q[np.arange(K), token[1:]] = 1.0
        lin = oracle.accept_request(p, q, token[1:], np.concatenate([u[1:], u[:1]]), 5)
        tr = oracle.tree_accept_request(parent, token, p, u, 5)
        for key in ("accept_len", "commit_len", "bonus", "new_seq_len", "err"):
            assert lin[key] == tr[key], (trial, key)
        assert np.array_equal(lin["out_tokens"], tr["out_tokens"])
        deepest = max(deepest, tr["accept_len"])
    assert deepest > 64
