"""The seeded input generators build the workloads they describe: the Tree
sampler's beam-shaped trees (sizes, levels, the kept prefixes are the best by
summed draft log-probability, sibling tokens are the drafter's top
candidates) and the top-candidate selection."""
import numpy as np

import oracle
from verify_attention_amd import synth


def test_top_indices_is_a_stable_descending_sort():
    rng = np.random.default_rng(0)
    for _ in range(300):
        n = int(rng.integers(1, 400))
        x = (rng.integers(0, 4, n).astype(float) if rng.random() < 0.5
             else rng.standard_normal(n))
        k = int(rng.integers(1, n + 1))
        assert np.array_equal(synth._top_indices(x, k), np.argsort(-x, kind="stable")[:k])


def test_beam_tree_keeps_the_best_prefixes():
    cfg = synth.config(10, bs=2, vocab=700, tree_depth=6, tree_width=8, block=49)
    par, masks = synth.make_trees(cfg, 5)
    ti = synth.make_tree_accept_inputs(cfg, 5, par)
    assert par.shape == (2, 49) and masks.shape == (2, 49)    # one mask word per row
    rp, rq = synth.rng_for(5, "plogit"), synth.rng_for(5, "qnoise")
    for b in range(2):
        lp = rp.standard_normal((49, 700)) * cfg.logit_sigma
        lq = lp + np.stack([rq.standard_normal(700) for _ in range(49)]) * cfg.q_noise_sigma
        logq = lq - np.log(np.exp(lq - lq.max(1, keepdims=True)).sum(1, keepdims=True)) \
            - lq.max(1, keepdims=True)
        depth = np.array(oracle.tree_depths(par[b]))
        assert np.array_equal(np.bincount(depth), [1] + [8] * 6)
        assert (np.diff(depth) >= 0).all()                 # level order
        score = np.zeros(49)
        for n in range(1, 49):
            score[n] = score[par[b, n]] + logq[par[b, n], ti.token[b, n]]
        for lev in range(1, 7):
            prev = np.flatnonzero(depth == lev - 1)
            kept = np.flatnonzero(depth == lev)
            # every extension of a kept prefix by one of its top-8 candidates
            # that was not kept scores at most the worst kept one
            worst = score[kept].min()
            for x in prev:
                top = np.argsort(-lq[x], kind="stable")[:8]
                mine = set(ti.token[b, kept[par[b, kept] == x]].tolist())
                # the kept children of x are its top candidates, in rank order
                kids = kept[par[b, kept] == x]
                assert list(ti.token[b, kids]) == list(top[:len(kids)])
                for t in top:
                    if t not in mine:
                        assert score[x] + logq[x, t] <= worst + 1e-12
