"""Pins for the float64 committed-prefix KV reference (CPU only).

The commit is pinned by the slot rule of the block preparation (the released
slots are the prepared cache slots past the committed length), by the
definition read back through the page table (the committed sequence is the
context and root followed by the accepted nodes' rows), by the chain (linear
verify: nothing moves) and by attention: after the commit, causal attention
of the last accepted node's query over the committed prefix equals that
node's tree attention over the uncommitted block. A planted off-by-one
destination must fail.
"""
import numpy as np
import pytest

import oracle
import oracle.commit
from verify_attention_amd import synth


def _case(seed, bs=3, B=12, depth=5):
    cfg = synth.config(6, bs=bs, block=B, tree_depth=depth, hq=4, hkv=2, d=16, dtype="f32",
                       ctx_lo=20, ctx_hi=45, vocab=50)
    x = synth.make_attn_inputs(cfg, seed)
    par, masks = synth.make_trees(cfg, seed)
    ti = synth.make_tree_accept_inputs(cfg, seed, par)
    acc = [oracle.tree_accept_request(ti.parent[b], ti.token[b], ti.p[b], ti.u[b], x.seq_lens[b])
           for b in range(bs)]
    depth_b = np.array([a["accept_len"] for a in acc])
    path = np.stack([a["path_nodes"] for a in acc])
    return cfg, x, masks, depth_b, path


def _paths_with_depth(cfg, x, masks, seed):
    """Deterministic accepted paths of every depth: the chain of node 0's
    descendants taken through each node's first child."""
    par, _ = synth.make_trees(cfg, seed)
    depth, path = [], []
    for b in range(cfg.bs):
        p, node = [], 0
        while True:
            kids = oracle.tree_children(par[b], node)
            if not kids:
                break
            node = kids[0]
            p.append(node)
        depth.append(len(p))
        path.append(p + [-1] * (cfg.block - len(p)))
    return np.array(depth), np.array(path)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_released_slots_are_the_prepared_slots_past_the_commit(seed):
    cfg, x, masks, depth, path = _case(seed)
    _, _, freed = oracle.commit_kv(x.k_pool, x.v_pool, x.page_table, x.seq_lens, depth, path,
                                   cfg.block)
    _, _, loc, err = oracle.prepare_block(np.zeros(cfg.bs), x.seq_lens, x.page_table, cfg.page,
                                          cfg.block, 0)
    assert err == 0
    for b in range(cfg.bs):
        d = depth[b]
        assert list(freed[b, :cfg.block - d - 1]) == list(loc[b, d + 1:])
        assert (freed[b, cfg.block - d - 1:] == -1).all()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_committed_sequence_is_context_then_accepted_nodes(seed):
    cfg, x, masks, _, _ = _case(seed)
    depth, path = _paths_with_depth(cfg, x, masks, seed)
    assert depth.max() >= 2
    k2, v2, _ = oracle.commit_kv(x.k_pool, x.v_pool, x.page_table, x.seq_lens, depth, path,
                                 cfg.block)
    for b in range(cfg.bs):
        L, d = int(x.seq_lens[b]), int(depth[b])
        for h in range(cfg.hkv):
            K0, V0 = oracle.unpage_kv(x.k_pool, x.v_pool, x.page_table[b], L + cfg.block, h)
            K1, V1 = oracle.unpage_kv(k2, v2, x.page_table[b], L + cfg.block, h)
            rows = list(range(L + 1)) + [L + int(n) for n in path[b, :d]]
            assert np.array_equal(K1[:L + d + 1], K0[rows])
            assert np.array_equal(V1[:L + d + 1], V0[rows])
            # positions past the committed prefix are untouched unless a node moved there
            assert np.array_equal(K1[L + d + 1:], K0[L + d + 1:])


def test_chain_path_moves_nothing():
    cfg, x, _, _, _ = _case(4)
    depth = np.array([0, 3, cfg.block - 1])
    k2, v2, freed = oracle.commit_kv(x.k_pool, x.v_pool, x.page_table, x.seq_lens, depth, None,
                                     cfg.block)
    assert np.array_equal(k2, x.k_pool) and np.array_equal(v2, x.v_pool)
    assert (freed[2] == -1).all() and (freed[0, :cfg.block - 1] >= 0).all()


@pytest.mark.parametrize("seed", [0, 3])
def test_causal_view_of_the_commit_equals_the_tree_view(seed):
    cfg, x, masks, _, _ = _case(seed)
    depth, path = _paths_with_depth(cfg, x, masks, seed)
    q = x.as_f64("q")
    kp, vp = x.as_f64("k_pool"), x.as_f64("v_pool")
    o_tree, _ = oracle.block_attn_rows(q, kp, vp, x.page_table, x.seq_lens, oracle.TREE, 0,
                                       tree=masks)
    k2, v2, _ = oracle.commit_kv(kp, vp, x.page_table, x.seq_lens, depth, path, cfg.block)
    for b in range(cfg.bs):
        d = int(depth[b])
        last = int(path[b, d - 1]) if d else 0
        # the last accepted node's query, as block row d of a causal block of d + 1
        qb = np.zeros((1, d + 1, cfg.hq, cfg.d))
        qb[0, d] = q[b, last]
        o_c, _ = oracle.block_attn_rows(qb, k2, v2, x.page_table[b:b + 1], x.seq_lens[b:b + 1],
                                        oracle.CAUSAL, 0, rows=[(0, d, h) for h in range(cfg.hq)])
        assert np.max(np.abs(o_c[0, d] - o_tree[b, last])) < 1e-12


def test_planted_off_by_one_destination_fails(monkeypatch):
    monkeypatch.setattr(oracle.commit, "dest_position", lambda L, k: L + k)
    with pytest.raises(AssertionError):
        test_causal_view_of_the_commit_equals_the_tree_view(0)
