"""Pins for the block-preparation reference (CPU only): the hand-worked
example of the DFlash block fill and the slot rule, and the capacity / slot
error conditions."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle.prepare import ERR_CAPACITY, ERR_SLOT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fx():
    return json.load(open(os.path.join(GOLDEN, "prepare_block_small.json")))


def test_golden_draft_pass():
    fx = _fx()
    ids, pos, loc, err = oracle.prepare_block(
        np.array(fx["verified_id"]), np.array(fx["seq_lens"]), np.array(fx["page_table"]),
        fx["page_size"], fx["block"], fx["mask_token_id"])
    e = fx["expect_draft_pass"]
    assert err == 0
    assert ids.tolist() == e["block_ids"]
    assert pos.tolist() == e["positions"]
    assert loc.tolist() == e["cache_loc"]


def test_golden_verify_pass():
    fx = _fx()
    ids, pos, loc, err = oracle.prepare_block(
        np.array(fx["verified_id"]), np.array(fx["seq_lens"]), np.array(fx["page_table"]),
        fx["page_size"], fx["block"], fx["mask_token_id"], np.array(fx["draft_tokens"]))
    assert err == 0
    assert ids.tolist() == fx["expect_verify_pass"]["block_ids"]
    assert loc.tolist() == fx["expect_draft_pass"]["cache_loc"]


def test_identity_table_gives_contiguous_slots():
    P, B = 16, 8
    L = np.array([0, 5, 31, 100])
    need = (L + 2 * B + P - 1) // P
    table = np.full((4, need.max()), -1)
    base = np.concatenate([[0], np.cumsum(need)[:-1]])
    for b in range(4):
        table[b, :need[b]] = base[b] + np.arange(need[b])
    _, pos, loc, err = oracle.prepare_block(np.zeros(4), L, table, P, B, 0)
    assert err == 0
    for b in range(4):
        assert loc[b].tolist() == list(base[b] * P + L[b] + np.arange(B))


def test_capacity_and_slot_errors():
    table = np.array([[3, -1]])
    _, _, loc, err = oracle.prepare_block(np.zeros(1), np.array([2]), table, 4, 4, 0)
    assert err == ERR_SLOT and loc[0].tolist() == [14, 15, -1, -1]
    _, _, _, err = oracle.prepare_block(np.zeros(1), np.array([5]), table, 4, 4, 0)
    assert err & ERR_CAPACITY
    _, _, loc, err = oracle.prepare_block(np.zeros(1), np.array([0]), np.array([[9, 1]]), 4, 4, 0,
                                          num_pages=5)
    assert err & ERR_SLOT and loc[0, 0] == -1


# ------------------------------------------------------------ tree blocks
def _tfx():
    return json.load(open(os.path.join(GOLDEN, "prepare_tree_small.json")))


def test_tree_golden():
    fx = _tfx()
    args = (np.array(fx["verified_id"]), np.array(fx["seq_lens"]), np.array(fx["page_table"]),
            fx["page_size"], np.array(fx["parent"]), fx["mask_token_id"])
    ids, pos, loc, err = oracle.prepare_tree(*args, np.array(fx["node_tokens"]))
    e = fx["expect"]
    assert err == 0
    assert ids.tolist() == e["block_ids"]
    assert pos.tolist() == e["positions"]
    assert loc.tolist() == e["cache_loc"]
    ids, _, _, _ = oracle.prepare_tree(*args)
    assert ids.tolist() == e["block_ids_mask_fill"]


@pytest.mark.parametrize("B,seed", [(1, 0), (8, 1), (16, 2), (64, 3), (300, 4)])
def test_chain_tree_is_the_linear_block(B, seed):
    """A chain (parent n - 1) is a linear block: ids, positions and slots
    equal spec_prepare_block's, for both passes."""
    rng = np.random.default_rng(seed)
    P, bs = 16, 5
    L = rng.integers(0, 300, size=bs)
    need = (L + 2 * B + P - 1) // P
    table = np.full((bs, need.max()), -1)
    perm = rng.permutation(int(need.sum()))
    o = 0
    for b in range(bs):
        table[b, :need[b]] = perm[o:o + need[b]]
        o += need[b]
    vid = rng.integers(0, 1000, size=bs)
    drafts = rng.integers(0, 1000, size=(bs, B - 1))
    chain = np.arange(-1, B - 1)
    nodes = np.concatenate([np.zeros((bs, 1), np.int64), drafts], axis=1)
    for d, nt in ((None, None), (drafts, nodes)):
        want = oracle.prepare_block(vid, L, table, P, B, 77, d, int(need.sum()))
        got = oracle.prepare_tree(vid, L, table, P, chain, 77, nt, int(need.sum()))
        for g, w in zip(got, want):
            assert np.array_equal(g, w)


def test_tree_positions_are_root_path_lengths():
    """positions - L is the length of each node's root path (ancestors
    counted by walking up), for random trees; siblings share a position."""
    from verify_attention_amd import synth
    rng = np.random.default_rng(5)
    for i in range(20):
        N = int(rng.integers(2, 65)) if i % 4 else int(rng.integers(65, 513))
        par = synth.random_tree_parents(rng, N, int(rng.integers(2, N + 1)))
        _, pos, _, err = oracle.prepare_tree(np.zeros(1), np.array([1000]),
                                             np.arange(160)[None, :], 16, par, 0)
        assert err == 0
        for n in range(N):
            up, x = 0, n
            while par[x] >= 0:
                x, up = par[x], up + 1
            assert pos[0, n] == 1000 + up
        for n in range(1, N):
            sib = [m for m in range(1, N) if par[m] == par[n]]
            assert len({int(pos[0, m]) for m in sib}) == 1


def test_tree_errors():
    par = np.array([-1, 0, 5, 2, 1])       # node 2's parent is later; node 3 descends from it
    _, pos, loc, err = oracle.prepare_tree(np.zeros(1), np.array([4]), np.array([[0, 1, 2]]), 4,
                                           par, 0)
    assert err & oracle.prepare.ERR_TREE
    assert pos[0].tolist() == [4, 5, -1, -1, 6]
    assert loc[0].tolist() == [4, 5, 6, 7, 8]
    _, _, _, err = oracle.prepare_tree(np.zeros(1), np.array([9]), np.array([[0, 1, 2]]), 4,
                                       par, 0)
    assert err & ERR_CAPACITY and err & ERR_SLOT


def test_quadratic_positions():
    """The quadratic layout in position order: spine token i at L + i, member
    m of the group after spine token j at L + j + 1 + m (the role table of the
    layout, built separately, names every position)."""
    from verify_attention_amd import synth
    for k in (1, 2, 4, 7, 15, 21):
        roles, _ = synth.quadratic_layout(k)
        par = synth.quadratic_parents(k)
        n = (k + 1) ** 2
        _, pos, _, err = oracle.prepare_tree(np.zeros(1), np.array([50]),
                                             np.arange(20)[None, :], 32, par, 0)
        assert err == 0
        for p_, (kind, j, m) in enumerate(roles):
            assert pos[0, p_] == (50 + j if kind == "spine" else 50 + j + 1 + m)
        assert n == len(roles)
