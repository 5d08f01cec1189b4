"""Pins for the quadratic layout's hand-off (CPU only): the hand-worked
example, the group rows named by the layout's role table (built separately),
lowest-index ties, the error form, and the spine's compaction: after the
commit with the spine path, causal attention of the last accepted spine token
over the committed prefix equals its attention in the quadratic block."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import quadratic
from verify_attention_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_handoff_golden():
    fx = json.load(open(os.path.join(GOLDEN, "quadratic_handoff_small.json")))
    logits = np.array(fx["logits"], np.float64)
    for c in fx["cases"]:
        nxt, block = quadratic.handoff(logits, c["accept_len"], fx["k"], fx["bonus"],
                                       fx["mask_token_id"])
        assert nxt.tolist() == c["next_draft"]
        assert block.tolist() == c["next_block"]


@pytest.mark.parametrize("k", [1, 2, 3, 4, 7, 8, 15])
def test_handoff_reads_the_group_the_role_table_names(k):
    """For every accept length a, the drafts are the greedy tokens of the
    rows whose layout role is (mask, group a, member m), in member order;
    the next block's spine positions are those the role table marks as
    spine tokens 1 .. k."""
    rng = np.random.default_rng(k)
    roles, _ = synth.quadratic_layout(k)
    n, V = (k + 1) ** 2, 97
    logits = rng.standard_normal((n, V))
    for a in range(k + 1):
        nxt, block = quadratic.handoff(logits, a, k, 5, 99)
        rows = {m: pos for pos, (kind, j, m) in enumerate(roles) if kind == "mask" and j == a}
        assert nxt.tolist() == [int(np.argmax(logits[rows[m]])) for m in range(k)]
        spine = {j: pos for pos, (kind, j, m) in enumerate(roles) if kind == "spine"}
        assert block[spine[0]] == 5
        for m in range(k):
            assert block[spine[m + 1]] == nxt[m]
        others = [p for p in range(n) if roles[p][0] == "mask"]
        assert (block[others] == 99).all()


def test_handoff_ties_and_range():
    k, V = 3, 10
    logits = np.zeros(((k + 1) ** 2, V))
    logits[:, 7] = 2.0
    logits[:, 3] = 2.0
    logits[quadratic.group_rows(k, 2)[1], 0] = np.nan
    nxt, _ = quadratic.handoff(logits, 2, k, 0, 1)
    assert nxt.tolist() == [3, 3, 3]             # lowest index among equal maxima, NaN never
    nxt, block = quadratic.handoff(logits, k + 1, k, 0, 1)
    assert nxt.tolist() == [-1] * k and block is None
    nxt, block = quadratic.handoff(logits, -1, k, 0, 1)
    assert nxt.tolist() == [-1] * k and block is None


@pytest.mark.parametrize("k,seed", [(2, 0), (4, 1), (7, 2), (9, 3)])
def test_spine_compaction_keeps_the_causal_view(k, seed):
    """After the accept of a spine drafts, the commit with path
    p_i = i (k + 1) makes the accepted spine contiguous: the last accepted
    spine token's causal attention over the committed prefix equals its
    attention in the quadratic block (which sees the spine up to it)."""
    n = (k + 1) ** 2
    cfg = synth.config(8, bs=3, block=n, quad_k=k, hq=4, hkv=2, d=16, dtype="f32", ctx_lo=10,
                       ctx_hi=70)
    x = synth.make_attn_inputs(cfg, seed)
    _, masks = synth.quadratic_layout(k)
    q, kp, vp = x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool")
    o_quad, _ = oracle.block_attn_rows(q, kp, vp, x.page_table, x.seq_lens, oracle.TREE, 0,
                                       tree=masks)
    acc = np.array([0, k // 2, k])
    path = np.tile(np.array(quadratic.spine_path(k) + [-1] * (n - k)), (3, 1))
    k2, v2, freed = oracle.commit_kv(kp, vp, x.page_table, x.seq_lens, acc, path, n)
    for b in range(3):
        a = int(acc[b])
        last = a * (k + 1)
        qb = np.zeros((1, a + 1, cfg.hq, cfg.d))
        qb[0, a] = q[b, last]
        o_c, _ = oracle.block_attn_rows(qb, k2, v2, x.page_table[b:b + 1], x.seq_lens[b:b + 1],
                                        oracle.CAUSAL, 0, rows=[(0, a, h) for h in range(cfg.hq)])
        assert np.max(np.abs(o_c[0, a] - o_quad[b, last])) < 1e-12
        assert (freed[b, :n - a - 1] >= 0).all() and (freed[b, n - a - 1:] == -1).all()


def test_planted_group_off_by_one_fails(monkeypatch):
    monkeypatch.setattr(quadratic, "group_rows",
                        lambda k, j: [j * (k + 1) + m for m in range(k)])
    with pytest.raises(AssertionError):
        test_handoff_reads_the_group_the_role_table_names(3)
