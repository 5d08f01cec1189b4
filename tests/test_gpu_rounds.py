"""GPU parity of the calls that join one round to the next, through the C
ABI: spec_prepare_tree (tree and quadratic blocks), spec_accept_prepare (the
accept and the next round's block in one call) and spec_quadratic_handoff
(the next round's drafts from the group after the last accepted spine
token), each against the float64 CPU reference; integer outputs bit for bit.
The last test runs two quadratic rounds back to back on the GPU and checks
every output of the chain against the reference chain."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import quadratic
import verify_attention_amd as va
from verify_attention_amd import synth
from _support import check_tie_share, print_case, to_dev

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    return t.cpu().numpy()


# ---------------------------------------------------------- prepare_tree
def test_prepare_tree_golden(gpu_lib):
    fx = json.load(open(os.path.join(GOLDEN, "prepare_tree_small.json")))
    print_case("prepare_tree golden")
    t = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    e = fx["expect"]
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids, pos, loc = va.prepare_tree(t(fx["verified_id"]), t(fx["seq_lens"]), t(fx["page_table"]),
                                    fx["page_size"], t(fx["parent"]), fx["mask_token_id"], 16,
                                    t(fx["node_tokens"]), err=err)
    assert ids.cpu().tolist() == e["block_ids"]
    assert pos.cpu().tolist() == e["positions"]
    assert loc.cpu().tolist() == e["cache_loc"]
    ids, _, _ = va.prepare_tree(t(fx["verified_id"]), t(fx["seq_lens"]), t(fx["page_table"]),
                                fx["page_size"], t(fx["parent"]), fx["mask_token_id"], 16)
    assert ids.cpu().tolist() == e["block_ids_mask_fill"]
    assert int(err.item()) == 0


def _tree_case(cfg, seed, per_request=True, quad=False):
    seq = synth.context_lengths(cfg, seed)
    table, num_pages = synth.page_layout(cfg, seq, seed)
    if quad:
        par = synth.quadratic_parents(cfg.quad_k)
        if per_request:
            par = np.tile(par, (cfg.bs, 1))
    else:
        par, _ = synth.make_trees(cfg, seed, per_request=per_request)
    verified, _ = synth.make_round_state(cfg, seed)
    tokens = np.random.default_rng(seed).integers(0, 1000, size=(cfg.bs, cfg.block)).astype(
        np.int32)
    return seq, table, num_pages, par.astype(np.int32), verified, tokens


@pytest.mark.parametrize("name,cid,over,per_req,quad", [
    ("tree_workload", 6, {}, True, False),
    ("tree_shared_64", 6, dict(bs=9, block=64, tree_depth=40), False, False),
    ("tree_single_node", 6, dict(bs=5, block=1, tree_depth=1), True, False),
    ("tree_p32_ragged", 6, dict(bs=37, page=32, block=45, tree_depth=12, ctx_lo=1, ctx_hi=3000),
     True, False),
    ("quadratic_k4", 8, {}, False, True),
    ("quadratic_k7_per_request", 8, dict(bs=6, block=64, quad_k=7), True, True),
    # more than 64 nodes: a workgroup per request, pointer jumping through LDS
    ("tree_sampler_481", 10, dict(bs=4, vocab=64), True, False),
    ("tree_65_shared", 6, dict(bs=5, block=65, tree_depth=64), False, False),
    ("deep_512", 6, dict(bs=3, block=512, tree_depth=512, ctx_lo=1, ctx_hi=900, page=32),
     True, False),
])
def test_prepare_tree_matches_reference(gpu_lib, name, cid, over, per_req, quad):
    cfg = synth.config(cid, **over)
    print_case("prepare_tree", name, cfg.bs, cfg.block)
    seq, table, num_pages, par, verified, tokens = _tree_case(cfg, 11, per_req, quad)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for nt in (None, tokens):
        got = va.prepare_tree(to_dev(verified), to_dev(seq), to_dev(table), cfg.page, to_dev(par),
                              123, num_pages, None if nt is None else to_dev(nt), err=err)
        ref = oracle.prepare_tree(verified, seq, table, cfg.page, par, 123, nt, num_pages)
        for g, r in zip(got, ref[:3]):
            assert np.array_equal(_np(g), r)
        assert ref[3] == 0
    assert int(err.item()) == 0


def test_prepare_tree_wide_error_flags(gpu_lib):
    """A 300-node block: a bad edge deep in the tree marks every descendant
    (position -1, SPEC_ERR_TREE), as the reference does."""
    print_case("prepare_tree wide errors")
    rng = np.random.default_rng(3)
    par = synth.random_tree_parents(rng, 300, 120)[None].repeat(2, 0)
    par[1, 150] = 200                           # not an earlier node
    seq = np.array([7, 100], np.int32)
    table = np.arange(2 * 30, dtype=np.int32).reshape(2, 30)
    verified = np.array([5, 6], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = va.prepare_tree(to_dev(verified), to_dev(seq), to_dev(table), 16, to_dev(par), 9, 60,
                          err=err)
    ref = oracle.prepare_tree(verified, seq, table, 16, par, 9, None, 60)
    for g, r in zip(got, ref[:3]):
        assert np.array_equal(_np(g), r)
    assert (ref[1][1] == -1).sum() >= 1 and (ref[1][0] >= 0).all()
    assert int(err.item()) == ref[3] == va.ERR_TREE


def test_prepare_tree_error_flags(gpu_lib):
    print_case("prepare_tree errors")
    seq = np.array([4, 9, 0], np.int32)
    table = np.array([[0, 1, 2], [3, 4, 5], [6, 40, 7]], np.int32)
    par = np.array([[-1, 0, 5, 2, 1], [-1, 0, 1, 2, 3], [-1, 0, 0, 0, 0]], np.int32)
    verified = np.array([1, 2, 3], np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = va.prepare_tree(to_dev(verified), to_dev(seq), to_dev(table), 4, to_dev(par), 0, 8,
                          err=err)
    ref = oracle.prepare_tree(verified, seq, table, 4, par, 0, None, 8)
    for g, r in zip(got, ref[:3]):
        assert np.array_equal(_np(g), r)
    assert int(err.item()) == ref[3] == (va.ERR_TREE | va.ERR_CAPACITY | va.ERR_SLOT)


# -------------------------------------------------------- accept_prepare
@pytest.mark.parametrize("cid,bs,B_next,greedy", [(2, None, 16, False), (4, None, 16, False),
                                                  (1, 40, 300, False), (2, 8, 32, True)])
def test_accept_prepare_is_accept_then_prepare(gpu_lib, cid, bs, B_next, greedy):
    """Every output equals spec_accept followed by spec_prepare_block on the
    bonus and the new lengths (both GPU calls), and the reference's accept
    and block preparation; B_next = 300 takes more than one pass over the
    workgroup's threads."""
    cfg = synth.config(cid)
    print_case("accept_prepare", cid, bs, B_next, greedy)
    x = synth.make_accept_inputs(cfg, seed=cid + 20, bs=bs)
    n = x.draft.shape[0]
    c2 = synth.config(cid, bs=n, block=B_next)
    seq = synth.context_lengths(c2, cid)
    table, num_pages = synth.page_layout(c2, seq + cfg.k_spec + 1, cid)
    p, q, d, u, s, tab = (to_dev(a) for a in (x.p, x.q, x.draft, x.u, seq, table))
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = va.accept_prepare(p, q, d, u, s, tab, cfg.page, B_next, 77, num_pages, greedy=greedy,
                            err=e1)
    acc = va.accept(p, q, d, u, s, greedy=greedy, err=e2)
    prep = va.prepare_block(acc["bonus"], acc["new_seq_lens"], tab, cfg.page, B_next, 77,
                            num_pages, err=e2)
    torch.cuda.synchronize()
    for k in ("accept_len", "commit_len", "bonus", "out_tokens", "new_seq_lens"):
        assert torch.equal(got[k], acc[k]), k
    for k, t in zip(("block_ids", "positions", "cache_loc"), prep):
        assert torch.equal(got[k], t), k
    assert int(e1.item()) == int(e2.item()) == 0
    # and against the reference
    ref = oracle.accept_batch(x.p, x.q, x.draft, x.u, seq, greedy=greedy)
    keep = ~ref["tie_sample"]
    check_tie_share(int((~keep).sum()), n, "accept_prepare")
    for kg, kr in (("accept_len", "accept_len"), ("bonus", "bonus"),
                   ("new_seq_lens", "new_seq_len")):
        assert np.array_equal(_np(got[kg])[keep], ref[kr][keep]), kg
    r_ids, r_pos, r_loc, r_err = oracle.prepare_block(ref["bonus"], ref["new_seq_len"], table,
                                                      cfg.page, B_next, 77, None, num_pages)
    assert r_err == 0
    assert np.array_equal(_np(got["block_ids"])[keep], r_ids[keep])
    assert np.array_equal(_np(got["positions"])[keep], r_pos[keep])
    assert np.array_equal(_np(got["cache_loc"])[keep], r_loc[keep])


def test_accept_prepare_flags_a_block_past_the_table(gpu_lib):
    cfg = synth.config(1, bs=3)
    print_case("accept_prepare capacity")
    x = synth.make_accept_inputs(cfg, seed=5, bs=3)
    seq = np.array([0, 10, 20], np.int32)
    table = np.array([[0, 1], [2, 3], [4, -1]], np.int32)   # 32 slots, request 2 short
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = va.accept_prepare(*(to_dev(a) for a in (x.p, x.q, x.draft, x.u, seq, table)), 16, 8, 0,
                            5, err=err)
    torch.cuda.synchronize()
    ref = oracle.accept_batch(x.p, x.q, x.draft, x.u, seq)
    r = oracle.prepare_block(ref["bonus"], ref["new_seq_len"], table, 16, 8, 0, None, 5)
    assert np.array_equal(_np(got["cache_loc"]), r[2])
    assert int(err.item()) == r[3] and r[3] != 0


# ----------------------------------------------------- quadratic hand-off
def test_quadratic_handoff_golden(gpu_lib):
    fx = json.load(open(os.path.join(GOLDEN, "quadratic_handoff_small.json")))
    print_case("handoff golden")
    k = fx["k"]
    logits = np.array(fx["logits"], np.float32)
    cases = fx["cases"]
    bs = len(cases)
    lg = np.broadcast_to(logits, (bs,) + logits.shape).copy()
    acc = np.array([c["accept_len"] for c in cases], np.int32)
    bonus = np.full(bs, fx["bonus"], np.int32)
    for dt in ("f32", "bf16"):
        t = to_dev(synth.bf16_bits(lg)) if dt == "bf16" else to_dev(lg)
        out = va.quadratic_handoff(t, to_dev(acc), k, to_dev(bonus), fx["mask_token_id"])
        for b, c in enumerate(cases):
            assert out["next_draft"][b].cpu().tolist() == c["next_draft"], dt
            assert out["next_block"][b].cpu().tolist() == c["next_block"], dt


@pytest.mark.parametrize("k,bs,V,dt", [(4, 32, 151936, "bf16"), (7, 5, 4099, "f32"),
                                       (1, 17, 1000, "bf16"), (15, 3, 5003, "f32"),
                                       (21, 2, 2000, "bf16")])
def test_quadratic_handoff_matches_reference(gpu_lib, k, bs, V, dt):
    """The quadratic workload's size (k = 4, bs 32, bf16 logits of V =
    151936: real equal maxima occur), k = 7, 15 (a 256-row next block) and
    21 (the largest layout, 484 rows) and k = 1; every accept length from 0
    to k, and one out of range."""
    print_case("handoff", k, bs, V, dt)
    rng = np.random.default_rng(k * 100 + bs)
    n = (k + 1) ** 2
    lg = (rng.standard_normal((bs, n, V), dtype=np.float32) * 3).astype(np.float32)
    if dt == "bf16":
        bits = synth.bf16_bits(lg)
        vals = synth.bf16_to_f32(bits)
        dev = to_dev(bits)
    else:
        vals, dev = lg, to_dev(lg)
    acc = rng.integers(0, k + 1, size=bs).astype(np.int32)
    acc[0] = k + 1                                   # out of range: drafts of -1, flagged
    bonus = rng.integers(0, V, size=bs).astype(np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = va.quadratic_handoff(dev, to_dev(acc), k, to_dev(bonus), 9, err=err)
    nd, nb = _np(out["next_draft"]), _np(out["next_block"])
    for b in range(bs):
        r_d, r_b = quadratic.handoff(vals[b], acc[b], k, bonus[b], 9)
        assert nd[b].tolist() == r_d.tolist(), b
        if r_b is not None:
            assert nb[b].tolist() == r_b.tolist(), b
    assert int(err.item()) == va.ERR_TREE
    # without the block output only the drafts are written
    out2 = va.quadratic_handoff(dev, to_dev(acc), k)
    assert torch.equal(out2["next_draft"], out["next_draft"])


def test_two_quadratic_rounds_chain(gpu_lib):
    """Round 1 on the GPU: quadratic block preparation, attention over the
    layout, the accept of the spine drafts, the hand-off and the spine's
    commit; round 2 prepares its block from round 1's outputs on the GPU.
    Every output of the chain equals the reference chain fed the reference's
    own outputs (bit for bit for ids, positions, slots, tokens and pools;
    attention to 1e-5 in fp32)."""
    k = 3
    n = (k + 1) ** 2
    cfg = synth.config(8, bs=6, block=n, quad_k=k, hq=8, hkv=2, d=64, dtype="f32", ctx_lo=30,
                       ctx_hi=200, vocab=3001, k_spec=k)
    print_case("two quadratic rounds", cfg)
    x = synth.make_attn_inputs(cfg, seed=8)
    acc_in = synth.make_accept_inputs(cfg, seed=8)
    for b in (0, 1):      # request b rejects at test b: q one-hot at the draft, u near 1
        acc_in.q[b, b] = 0.0
        acc_in.q[b, b, acc_in.draft[b, b]] = 1.0
        acc_in.u[b, b] = np.float32(0.99999)
    par = synth.quadratic_parents(k)
    _, masks = synth.quadratic_layout(k)
    verified, _ = synth.make_round_state(cfg, 8)
    rng = np.random.default_rng(8)
    logits = rng.standard_normal((cfg.bs, n, cfg.vocab)).astype(np.float32)
    node_tokens = np.full((cfg.bs, n), 55, np.int32)
    node_tokens[:, quadratic.spine_path(k)] = acc_in.draft
    D = lambda a: to_dev(np.ascontiguousarray(a))
    seq, table = D(x.seq_lens), D(x.page_table)
    kp, vp = D(x.k_pool), D(x.v_pool)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids, pos, loc = va.prepare_tree(D(verified), seq, table, cfg.page, D(par), 55, x.num_pages,
                                    D(node_tokens), err=err)
    o = va.block_attn_tree(D(masks.view(np.int64)), D(x.q), kp, vp, table, seq,
                           int(x.seq_lens.max()) + n, err=err)
    acc = va.accept(D(acc_in.p), D(acc_in.q), D(acc_in.draft), D(acc_in.u), seq, err=err)
    ho = va.quadratic_handoff(D(logits), acc["accept_len"], k, acc["bonus"], 55, err=err)
    spine = np.full((cfg.bs, n), -1, np.int32)
    spine[:, :k] = quadratic.spine_path(k)
    freed = va.commit_kv(kp, vp, table, seq, acc["accept_len"], n, D(spine), err=err)
    ids2, pos2, loc2 = va.prepare_tree(acc["bonus"], acc["new_seq_lens"], table, cfg.page, D(par),
                                       55, x.num_pages, ho["next_block"], err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # the reference chain
    r1 = oracle.prepare_tree(verified, x.seq_lens, x.page_table, cfg.page, par, 55, node_tokens,
                             x.num_pages)
    for g, r in zip((ids, pos, loc), r1[:3]):
        assert np.array_equal(_np(g), r)
    ro, _ = oracle.block_attn_dense(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                    x.page_table, x.seq_lens, oracle.TREE, 0, tree=masks)
    assert np.max(np.abs(_np(o).astype(np.float64) - ro)) <= 1e-5
    ra = oracle.accept_batch(acc_in.p, acc_in.q, acc_in.draft, acc_in.u, x.seq_lens)
    assert not ra["tie_sample"].any()
    assert np.array_equal(_np(acc["accept_len"]), ra["accept_len"])
    assert np.array_equal(_np(acc["bonus"]), ra["bonus"])
    nb_ref = np.zeros((cfg.bs, n), np.int64)
    for b in range(cfg.bs):
        r_d, r_b = quadratic.handoff(logits[b], ra["accept_len"][b], k, ra["bonus"][b], 55)
        assert _np(ho["next_draft"][b]).tolist() == r_d.tolist()
        nb_ref[b] = r_b
    assert np.array_equal(_np(ho["next_block"]), nb_ref)
    rk, rv, rfreed = oracle.commit_kv(x.k_pool, x.v_pool, x.page_table, x.seq_lens,
                                      ra["accept_len"], spine, n)
    assert np.array_equal(_np(kp), rk) and np.array_equal(_np(vp), rv)
    assert np.array_equal(_np(freed), rfreed)
    r2 = oracle.prepare_tree(ra["bonus"], ra["new_seq_len"], x.page_table, cfg.page, par, 55,
                             nb_ref, x.num_pages)
    for g, r in zip((ids2, pos2, loc2), r2[:3]):
        assert np.array_equal(_np(g), r)
    assert set(ra["accept_len"].tolist()) >= {0, 1, k}


@pytest.mark.parametrize("name,over,logit_dt", [
    ("quadratic_workload", {}, "bf16"),
    ("k7_f32_d64_p32", dict(bs=5, block=64, quad_k=7, k_spec=7, hq=4, hkv=2, d=64, page=32,
                            dtype="f32", vocab=4099, ctx_lo=20, ctx_hi=300), "f32"),
    ("k1_bf16", dict(bs=9, block=4, quad_k=1, k_spec=1, vocab=1000, ctx_lo=3, ctx_hi=90),
     "bf16"),
    ("k15_bf16_block256", dict(bs=4, block=256, quad_k=15, k_spec=15, vocab=3001, ctx_lo=10,
                               ctx_hi=400), "bf16"),
])
def test_accept_quadratic_is_the_three_calls(gpu_lib, name, over, logit_dt):
    """spec_accept_quadratic equals spec_accept, spec_quadratic_handoff,
    spec_commit_kv (spine path) and spec_prepare_tree of the next block
    called in order -- every output, both pools, the released slots and the
    next block's positions and slots, bit for bit -- and the reference
    chain."""
    cfg = synth.config(8, **over)
    k, n, V = cfg.quad_k, cfg.block, cfg.vocab
    print_case("accept_quadratic", name, cfg.bs, k, V)
    x = synth.make_attn_inputs(cfg, seed=12)
    acc = synth.make_accept_inputs(cfg, seed=12)
    for b in (0, 1):      # requests rejecting at the first / second test
        if b < k:
            acc.q[b, b] = 0.0
            acc.q[b, b, acc.draft[b, b]] = 1.0
            acc.u[b, b] = np.float32(0.99999)
    rng = np.random.default_rng(12)
    lg = (rng.standard_normal((cfg.bs, n, V), dtype=np.float32) * 3).astype(np.float32)
    if logit_dt == "bf16":
        bits = synth.bf16_bits(lg)
        lvals, ldev = synth.bf16_to_f32(bits), to_dev(bits)
    else:
        lvals, ldev = lg, to_dev(lg)
    D = lambda a: to_dev(np.ascontiguousarray(a))
    seq, table = D(x.seq_lens), D(x.page_table)
    p, q, d, u = D(acc.p), D(acc.q), D(acc.draft), D(acc.u)
    # fused
    k1, v1 = D(x.k_pool), D(x.v_pool)
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = va.accept_quadratic(p, q, d, u, seq, ldev, k1, v1, table, 77, prepare_next=True,
                              err=e1)
    # the three calls
    k2, v2 = D(x.k_pool), D(x.v_pool)
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    a2 = va.accept(p, q, d, u, seq, err=e2)
    h2 = va.quadratic_handoff(ldev, a2["accept_len"], k, a2["bonus"], 77, err=e2)
    spine = np.full((cfg.bs, n), -1, np.int32)
    spine[:, :k] = quadratic.spine_path(k)
    f2 = va.commit_kv(k2, v2, table, seq, a2["accept_len"], n, D(spine), err=e2)
    par = D(synth.quadratic_parents(k))
    p2 = va.prepare_tree(a2["bonus"], a2["new_seq_lens"], table, cfg.page, par, 77, x.num_pages,
                         h2["next_block"], err=e2)
    # without the next block
    k3, v3 = D(x.k_pool), D(x.v_pool)
    got3 = va.accept_quadratic(p, q, d, u, seq, ldev, k3, v3, table, 77, next_block=False)
    torch.cuda.synchronize()
    for key in ("accept_len", "commit_len", "bonus", "out_tokens", "new_seq_lens"):
        assert torch.equal(got[key], a2[key]), key
        assert torch.equal(got3[key], a2[key]), key
    assert torch.equal(got["next_draft"], h2["next_draft"])
    assert torch.equal(got3["next_draft"], h2["next_draft"])
    assert torch.equal(got["next_block"], h2["next_block"])
    assert torch.equal(got["freed"], f2) and torch.equal(got3["freed"], f2)
    assert torch.equal(got["positions"], p2[1]) and torch.equal(got["cache_loc"], p2[2])
    assert "positions" not in got3
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(k3, k2) and torch.equal(v3, v2)
    assert int(e1.item()) == int(e2.item()) == 0
    # and the reference chain
    ra = oracle.accept_batch(acc.p, acc.q, acc.draft, acc.u, x.seq_lens)
    keep = ~ra["tie_sample"]
    check_tie_share(int((~keep).sum()), cfg.bs, "accept_quadratic")
    al = _np(got["accept_len"])
    assert np.array_equal(al[keep], ra["accept_len"][keep])
    assert np.array_equal(_np(got["bonus"])[keep], ra["bonus"][keep])
    for b in np.flatnonzero(keep):
        r_d, r_b = quadratic.handoff(lvals[b], ra["accept_len"][b], k, ra["bonus"][b], 77)
        assert _np(got["next_draft"][b]).tolist() == r_d.tolist(), b
        assert _np(got["next_block"][b]).tolist() == r_b.tolist(), b
    rk, rv, rfreed = oracle.commit_kv(x.k_pool, x.v_pool, x.page_table, x.seq_lens, al, spine, n)
    view = (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)) \
        if x.k_pool.dtype == np.uint16 else _np
    assert np.array_equal(view(k1), rk) and np.array_equal(view(v1), rv)
    assert np.array_equal(_np(got["freed"]), rfreed)
    _, r_pos, r_loc, r_err = oracle.prepare_tree(_np(got["bonus"]), _np(got["new_seq_lens"]),
                                                 x.page_table, cfg.page,
                                                 synth.quadratic_parents(k), 77, None,
                                                 x.num_pages)
    assert r_err == 0
    assert np.array_equal(_np(got["positions"]), r_pos)
    assert np.array_equal(_np(got["cache_loc"]), r_loc)
    assert (al == 0).any() and (al > 0).any()
