"""Pins for the float64 attention reference (CPU only).

Each test checks the reference against something other than itself: a
library routine (torch's scaled_dot_product_attention, scipy's logsumexp),
closed forms, the two independent forms against each other, or invariances
that the pages' mask definition implies.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from oracle import BIDIR, CAUSAL, MIXED
from verify_attention_amd import synth

MODES = [(BIDIR, 0), (CAUSAL, 0), (MIXED, 3), (MIXED, 0), (MIXED, 6)]


def tiny(bs=2, hq=4, hkv=2, d=16, page=4, block=6, ctx=(3, 13), dtype="f32", seed=0):
    cfg = synth.RoundConfig("tiny", bs=bs, hq=hq, hkv=hkv, d=d, page=page, block=block,
                            modes=(BIDIR,), dtype=dtype, ctx_lo=ctx[0], ctx_hi=ctx[1])
    return synth.make_attn_inputs(cfg, seed)


def run_dense(x, mode, nc):
    return oracle.block_attn_dense(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                   x.page_table, x.seq_lens, mode, nc)


def run_rows(x, mode, nc):
    return oracle.block_attn_rows(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                  x.page_table, x.seq_lens, mode, nc)


def gather_torch(x):
    """Logical K/V [bs, Hkv, Lmax+B, D] by tensor indexing (independent of the
    reference's per-token loop)."""
    cfg = x.cfg
    P = cfg.page
    kp = torch.from_numpy(x.as_f64("k_pool"))
    vp = torch.from_numpy(x.as_f64("v_pool")).transpose(2, 3)   # -> [pages, Hkv, P, D]
    out_k, out_v = [], []
    for b in range(cfg.bs):
        n = int(x.seq_lens[b]) + cfg.block
        pos = torch.arange(n)
        pages = torch.from_numpy(x.page_table[b].astype(np.int64))[pos // P]
        out_k.append(kp[pages, :, pos % P, :].transpose(0, 1))   # [Hkv, n, D]
        out_v.append(vp[pages, :, pos % P, :].transpose(0, 1))
    return out_k, out_v


@pytest.mark.parametrize("mode,nc", MODES)
def test_rows_and_dense_forms_agree(mode, nc):
    x = tiny(seed=1)
    o1, l1 = run_rows(x, mode, nc)
    o2, l2 = run_dense(x, mode, nc)
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(l1 - l2)) < 1e-12


@pytest.mark.parametrize("mode,nc", MODES)
def test_matches_torch_sdpa_with_explicit_mask(mode, nc):
    """Library routine: torch SDPA in float64 on CPU, fed the mask the pages
    draw (context columns all visible; rectangle / triangle / mixed block)."""
    x = tiny(seed=2, block=5, ctx=(0, 9))
    o, _ = run_dense(x, mode, nc)
    ks, vs = gather_torch(x)
    cfg = x.cfg
    g = cfg.hq // cfg.hkv
    q = torch.from_numpy(x.as_f64("q"))
    for b in range(cfg.bs):
        L = int(x.seq_lens[b])
        B = cfg.block
        allow = torch.ones(B, L + B, dtype=torch.bool)
        for i in range(B):
            for jb in range(B):
                if mode == CAUSAL:
                    allow[i, L + jb] = jb <= i
                elif mode == MIXED:
                    allow[i, L + jb] = (i >= nc) or (jb <= i)
        qb = q[b].transpose(0, 1)                        # [Hq, B, D]
        kb = ks[b].repeat_interleave(g, dim=0)           # [Hq, n, D]
        vb = vs[b].repeat_interleave(g, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=allow)
        got = torch.from_numpy(o[b]).transpose(0, 1)
        assert torch.max(torch.abs(ref - got)).item() < 1e-12


def test_lse_matches_scipy_logsumexp():
    x = tiny(seed=3)
    _, lse = run_rows(x, CAUSAL, 0)
    ks, _ = gather_torch(x)
    cfg = x.cfg
    g = cfg.hq // cfg.hkv
    q = x.as_f64("q")
    for b in range(cfg.bs):
        L = int(x.seq_lens[b])
        for h in range(cfg.hq):
            K = ks[b][h // g].numpy()
            for i in range(cfg.block):
                s = K[:L + i + 1] @ q[b, i, h] / np.sqrt(cfg.d)
                assert abs(logsumexp(s) - lse[b, i, h]) < 1e-12


@pytest.mark.parametrize("mode,nc", MODES)
def test_zero_query_gives_mean_of_visible_values(mode, nc):
    """Q = 0: every visible key scores 0, so each output row is the plain mean
    of the V rows it may see -- a different set per mode and row."""
    x = tiny(seed=4)
    x.q[...] = 0
    o, lse = run_dense(x, mode, nc)
    _, vs = gather_torch(x)
    cfg = x.cfg
    g = cfg.hq // cfg.hkv
    B = cfg.block
    for b in range(cfg.bs):
        L = int(x.seq_lens[b])
        for h in range(cfg.hq):
            V = vs[b][h // g].numpy()
            for i in range(B):
                if mode == BIDIR or (mode == MIXED and i >= nc):
                    n_vis = L + B
                else:
                    n_vis = L + i + 1
                want = V[:n_vis].mean(axis=0)
                assert np.max(np.abs(o[b, i, h] - want)) < 1e-13
                assert abs(lse[b, i, h] - np.log(n_vis)) < 1e-13


def test_single_token_no_context_returns_its_value():
    x = tiny(seed=5, block=1, ctx=(0, 0))
    for mode in (BIDIR, CAUSAL, MIXED):
        o, lse = run_rows(x, mode, 0)
        _, vs = gather_torch(x)
        g = x.cfg.hq // x.cfg.hkv
        for b in range(x.cfg.bs):
            for h in range(x.cfg.hq):
                assert np.array_equal(o[b, 0, h], vs[b][h // g][0].numpy())


def test_rank_one_keys_give_uniform_weights():
    """All keys equal: scores are equal, weights uniform, O = mean of V."""
    x = tiny(seed=6)
    x.k_pool[...] = x.k_pool[0, 0, 0, :]
    o, _ = run_dense(x, BIDIR, 0)
    _, vs = gather_torch(x)
    g = x.cfg.hq // x.cfg.hkv
    for b in range(x.cfg.bs):
        for h in range(x.cfg.hq):
            want = vs[b][h // g].numpy().mean(axis=0)
            assert np.max(np.abs(o[b, :, h] - want)) < 1e-12


def test_mode_special_cases():
    x = tiny(seed=7, block=6)
    B = x.cfg.block
    ob, _ = run_dense(x, BIDIR, 0)
    oc, _ = run_dense(x, CAUSAL, 0)
    # the last block row sees the whole block under both masks
    assert np.array_equal(ob[:, B - 1], oc[:, B - 1])
    # every other row differs between the rectangle and the triangle
    assert np.min(np.abs(ob[:, :B - 1] - oc[:, :B - 1]).max(axis=-1)) > 0
    # MIXED with every position clean is CAUSAL; with none clean it is BIDIR
    om_all, _ = run_dense(x, MIXED, B)
    om_none, _ = run_dense(x, MIXED, 0)
    assert np.array_equal(om_all, oc)
    assert np.array_equal(om_none, ob)
    # MIXED with 3 clean rows: clean rows follow CAUSAL, MASK rows follow BIDIR
    om3, _ = run_dense(x, MIXED, 3)
    assert np.array_equal(om3[:, :3], oc[:, :3])
    assert np.array_equal(om3[:, 3:], ob[:, 3:])
    # a single-token block is ordinary decode under every mask
    y = tiny(seed=8, block=1)
    outs = [run_dense(y, m, 0)[0] for m in (BIDIR, CAUSAL, MIXED)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_page_permutation_changes_nothing():
    """The same logical KV placed in two different physical page orders."""
    cfg = synth.RoundConfig("perm", bs=3, hq=4, hkv=2, d=8, page=4, block=5,
                            modes=(CAUSAL,), dtype="f32", ctx_lo=2, ctx_hi=17)
    a = synth.make_attn_inputs(cfg, 11, shuffle=False)
    b = synth.make_attn_inputs(cfg, 11, shuffle=True)
    # move a's pages to b's physical ids
    for r in range(cfg.bs):
        for n in range(a.page_table.shape[1]):
            pa, pb = a.page_table[r, n], b.page_table[r, n]
            if pa >= 0:
                b.k_pool[pb] = a.k_pool[pa]
                b.v_pool[pb] = a.v_pool[pa]
    oa, la = run_rows(a, CAUSAL, 0)
    ob, lb = run_rows(b, CAUSAL, 0)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_rows_subset_matches_full():
    x = tiny(seed=9)
    full, fl = run_rows(x, CAUSAL, 0)
    rows = [(1, 2, 3), (0, 5, 0)]
    part, pl = oracle.block_attn_rows(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                      x.page_table, x.seq_lens, CAUSAL, 0, rows=rows)
    for b, i, h in rows:
        assert np.array_equal(part[b, i, h], full[b, i, h])
        assert pl[b, i, h] == fl[b, i, h]


def test_planted_mask_mistake_is_caught(monkeypatch):
    """Discrimination check: a triangle that drops its diagonal (jb < i) in the
    reference must fail the zero-query closed form."""
    x = tiny(seed=10)
    x.q[...] = 0
    monkeypatch.setattr(oracle.attention, "visible",
                        lambda mode, i, jb, nc, tree_row=0: jb < i if mode == CAUSAL else True)
    o, _ = oracle.block_attn_rows(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                  x.page_table, x.seq_lens, CAUSAL, 0, rows=[(0, 2, 0)])
    _, vs = gather_torch(x)
    L = int(x.seq_lens[0])
    want = vs[0][0].numpy()[:L + 3].mean(axis=0)
    assert np.max(np.abs(o[0, 2, 0] - want)) > 1e-6


# ------------------------------------------------------------------ TREE mode
def test_tree_mode_chain_and_full_masks_reduce_to_causal_and_bidir():
    """A chain tree (parent[n] = n - 1) gives the causal triangle; all-ones
    rows give the rectangle."""
    x = tiny(seed=21, block=7, ctx=(0, 11))
    B = x.cfg.block
    chain = synth.tree_row_masks(np.arange(-1, B - 1, dtype=np.int32))
    full = np.full(B, (1 << B) - 1, dtype=np.uint64)
    for tree, mode in ((chain, CAUSAL), (full, BIDIR)):
        o_t, l_t = oracle.block_attn_dense(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                           x.page_table, x.seq_lens, oracle.TREE, 0, tree=tree)
        o_m, l_m = run_dense(x, mode, 0)
        assert np.max(np.abs(o_t - o_m)) < 1e-12 and np.max(np.abs(l_t - l_m)) < 1e-12


@pytest.mark.parametrize("block,depth,hq,page", [(9, 6, 4, 4), (80, 12, 2, 16), (150, 20, 2, 16)])
def test_tree_node_equals_causal_attention_over_its_root_path(block, depth, hq, page):
    """Defining property of tree attention: node n's output equals ordinary
    causal attention of the last row of a block laid out as the node's root
    path (ancestors in order, then n) after the same context. The path block
    is built as a separate paged cache, so this does not go through the tree
    mask at all. Blocks of 80 and 150 nodes take their masks as two and three
    64-bit words per row."""
    x = tiny(bs=2, hq=hq, hkv=2 if hq >= 2 else 1, d=16, page=page, block=block, ctx=(2, 10),
             seed=22)
    cfg = x.cfg
    B, P = cfg.block, cfg.page
    par, masks = synth.make_trees(dataclasses_replace(cfg, tree_depth=depth), 3)
    if B > 64:
        assert masks.shape == (cfg.bs, B, (B + 63) // 64)
    q64, k64, v64 = x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool")
    o_t, l_t = oracle.block_attn_rows(q64, k64, v64, x.page_table, x.seq_lens, oracle.TREE, 0,
                                      tree=masks)
    for b in range(cfg.bs):
        L = int(x.seq_lens[b])
        for n in range(B):
            path = []
            m = n
            while m >= 0:
                path.append(m)
                m = int(par[b][m])
            path = path[::-1]
            Lp = L + len(path)
            # a fresh identity-paged cache holding context, then the path's block rows
            npg = (Lp + P - 1) // P
            kp = np.zeros((npg, cfg.hkv, P, cfg.d))
            vp = np.zeros((npg, cfg.hkv, cfg.d, P))
            for t in range(Lp):
                src = t if t < L else L + path[t - L]
                pg, off = int(x.page_table[b, src // P]), src % P
                kp[t // P, :, t % P, :] = k64[pg, :, off, :]
                vp[t // P, :, :, t % P] = v64[pg, :, :, off]
            qp = np.zeros((1, len(path), cfg.hq, cfg.d))
            qp[0, -1] = q64[b, n]
            o_c, l_c = oracle.block_attn_rows(qp, kp, vp, np.arange(npg)[None, :],
                                              np.array([L]), CAUSAL, 0,
                                              rows=[(0, len(path) - 1, h) for h in range(cfg.hq)])
            assert np.max(np.abs(o_c[0, -1] - o_t[b, n])) < 1e-12, (b, n)
            assert np.max(np.abs(l_c[0, -1] - l_t[b, n])) < 1e-12, (b, n)


def test_tree_rows_and_dense_forms_agree_and_planted_bit_matters():
    x = tiny(seed=23, block=8, ctx=(1, 12))
    par, masks = synth.make_trees(dataclasses_replace(x.cfg, tree_depth=5), 4)
    args = (x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"), x.page_table, x.seq_lens,
            oracle.TREE, 0)
    o1, l1 = oracle.block_attn_rows(*args, tree=masks)
    o2, l2 = oracle.block_attn_dense(*args, tree=masks)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12
    # a shared [B] tree is the per-request tree broadcast
    o3, _ = oracle.block_attn_dense(*args, tree=masks[0])
    o4, _ = oracle.block_attn_dense(*args, tree=np.stack([masks[0]] * x.cfg.bs))
    assert np.max(np.abs(o3 - o4)) == 0.0
    # dropping one ancestor bit changes exactly that node's rows
    bad = masks.copy()
    n = int(np.argmax([bin(int(v)).count("1") for v in bad[0]]))
    top = int(bad[0][n]) & ~(1 << n)
    j = top.bit_length() - 1
    bad[0][n] = np.uint64(int(bad[0][n]) & ~(1 << j))
    o5, _ = oracle.block_attn_dense(*args, tree=bad)
    diff = np.abs(o5 - o2).max(axis=(2, 3))
    assert diff[0, n] > 1e-6 and np.delete(diff[0], n).max() == 0.0 and diff[1:].max() == 0.0


def dataclasses_replace(cfg, **kw):
    import dataclasses
    return dataclasses.replace(cfg, **kw)


# ---------------------------------------------------------- quadratic layout
def _separate_block(x, b, rows, L):
    """A fresh identity-paged cache of request b holding its context and then
    the listed block rows (positions L + r of the original block) in order."""
    cfg = x.cfg
    P = cfg.page
    k64, v64 = x.as_f64("k_pool"), x.as_f64("v_pool")
    n = L + len(rows)
    npg = (n + P - 1) // P
    kp = np.zeros((npg, cfg.hkv, P, cfg.d))
    vp = np.zeros((npg, cfg.hkv, cfg.d, P))
    for t in range(n):
        src = t if t < L else L + rows[t - L]
        pg, off = int(x.page_table[b, src // P]), src % P
        kp[t // P, :, t % P, :] = k64[pg, :, off, :]
        vp[t // P, :, :, t % P] = v64[pg, :, :, off]
    return kp, vp, np.arange(npg)[None, :]


@pytest.mark.parametrize("k", [1, 2, 4, 7, 8])
def test_quadratic_layout_rows_follow_their_definition(k):
    """Each row of the quadratic layout, run through the bitmask mode, equals
    the attention that defines it on a separately built block: spine token i
    is the last row of a causal block of spine tokens 0 .. i; a member of
    group G_j is a row of a bidirectional block made of spine tokens 0 .. j
    and the members of G_j."""
    n = (k + 1) ** 2
    x = tiny(bs=2, hq=4, hkv=2, d=16, page=4, block=n, ctx=(3, 9), seed=30 + k)
    cfg = x.cfg
    role, masks = synth.quadratic_layout(k)
    q64 = x.as_f64("q")
    o_q, l_q = oracle.block_attn_rows(q64, x.as_f64("k_pool"), x.as_f64("v_pool"), x.page_table,
                                      x.seq_lens, oracle.TREE, 0, tree=masks)
    for b in range(cfg.bs):
        L = int(x.seq_lens[b])
        for pos, (kind, j, m) in enumerate(role):
            spine = [t * (k + 1) for t in range(j + 1)]
            if kind == "spine":
                rows, mode, at = spine, CAUSAL, len(spine) - 1
            else:
                group = [j * (k + 1) + 1 + t for t in range(k)]
                rows, mode, at = spine + group, BIDIR, len(spine) + m
            kp, vp, tab = _separate_block(x, b, rows, L)
            qp = np.zeros((1, len(rows), cfg.hq, cfg.d))
            qp[0, at] = q64[b, pos]
            o_c, l_c = oracle.block_attn_rows(qp, kp, vp, tab, np.array([L]), mode, 0,
                                              rows=[(0, at, h) for h in range(cfg.hq)])
            assert np.max(np.abs(o_c[0, at] - o_q[b, pos])) < 1e-12, (b, pos)
            assert np.max(np.abs(l_c[0, at] - l_q[b, pos])) < 1e-12, (b, pos)


def test_quadratic_layout_shape_and_limits():
    role, masks = synth.quadratic_layout(3)
    assert len(role) == 16 and role[0] == ("spine", 0, 0) and role[4] == ("spine", 1, 0)
    assert int(masks[0]) == 1 and int(masks[8]) == 1 | 16 | 256
    # group G_1 (positions 5, 6, 7) sees spine 0, 4 and itself
    assert int(masks[6]) == 1 | 16 | (7 << 5)
    # past 64 positions the rows are words: k = 8 has 81 rows of two words,
    # spine token 8 (position 72) sees spine positions 0, 9, .., 63 and itself;
    # member 7 of G_8 (position 80) also sees the members 73 .. 80
    role, masks = synth.quadratic_layout(8)
    assert masks.shape == (1, 81, 2) and role[72] == ("spine", 8, 0)
    row = lambda r: int(masks[0, r, 0]) | (int(masks[0, r, 1]) << 64)
    assert row(72) == sum(1 << (9 * t) for t in range(9))
    assert role[80] == ("mask", 8, 7) and row(80) == row(72) | sum(1 << t for t in range(73, 81))
    role, masks = synth.quadratic_layout(21)
    assert masks.shape == (1, 484, 8)
    with pytest.raises(ValueError):
        synth.quadratic_layout(22)


def test_mask_words_agree_with_one_word_rows_and_wide_chains_are_causal():
    """Up to 64 nodes the word layout [bs, B, 1] is the one-word layout; past
    64 nodes a chain tree in words is the causal triangle and all-ones words
    the rectangle (B = 70 and 129: the second and third words carry the last
    rows' bits)."""
    x = tiny(seed=24, block=40, ctx=(0, 9))
    par, masks = synth.make_trees(dataclasses_replace(x.cfg, tree_depth=10), 5)
    words = np.stack([synth.tree_row_words(p) for p in par])
    assert words.shape == (x.cfg.bs, 40, 1) and np.array_equal(words[:, :, 0], masks)
    args = (x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"), x.page_table, x.seq_lens,
            oracle.TREE, 0)
    o1, _ = oracle.block_attn_dense(*args, tree=masks)
    o2, _ = oracle.block_attn_dense(*args, tree=words)
    assert np.max(np.abs(o1 - o2)) == 0.0
    for B in (70, 129):
        xw = tiny(seed=25, hq=2, hkv=1, d=8, page=16, block=B, ctx=(0, 20))
        chain = synth.tree_row_words(np.arange(-1, B - 1, dtype=np.int32))[None]
        W = (B + 63) // 64
        full = np.zeros((1, B, W), dtype=np.uint64)
        for w in range(W):
            nb = min(64, B - 64 * w)
            full[:, :, w] = np.uint64((1 << nb) - 1)
        a = (xw.as_f64("q"), xw.as_f64("k_pool"), xw.as_f64("v_pool"), xw.page_table,
             xw.seq_lens)
        for tree, mode in ((chain, CAUSAL), (full, BIDIR)):
            o_t, l_t = oracle.block_attn_dense(*a, oracle.TREE, 0, tree=tree)
            o_m, l_m = oracle.block_attn_dense(*a, mode, 0)
            assert np.max(np.abs(o_t - o_m)) < 1e-12 and np.max(np.abs(l_t - l_m)) < 1e-12


def test_planted_bit_in_a_later_word_matters():
    """Clearing one ancestor bit held in the second word of a row changes that
    node's rows only."""
    x = tiny(bs=1, seed=26, hq=2, hkv=1, d=8, page=16, block=100, ctx=(5, 6))
    par = np.arange(-1, 99, dtype=np.int32)          # a chain: node n sees 0 .. n
    words = synth.tree_row_words(par)[None].copy()
    args = (x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"), x.page_table, x.seq_lens,
            oracle.TREE, 0)
    o1, _ = oracle.block_attn_dense(*args, tree=words)
    words[0, 90, 1] &= ~np.uint64(1 << (70 - 64))   # row 90 loses ancestor 70
    o2, _ = oracle.block_attn_dense(*args, tree=words)
    diff = np.abs(o2 - o1).max(axis=(2, 3))[0]
    assert diff[90] > 1e-6 and np.delete(diff, 90).max() == 0.0
