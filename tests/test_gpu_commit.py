"""GPU parity of spec_commit_kv through the C ABI: the K/V pools after the
commit and the released slots must equal the float64 CPU reference's bit for
bit (the commit only moves stored values). Accepted paths come from the CPU
reference's tree accept or are constructed (deepest first-child chains,
overlapping moves), never from the GPU."""
import numpy as np
import pytest
import torch

import oracle
import verify_attention_amd as va
from verify_attention_amd import synth
from _support import print_case, to_dev

pytestmark = pytest.mark.gpu


def run_commit(x, depth, path, B, err=None):
    k, v = to_dev(x.k_pool), to_dev(x.v_pool)
    freed = va.commit_kv(k, v, to_dev(x.page_table), to_dev(x.seq_lens),
                         to_dev(np.asarray(depth, np.int32)), B,
                         None if path is None else to_dev(np.asarray(path, np.int32)), err=err)
    torch.cuda.synchronize()
    view = (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)) \
        if x.k_pool.dtype == np.uint16 else (lambda t: t.cpu().numpy())
    return view(k), view(v), freed.cpu().numpy()


def check(x, depth, path, B):
    k, v, freed = run_commit(x, depth, path, B)
    rk, rv, rfreed = oracle.commit_kv(x.k_pool, x.v_pool, x.page_table, x.seq_lens, depth, path, B)
    assert np.array_equal(freed, rfreed)
    assert np.array_equal(k, rk) and np.array_equal(v, rv)
    moved = sum(int(d) for d in depth)
    print(f"commit: {len(depth)} requests, {moved} rows moved, max depth {max(depth)}", flush=True)


def deepest_paths(par, B):
    depth, path = [], []
    for p in par:
        chain, node = [], 0
        while True:
            kids = oracle.tree_children(p, node)
            if not kids:
                break
            node = kids[0]
            chain.append(node)
        depth.append(len(chain))
        path.append(chain + [-1] * (B - len(chain)))
    return np.array(depth, np.int32), np.array(path, np.int32)


def test_commit_tree_verify_workload():
    # the tree verify workload (bs 32, 32-node trees, 8 KV heads, D 128, bf16,
    # page 16): paths from the reference tree accept, then the deepest chains
    cfg = synth.config(6)
    print_case("commit tree workload")
    x = synth.make_attn_inputs(cfg, seed=2)
    par, _ = synth.make_trees(cfg, 2)
    ti = synth.make_tree_accept_inputs(cfg, 2, par)
    acc = [oracle.tree_accept_request(ti.parent[b], ti.token[b], ti.p[b], ti.u[b], x.seq_lens[b])
           for b in range(cfg.bs)]
    depth = np.array([a["accept_len"] for a in acc], np.int32)
    path = np.stack([a["path_nodes"] for a in acc]).astype(np.int32)
    check(x, depth, path, cfg.block)
    depth, path = deepest_paths(par, cfg.block)
    assert depth.max() >= 8
    check(x, depth, path, cfg.block)


@pytest.mark.parametrize("dtype,d,page", [("f32", 64, 32), ("bf16", 64, 16), ("f32", 128, 16)])
def test_commit_small_shapes_and_overlapping_moves(dtype, d, page):
    cfg = synth.config(6, bs=5, block=12, hq=4, hkv=2, d=d, page=page, dtype=dtype, ctx_lo=17,
                       ctx_hi=70, tree_depth=6)
    print_case("commit small", dtype, d, page)
    x = synth.make_attn_inputs(cfg, seed=7)
    depth = np.array([0, 1, 3, 11, 4], np.int32)
    path = np.full((5, 12), -1, np.int32)
    path[1, :1] = [5]
    path[2, :3] = [2, 3, 4]                # every source but the first is another destination
    path[3, :11] = np.arange(1, 12)        # the full chain: nothing moves
    path[4, :4] = [3, 5, 6, 11]
    check(x, depth, path, cfg.block)


@pytest.mark.parametrize("cid,over", [
    (10, dict(bs=3, vocab=64)),
    (6, dict(bs=2, block=512, tree_depth=512, hq=8, hkv=2, d=64, dtype="f32", ctx_lo=3,
             ctx_hi=300, page=32)),
])
def test_commit_wide_blocks(cid, over):
    """Blocks of 481 and 512 nodes: the deepest first-child chains, every
    other node (rows k <- 2k, more than one round of 64 rows), and random
    increasing paths of up to 511 rows."""
    cfg = synth.config(cid, **over)
    print_case("commit wide", cid, cfg.block, cfg.dtype)
    x = synth.make_attn_inputs(cfg, seed=4)
    par, _ = synth.make_trees(cfg, 4)
    B = cfg.block
    depth, path = deepest_paths(par, B)
    check(x, depth, path, B)
    rng = np.random.default_rng(cid)
    depth = np.zeros(cfg.bs, np.int32)
    path = np.full((cfg.bs, B), -1, np.int32)
    for b in range(cfg.bs):
        if b == 0:
            d, p = (B - 1) // 2, 2 * np.arange(1, (B - 1) // 2 + 1)
        else:
            d = int(rng.integers(65, B))
            p = np.sort(rng.choice(np.arange(1, B), size=d, replace=False))
        depth[b], path[b, :d] = d, p
    check(x, depth, path, B)


def test_commit_linear_verify_moves_nothing():
    cfg = synth.config(2, bs=8)
    print_case("commit linear")
    x = synth.make_attn_inputs(cfg, seed=3)
    depth = np.array([0, 1, 5, 15, 7, 2, 9, 15], np.int32)
    check(x, depth, None, cfg.block)


def test_commit_flags_bad_requests_and_leaves_them_unchanged():
    cfg = synth.config(6, bs=4, block=8, hq=4, hkv=2, d=64, dtype="f32", ctx_lo=20, ctx_hi=20,
                       tree_depth=5)
    print_case("commit error paths")
    x = synth.make_attn_inputs(cfg, seed=9)
    depth = np.array([2, 9, 2, 2], np.int32)   # request 1: depth past the block
    path = np.full((4, 8), -1, np.int32)
    path[0, :2] = [1, 3]
    path[2, :2] = [3, 3]                       # not increasing
    path[3, :2] = [2, 6]
    seq = x.seq_lens.copy()
    x.seq_lens[3] = x.page_table.shape[1] * cfg.page   # request 3: block past the page table
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    k, v, freed = run_commit(x, depth, path, cfg.block, err=err)
    e = int(err.item())
    assert e & va.ERR_TREE and e & va.ERR_CAPACITY
    assert (freed[1:] == -1).all()
    # only request 0 changed: compare with the reference committing request 0 alone
    x.seq_lens = seq
    rk, rv, rfreed = oracle.commit_kv(x.k_pool, x.v_pool, x.page_table, x.seq_lens,
                                      np.array([2, 0, 0, 0]), path, cfg.block)
    assert np.array_equal(k, rk) and np.array_equal(v, rv)
    assert np.array_equal(freed[0], rfreed[0])


def _tree_case(cfg, seed):
    x = synth.make_attn_inputs(cfg, seed=seed)
    par, _ = synth.make_trees(cfg, seed)
    ti = synth.make_tree_accept_inputs(cfg, seed, par)
    return x, ti


def _pools(x):
    return to_dev(x.k_pool), to_dev(x.v_pool)


def _host(t, bf16):
    return t.view(torch.int16).cpu().numpy().view(np.uint16) if bf16 else t.cpu().numpy()


@pytest.mark.parametrize("cid,over", [(6, {}), (6, dict(bs=5, block=12, hq=4, hkv=2, d=64, page=32,
                                                          dtype="f32", ctx_lo=17, ctx_hi=70,
                                                          tree_depth=6, vocab=300)),
                                      (10, dict(bs=4, vocab=500))])
def test_accept_tree_commit_equals_the_two_calls(cid, over):
    """spec_accept_tree_commit gives exactly the outputs, pools and released
    slots of spec_accept_tree followed by spec_commit_kv, and the pools equal
    the reference commit of the reference accept's path."""
    cfg = synth.config(cid, **over)
    print_case("accept_tree_commit", cfg.name, over)
    x, ti = _tree_case(cfg, 2)
    bf16 = x.k_pool.dtype == np.uint16
    args = [to_dev(a) for a in (ti.parent, ti.token, ti.p, ti.u)]
    seq, tab = to_dev(x.seq_lens), to_dev(x.page_table)
    # two calls
    k1, v1 = _pools(x)
    out1 = va.accept_tree(*args, seq)
    freed1 = va.commit_kv(k1, v1, tab, seq, out1["accept_len"], cfg.block, out1["path_nodes"])
    # one call
    k2, v2 = _pools(x)
    out2 = va.accept_tree_commit(*args, seq, k2, v2, tab)
    torch.cuda.synchronize()
    for key in ("accept_len", "commit_len", "bonus", "out_tokens", "path_nodes", "new_seq_lens"):
        assert torch.equal(out1[key], out2[key]), key
    assert torch.equal(freed1, out2["freed"])
    assert np.array_equal(_host(k1, bf16), _host(k2, bf16))
    assert np.array_equal(_host(v1, bf16), _host(v2, bf16))
    # and the reference: commit of the reference accept's path
    acc = [oracle.tree_accept_request(ti.parent[b], ti.token[b], ti.p[b], ti.u[b], x.seq_lens[b])
           for b in range(cfg.bs)]
    depth = np.array([a["accept_len"] for a in acc], np.int32)
    path = np.stack([a["path_nodes"] for a in acc]).astype(np.int32)
    assert np.array_equal(out2["accept_len"].cpu().numpy(), depth)
    rk, rv, rfreed = oracle.commit_kv(x.k_pool, x.v_pool, x.page_table, x.seq_lens, depth, path,
                                      cfg.block)
    assert np.array_equal(_host(k2, bf16), rk) and np.array_equal(_host(v2, bf16), rv)
    assert np.array_equal(out2["freed"].cpu().numpy(), rfreed)
    print(f"accept_tree_commit: depths {depth.tolist()[:8]}...", flush=True)


def test_accept_tree_commit_flags_a_block_past_the_table():
    cfg = synth.config(6, bs=4, block=8, hq=4, hkv=2, d=64, dtype="f32", ctx_lo=20, ctx_hi=20,
                       tree_depth=5, vocab=64)
    print_case("accept_tree_commit capacity")
    x, ti = _tree_case(cfg, 9)
    x.seq_lens[2] = x.page_table.shape[1] * cfg.page   # request 2: block past its table
    args = [to_dev(a) for a in (ti.parent, ti.token, ti.p, ti.u)]
    seq, tab = to_dev(x.seq_lens), to_dev(x.page_table)
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    k1, v1 = _pools(x)
    out1 = va.accept_tree(*args, seq, err=e1)
    freed1 = va.commit_kv(k1, v1, tab, seq, out1["accept_len"], cfg.block, out1["path_nodes"],
                          err=e1)
    k2, v2 = _pools(x)
    out2 = va.accept_tree_commit(*args, seq, k2, v2, tab, err=e2)
    torch.cuda.synchronize()
    assert int(e2.item()) & va.ERR_CAPACITY and int(e1.item()) == int(e2.item())
    assert torch.equal(freed1, out2["freed"]) and (out2["freed"][2] == -1).all()
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
