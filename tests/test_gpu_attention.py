"""GPU parity of block_attn against the float64 CPU reference.

Agreement required: max abs error <= 1e-2 for bf16 inputs, <= 1e-5 for fp32
inputs (outputs written in the input dtype); lse within 1e-3 (bf16) / 1e-5.
Small cases compare every output row with the dense reference; full-size
workloads compare sampled rows computed one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import verify_attention_amd as va
from verify_attention_amd import synth
from _support import AttnCase, print_case, to_f64

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "f32": 1e-5}
LSE_TOL = {"bf16": 1e-3, "f32": 1e-5}


def run(case, mode, max_kv=None, nc_per_req=False, err=None):
    x = case.x
    lse = torch.empty((x.cfg.bs, x.cfg.block, x.cfg.hq), dtype=torch.float32, device="cuda")
    o = va.block_attn(mode, case.q, case.k, case.v, case.table, case.seq,
                      max_kv or case.max_kv, n_causal=x.cfg.n_causal,
                      n_causal_per_req=case.nc if nc_per_req else None, lse=lse, err=err)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy().astype(np.float64)


def ref_dense(x, mode, nc):
    return oracle.block_attn_dense(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                   x.page_table, x.seq_lens, mode, nc)


def check_all(x, got_o, got_lse, mode, nc):
    ro, rl = ref_dense(x, mode, nc)
    eo = np.max(np.abs(got_o - ro))
    el = np.max(np.abs(got_lse - rl))
    assert eo <= TOL[x.cfg.dtype], f"max abs error {eo}"
    assert el <= LSE_TOL[x.cfg.dtype], f"lse error {el}"
    return eo


SMALL = [
    # (name, config id, overrides, mode)
    ("tiny_f32_bidir", 1, {}, synth.BIDIR),
    ("tiny_f32_causal", 1, {}, synth.CAUSAL),
    ("tiny_f32_mixed", 1, dict(n_causal=3), synth.MIXED),
    ("verify_bs2", 2, dict(bs=2), synth.CAUSAL),
    ("verify_bs3_bidir", 2, dict(bs=3), synth.BIDIR),
    ("draft_b32_p32_ragged", 3, dict(bs=3, ctx_lo=700, ctx_hi=1500), synth.BIDIR),
    ("ragged_verify_bs5", 4, dict(bs=5, ctx_lo=30, ctx_hi=1300), synth.CAUSAL),
    ("mixed_bs2", 5, dict(bs=2, ctx_lo=900, ctx_hi=1100), synth.MIXED),
    ("no_context", 2, dict(bs=2, ctx_lo=0, ctx_hi=0), synth.CAUSAL),
    ("short_ctx_mixed", 5, dict(bs=3, ctx_lo=1, ctx_hi=40), synth.MIXED),
    ("single_token_block", 2, dict(bs=3, block=1, ctx_lo=5, ctx_hi=300), synth.CAUSAL),
    ("g1_b8_d64", 1, dict(bs=4, hq=4, hkv=4, dtype="bf16", ctx_lo=100, ctx_hi=700), synth.BIDIR),
    ("g2_b40_d128", 2, dict(bs=2, hq=4, hkv=2, block=40, ctx_lo=50, ctx_hi=400), synth.CAUSAL),
    ("f32_d128_m64", 2, dict(bs=2, dtype="f32", ctx_lo=200, ctx_hi=600), synth.CAUSAL),
    # more than 128 query rows per KV head: row groups, each streaming the keys
    ("rows160_g4_causal", 2, dict(bs=2, block=40, ctx_lo=50, ctx_hi=400), synth.CAUSAL),
    ("rows512_g4_bidir_p32", 3, dict(bs=2, block=128, ctx_lo=300, ctx_hi=700), synth.BIDIR),
    ("rows200_mixed", 5, dict(bs=2, block=50, n_causal=20, ctx_lo=100, ctx_hi=500), synth.MIXED),
    ("rows144_f32_d64", 1, dict(bs=2, block=72, ctx_lo=40, ctx_hi=300), synth.BIDIR),
    ("rows129_g3_ragged", 4, dict(bs=3, hq=24, hkv=8, block=43, ctx_lo=20, ctx_hi=900),
     synth.CAUSAL),
    ("rows2048_g8_max", 2, dict(bs=1, hq=64, hkv=8, block=256, ctx_lo=90, ctx_hi=90), synth.CAUSAL),
]


@pytest.mark.parametrize("name,cid,over,mode", SMALL, ids=[s[0] for s in SMALL])
def test_small_all_rows(gpu_lib, name, cid, over, mode):
    cfg = synth.config(cid, **over)
    print_case("block_attn", name, cfg)
    x = synth.make_attn_inputs(cfg, seed=100 + cid)
    case = AttnCase(x)
    o, lse = run(case, mode)
    check_all(x, o, lse, mode, cfg.n_causal)


def test_mixed_per_request_clean_counts(gpu_lib):
    """I-DLM batches mix verify rows (N clean positions) with cold starts (1
    clean position): n_causal differs per request."""
    cfg = synth.config(5, bs=6, ctx_lo=64, ctx_hi=700)
    print_case("block_attn mixed per-request", cfg)
    x = synth.make_attn_inputs(cfg, seed=7, n_causal_per_req=True)
    case = AttnCase(x)
    o, lse = run(case, synth.MIXED, nc_per_req=True)
    ro = np.empty_like(o)
    rl = np.empty_like(lse)
    for b in range(cfg.bs):
        one = synth.AttnInputs(cfg, x.seq_lens[b:b + 1], x.page_table[b:b + 1], x.num_pages,
                               x.q[b:b + 1], x.k_pool, x.v_pool, x.n_causal[b:b + 1])
        r = ref_dense(one, synth.MIXED, int(x.n_causal[b]))
        ro[b], rl[b] = r[0][0], r[1][0]
    assert np.max(np.abs(o - ro)) <= TOL["bf16"]
    assert np.max(np.abs(lse - rl)) <= LSE_TOL["bf16"]


def test_poisoned_tail_slots_never_read(gpu_lib):
    """Slots past L_b + B hold NaN; no output may change or turn NaN."""
    cfg = synth.config(4, bs=4, ctx_lo=17, ctx_hi=900)
    print_case("block_attn poisoned tail", cfg)
    x = synth.make_attn_inputs(cfg, seed=3, poison_tail=True)
    o, lse = run(AttnCase(x), synth.CAUSAL)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    check_all(x, o, lse, synth.CAUSAL, 0)


def test_split_kv_plans_agree(gpu_lib):
    """A loose host upper bound on the context length makes the planner split
    every (request, KV head) many ways (most splits then hold no key): the
    result must not change beyond fp32 rounding."""
    cfg = synth.config(2, bs=2, ctx_lo=1500, ctx_hi=2600)
    print_case("block_attn split plans", cfg)
    x = synth.make_attn_inputs(cfg, seed=5)
    case = AttnCase(x)
    o1, l1 = run(case, synth.CAUSAL)
    o2, l2 = run(case, synth.CAUSAL, max_kv=9216)
    o3, l3 = run(case, synth.CAUSAL, max_kv=20000)
    assert va.attn_workspace_bytes(2, 16, 32, 8, 128, 20000) > va.attn_workspace_bytes(2, 16, 32, 8, 128, 2616)
    assert np.max(np.abs(o1 - o2)) <= 2 ** -7 and np.max(np.abs(o1 - o3)) <= 2 ** -7
    assert np.max(np.abs(l1 - l3)) <= 1e-4
    check_all(x, o3, l3, synth.CAUSAL, 0)
    # so loose a bound that the balanced schedule is chosen: the few stage
    # pairs are shared by 256 workgroups (most ranges empty, most units cut)
    o4, l4 = run(case, synth.CAUSAL, max_kv=65536)
    assert np.max(np.abs(o1 - o4)) <= 2 ** -7 and np.max(np.abs(l1 - l4)) <= 1e-4
    check_all(x, o4, l4, synth.CAUSAL, 0)
    # repeated calls on one workspace reproduce the balanced result exactly
    ws = va.workspace(va.attn_workspace_bytes(2, 16, 32, 8, 128, 65536))
    for _ in range(2):
        o = va.block_attn(synth.CAUSAL, case.q, case.k, case.v, case.table, case.seq, 65536, ws=ws)
        torch.cuda.synchronize()
        assert np.max(np.abs(to_f64(o) - o4)) == 0.0


def test_row_groups_every_schedule(gpu_lib):
    """512 query rows per KV head (4 row groups): the split plan, a loose
    bound that splits every unit many ways, and the balanced schedule (row
    group teams, cut units merged per group) all match the reference."""
    cfg = synth.config(3, bs=3, block=128, ctx_lo=900, ctx_hi=2100)
    print_case("block_attn row groups, every schedule", cfg)
    x = synth.make_attn_inputs(cfg, seed=21)
    case = AttnCase(x)
    o1, l1 = run(case, synth.BIDIR)
    check_all(x, o1, l1, synth.BIDIR, 0)
    o2, l2 = run(case, synth.BIDIR, max_kv=20000)
    check_all(x, o2, l2, synth.BIDIR, 0)
    o3, l3 = run(case, synth.BIDIR, max_kv=65536 * 4)
    check_all(x, o3, l3, synth.BIDIR, 0)
    assert np.max(np.abs(o1 - o3)) <= 2 ** -7 and np.max(np.abs(l1 - l3)) <= 1e-4


def test_bad_page_id_is_flagged(gpu_lib):
    cfg = synth.config(2, bs=2, ctx_lo=300, ctx_hi=300)
    print_case("block_attn bad page id", cfg)
    x = synth.make_attn_inputs(cfg, seed=9)
    x.page_table[1, 3] = x.num_pages + 5
    case = AttnCase(x)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, _ = run(case, synth.CAUSAL, err=err)
    assert int(err.item()) & va.ERR_SLOT
    # request 0 is untouched by request 1's bad entry
    good = synth.AttnInputs(cfg, x.seq_lens[:1], x.page_table[:1], x.num_pages, x.q[:1],
                            x.k_pool, x.v_pool, x.n_causal[:1])
    ro, _ = ref_dense(good, synth.CAUSAL, 0)
    assert np.max(np.abs(o[:1] - ro)) <= TOL["bf16"]


BALANCED = [
    # (name, config id, overrides, mode, per-request n_causal): batches large
    # enough (units x stages of the longest request >= 32768) for the balanced
    # schedule, with ragged lengths so that share boundaries cut units
    ("g1_b8_d64_ragged", 2, dict(bs=64, hq=8, hkv=8, d=64, block=8, ctx_lo=1, ctx_hi=6000),
     synth.CAUSAL, False),
    ("g4_b16_d128_mixed_nc", 5, dict(bs=128, hq=8, hkv=2, ctx_lo=1, ctx_hi=4500), synth.MIXED,
     True),
    ("g4_b32_d128_p32_bidir", 3, dict(bs=128, hq=8, hkv=2, ctx_lo=1, ctx_hi=4100), synth.BIDIR,
     False),
    ("f32_d64_ragged", 1, dict(bs=64, hq=4, hkv=4, block=16, ctx_lo=1, ctx_hi=5000),
     synth.CAUSAL, False),
]


@pytest.mark.parametrize("name,cid,over,mode,nc_req", BALANCED, ids=[s[0] for s in BALANCED])
def test_balanced_schedule_all_rows(gpu_lib, name, cid, over, mode, nc_req):
    cfg = synth.config(cid, **over)
    print_case("block_attn balanced", name, cfg)
    x = synth.make_attn_inputs(cfg, seed=11 + cid, n_causal_per_req=nc_req)
    case = AttnCase(x)
    steps = (case.max_kv + 31) // 32
    assert cfg.bs * cfg.hkv * steps >= 32768
    o, lse = run(case, mode, nc_per_req=nc_req)
    if not nc_req:
        check_all(x, o, lse, mode, cfg.n_causal)
        return
    q64, k64, v64 = x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool")
    for b in range(cfg.bs):
        ro, rl = oracle.block_attn_dense(q64[b:b + 1], k64, v64, x.page_table[b:b + 1],
                                         x.seq_lens[b:b + 1], mode, int(x.n_causal[b]))
        assert np.max(np.abs(o[b] - ro[0])) <= TOL[cfg.dtype], b
        assert np.max(np.abs(lse[b] - rl[0])) <= LSE_TOL[cfg.dtype], b


def run_tree(case, masks, max_kv=None):
    x = case.x
    if masks.ndim == 3 and masks.shape[0] == 1 and x.cfg.bs > 1:
        masks = masks[0]     # one shared tree of mask words: [B, W]
    tm = torch.from_numpy(np.ascontiguousarray(masks).view(np.int64)).to("cuda")
    lse = torch.empty((x.cfg.bs, x.cfg.block, x.cfg.hq), dtype=torch.float32, device="cuda")
    o = va.block_attn_tree(tm, case.q, case.k, case.v, case.table, case.seq,
                           max_kv or case.max_kv, lse=lse)
    torch.cuda.synchronize()
    return to_f64(o), lse.cpu().numpy().astype(np.float64)


TREES = [
    # (name, config id, overrides, one tree per request)
    ("b32_g4_d128_per_request", 6, dict(bs=4, ctx_lo=100, ctx_hi=900), True),
    ("b64_g2_d64_shared", 6, dict(bs=3, hq=4, hkv=2, d=64, block=64, tree_depth=20, ctx_lo=0,
                                  ctx_hi=600), False),
    ("b16_g4_f32_d64", 6, dict(bs=3, hq=8, hkv=2, d=64, block=16, tree_depth=8, dtype="f32",
                               ctx_lo=40, ctx_hi=500), True),
    ("b32_p32_balanced", 6, dict(bs=128, hq=8, hkv=2, page=32, ctx_lo=1, ctx_hi=4200), True),
    # more than 64 nodes: W = ceil(B / 64) mask words per row, staged in LDS
    ("b80_g4_d128_rowgroups", 6, dict(bs=3, block=80, tree_depth=20, ctx_lo=50, ctx_hi=700),
     True),
    ("b150_g2_d64_shared", 6, dict(bs=3, hq=4, hkv=2, d=64, block=150, tree_depth=40, ctx_lo=0,
                                   ctx_hi=500), False),
    ("b200_g1_p32", 6, dict(bs=2, hq=2, hkv=2, page=32, block=200, tree_depth=30, ctx_lo=1,
                            ctx_hi=400), True),
    ("b100_f32_d128_two_tiles", 6, dict(bs=2, hq=8, hkv=2, block=100, tree_depth=16,
                                        dtype="f32", ctx_lo=20, ctx_hi=300), True),
    ("b512_g4_max", 6, dict(bs=2, hq=8, hkv=2, block=512, tree_depth=16, ctx_lo=0, ctx_hi=200),
     True),
    # the balanced schedule (a workgroup's pieces span requests: the mask
    # words are restaged per request)
    ("b72_g4_balanced", 6, dict(bs=96, hq=8, hkv=2, block=72, tree_depth=20, ctx_lo=1,
                                ctx_hi=3000), True),
    ("b200_g1_shared_balanced", 6, dict(bs=128, hq=2, hkv=2, block=200, tree_depth=30, ctx_lo=1,
                                        ctx_hi=4000), False),
    ("b66_f32_d64_balanced", 6, dict(bs=96, hq=4, hkv=2, d=64, block=66, tree_depth=12,
                                     dtype="f32", ctx_lo=1, ctx_hi=3000), True),
]


@pytest.mark.parametrize("name,cid,over,per_req", TREES, ids=[t[0] for t in TREES])
def test_tree_mode_all_rows(gpu_lib, name, cid, over, per_req):
    cfg = synth.config(cid, **over)
    print_case("block_attn_tree", name, cfg)
    x = synth.make_attn_inputs(cfg, seed=31)
    _, masks = synth.make_trees(cfg, 31, per_request=per_req)
    o, lse = run_tree(AttnCase(x), masks)
    ro, rl = oracle.block_attn_dense(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                     x.page_table, x.seq_lens, oracle.TREE, 0, tree=masks)
    assert np.max(np.abs(o - ro)) <= TOL[cfg.dtype]
    assert np.max(np.abs(lse - rl)) <= LSE_TOL[cfg.dtype]


def test_tree_chain_is_bitwise_causal(gpu_lib):
    """A chain tree takes the same path through the kernel as the causal
    mask: outputs must be identical, bit for bit."""
    cfg = synth.config(2, bs=3, ctx_lo=200, ctx_hi=700)
    print_case("block_attn_tree chain", cfg)
    x = synth.make_attn_inputs(cfg, seed=32)
    case = AttnCase(x)
    chain = synth.tree_row_masks(np.arange(-1, cfg.block - 1, dtype=np.int32))
    o_t, l_t = run_tree(case, chain)
    o_c, l_c = run(case, synth.CAUSAL)
    assert np.array_equal(o_t, o_c) and np.array_equal(l_t, l_c)


@pytest.mark.parametrize("B", [127, 128, 129, 256, 257])
def test_tree_mask_word_boundaries(gpu_lib, B):
    """Blocks at and around mask-word boundaries (W = 2, 3, 4, 5), random
    per-request trees and a chain: every row against the dense reference,
    the chain also bitwise equal to CAUSAL."""
    cfg = synth.config(6, bs=2, hq=4, hkv=2, d=64, block=B, tree_depth=B // 3, ctx_lo=5,
                       ctx_hi=90)
    print_case("block_attn_tree word boundaries", B)
    x = synth.make_attn_inputs(cfg, seed=B)
    case = AttnCase(x)
    _, masks = synth.make_trees(cfg, B)
    o, lse = run_tree(case, masks)
    ro, rl = oracle.block_attn_dense(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                     x.page_table, x.seq_lens, oracle.TREE, 0, tree=masks)
    assert np.max(np.abs(o - ro)) <= TOL[cfg.dtype]
    assert np.max(np.abs(lse - rl)) <= LSE_TOL[cfg.dtype]
    chain = synth.tree_row_words(np.arange(-1, B - 1, dtype=np.int32))
    o_t, l_t = run_tree(case, chain)
    o_c, l_c = run(case, synth.CAUSAL)
    assert np.array_equal(o_t, o_c) and np.array_equal(l_t, l_c)


def test_wide_chain_tree_is_bitwise_causal(gpu_lib):
    """A chain of 150 nodes (three mask words per row, read from LDS) gives
    the causal mask's outputs bit for bit; both take the split schedule."""
    cfg = synth.config(2, bs=2, hq=8, hkv=2, block=150, ctx_lo=100, ctx_hi=600)
    print_case("block_attn_tree wide chain", cfg)
    x = synth.make_attn_inputs(cfg, seed=34)
    case = AttnCase(x)
    chain = synth.tree_row_words(np.arange(-1, cfg.block - 1, dtype=np.int32))
    o_t, l_t = run_tree(case, chain)
    o_c, l_c = run(case, synth.CAUSAL)
    assert np.array_equal(o_t, o_c) and np.array_equal(l_t, l_c)


F32_P32 = [
    # (name, config id, overrides, mode): fp32 inputs in 32-token pages (both
    # halves of a DMA stage from one page, the V tail of a 32-token page), D 64
    # and 128, every mask mode; ragged lengths end inside a page
    ("f32_p32_d64_causal", 2, dict(bs=3, hq=4, hkv=2, d=64, page=32, dtype="f32", ctx_lo=1,
                                   ctx_hi=1700), synth.CAUSAL),
    ("f32_p32_d128_bidir", 3, dict(bs=2, hq=8, hkv=2, page=32, dtype="f32", ctx_lo=200,
                                   ctx_hi=1300), synth.BIDIR),
    ("f32_p32_d128_mixed", 5, dict(bs=3, hq=8, hkv=2, page=32, dtype="f32", n_causal=5,
                                   ctx_lo=30, ctx_hi=900), synth.MIXED),
    ("f32_p32_d64_mixed", 5, dict(bs=2, hq=4, hkv=1, d=64, page=32, dtype="f32", n_causal=11,
                                  ctx_lo=500, ctx_hi=1500), synth.MIXED),
    ("f32_p32_d128_tree", 6, dict(bs=3, hq=8, hkv=2, page=32, dtype="f32", block=24,
                                  tree_depth=9, ctx_lo=50, ctx_hi=1100), synth.TREE),
    ("f32_p32_d64_tree", 6, dict(bs=2, hq=4, hkv=2, d=64, page=32, dtype="f32", block=40,
                                 tree_depth=12, ctx_lo=0, ctx_hi=800), synth.TREE),
]


@pytest.mark.parametrize("name,cid,over,mode", F32_P32, ids=[c[0] for c in F32_P32])
def test_f32_page32_every_schedule(gpu_lib, name, cid, over, mode):
    """fp32 with 32-token pages under the default plan, a loose bound that
    splits every unit many ways, and a bound loose enough for the balanced
    schedule: every output row against the dense reference at 1e-5."""
    cfg = synth.config(cid, **over)
    print_case("block_attn f32 page 32", name, cfg)
    x = synth.make_attn_inputs(cfg, seed=61)
    case = AttnCase(x)
    masks = synth.make_trees(cfg, 61)[1] if mode == synth.TREE else None
    units = cfg.bs * cfg.hkv
    balanced = 32 * (-(-32768 // units))      # units x stages >= 32768
    ref = oracle.block_attn_dense(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                  x.page_table, x.seq_lens, mode, cfg.n_causal, tree=masks)
    for max_kv in (case.max_kv, 4 * case.max_kv + 3000, balanced):
        if mode == synth.TREE:
            o, lse = run_tree(case, masks, max_kv=max_kv)
        else:
            o, lse = run(case, mode, max_kv=max_kv)
        assert np.max(np.abs(o - ref[0])) <= TOL["f32"], max_kv
        assert np.max(np.abs(lse - ref[1])) <= LSE_TOL["f32"], max_kv
    assert va.attn_workspace_bytes(cfg.bs, cfg.block, cfg.hq, cfg.hkv, cfg.d, balanced) > 0


def sampled_rows(x, n, rng):
    rows = set()
    B, hq = x.cfg.block, x.cfg.hq
    while len(rows) < n:
        rows.add((int(rng.integers(x.cfg.bs)), int(rng.integers(B)), int(rng.integers(hq))))
    # always the first and last block rows of the longest and shortest request
    for b in (int(np.argmax(x.seq_lens)), int(np.argmin(x.seq_lens))):
        rows.update({(b, 0, 0), (b, B - 1, hq - 1)})
    return sorted(rows)


QUADS = [
    # (name, overrides of the quadratic workload): k drafts, (k + 1)^2 rows
    ("k4_g4_bf16", dict(bs=3, ctx_lo=60, ctx_hi=700)),
    ("k7_g2_d64_f32", dict(bs=2, hq=4, hkv=2, d=64, block=64, quad_k=7, dtype="f32", ctx_lo=0,
                           ctx_hi=500)),
    ("k3_g8_p32", dict(bs=4, hq=16, hkv=2, page=32, block=16, quad_k=3, ctx_lo=1, ctx_hi=300)),
    ("k7_g4_bf16_rowgroups", dict(bs=2, block=64, quad_k=7, ctx_lo=10, ctx_hi=600)),
    # past 64 rows: mask words (a block of 16 drafted positions has k = 15)
    ("k15_g4_bf16_words", dict(bs=2, block=256, quad_k=15, ctx_lo=10, ctx_hi=400)),
    ("k21_g2_d64_f32_words", dict(bs=1, hq=4, hkv=2, d=64, block=484, quad_k=21, dtype="f32",
                                  ctx_lo=0, ctx_hi=200)),
]


@pytest.mark.parametrize("name,over", QUADS, ids=[q[0] for q in QUADS])
def test_quadratic_layout_all_rows(gpu_lib, name, over):
    """The quadratic layout (draft groups after every spine token) through the
    bitmask mode, every output row against the dense reference."""
    cfg = synth.config(8, **over)
    print_case("block_attn_tree quadratic", name, cfg)
    x = synth.make_attn_inputs(cfg, seed=33)
    _, masks = synth.quadratic_layout(cfg.quad_k)
    o, lse = run_tree(AttnCase(x), masks)
    ro, rl = oracle.block_attn_dense(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                     x.page_table, x.seq_lens, oracle.TREE, 0, tree=masks)
    assert np.max(np.abs(o - ro)) <= TOL[cfg.dtype]
    assert np.max(np.abs(lse - rl)) <= LSE_TOL[cfg.dtype]


@pytest.mark.parametrize("cid", [2, 3, 4, 5, 6, 8, 9, 10, 11])
def test_full_size_sampled_rows(gpu_lib, cid):
    """Full workload shapes in the bench's launch configuration; the reference
    computes sampled rows one at a time."""
    cfg = synth.config(cid)
    print_case("block_attn full size", cid, cfg.name)
    x = synth.make_attn_inputs(cfg, seed=cid)
    case = AttnCase(x)
    mode = cfg.modes[0]
    masks = None
    if mode == synth.TREE:
        if cfg.quad_k:
            _, masks = synth.quadratic_layout(cfg.quad_k)
        else:
            _, masks = synth.make_trees(cfg, cid)
        o, lse = run_tree(case, masks)
    else:
        o, lse = run(case, mode)
    assert np.isfinite(o).all()
    rows = sampled_rows(x, 40, np.random.default_rng(cid))
    ro, rl = oracle.block_attn_rows(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                    x.page_table, x.seq_lens, mode, cfg.n_causal, rows=rows,
                                    tree=masks)
    for (b, i, h) in rows:
        assert np.max(np.abs(o[b, i, h] - ro[b, i, h])) <= TOL[cfg.dtype], (b, i, h)
        assert abs(lse[b, i, h] - rl[b, i, h]) <= LSE_TOL[cfg.dtype], (b, i, h)


def compact_for_requests(x, reqs):
    """The inputs of requests `reqs` alone, over a pool holding only their
    pages (the page table renumbered), so that a float64 copy stays small."""
    need = [-(-(int(x.seq_lens[b]) + x.cfg.block) // x.cfg.page) for b in reqs]
    pages = np.unique(np.concatenate([x.page_table[b, :n] for b, n in zip(reqs, need)]))
    remap = np.full(x.num_pages, -1, dtype=np.int64)
    remap[pages] = np.arange(len(pages))
    table = np.zeros((len(reqs), x.max_pages), dtype=np.int32)
    for r, (b, n) in enumerate(zip(reqs, need)):
        table[r, :n] = remap[x.page_table[b, :n]]
    return synth.AttnInputs(x.cfg, x.seq_lens[reqs], table, len(pages), x.q[reqs],
                            x.k_pool[pages], x.v_pool[pages], x.n_causal[reqs])


SPANS = [
    # (name, config id, overrides, mode): requests of 17-18k keys (more than
    # one 512-stage window of staged page offsets) and batches whose balanced
    # shares (units x stages / 256) exceed 512 stages, so that pieces cross
    # windows; one and two row tiles per wave
    ("g2_b16_d64_causal", 2, dict(bs=64, hq=8, hkv=4, d=64, ctx_lo=17000, ctx_hi=18000),
     synth.CAUSAL),
    ("g4_b32_d64_bidir", 3, dict(bs=32, hq=32, hkv=8, d=64, ctx_lo=17000, ctx_hi=18000),
     synth.BIDIR),
]


@pytest.mark.parametrize("name,cid,over,mode", SPANS, ids=[s[0] for s in SPANS])
def test_balanced_pieces_span_page_windows(gpu_lib, name, cid, over, mode):
    """A balanced piece's first window of page offsets is staged during the
    previous piece's merge, its later windows in place; sampled rows (every
    request's first and last block row included) against the reference."""
    cfg = synth.config(cid, **over)
    print_case("block_attn balanced, multi-window pieces", name, cfg)
    x = synth.make_attn_inputs(cfg, seed=41 + cid)
    case = AttnCase(x)
    units = cfg.bs * cfg.hkv
    assert units * ((case.max_kv + 31) // 32) >= 32768
    assert units * ((int(x.seq_lens.min()) + cfg.block) // 32) // 256 > 512
    o, lse = run(case, mode)
    assert np.isfinite(o).all()
    rng = np.random.default_rng(41 + cid)
    reqs = sorted({int(b) for b in rng.choice(cfg.bs, size=4, replace=False)} |
                  {int(np.argmax(x.seq_lens))})
    sub = compact_for_requests(x, reqs)
    rows = [(r, i, h) for r in range(len(reqs)) for i in (0, cfg.block - 1)
            for h in (0, cfg.hq - 1)]
    rows += [(r, int(rng.integers(cfg.block)), int(rng.integers(cfg.hq))) for r in range(len(reqs))]
    ro, rl = oracle.block_attn_rows(sub.as_f64("q"), sub.as_f64("k_pool"), sub.as_f64("v_pool"),
                                    sub.page_table, sub.seq_lens, mode, cfg.n_causal, rows=rows)
    for (r, i, h) in rows:
        b = reqs[r]
        assert np.max(np.abs(o[b, i, h] - ro[r, i, h])) <= TOL[cfg.dtype], (b, i, h)
        assert abs(lse[b, i, h] - rl[r, i, h]) <= LSE_TOL[cfg.dtype], (b, i, h)


ROW_GROUPS = [
    # (name, config id, overrides, mode, per-request clean counts): 256 query
    # rows per KV head (two row groups of 128) in the other element types and
    # head sizes
    ("f32_d64_g2_b128_causal", 1, dict(bs=3, hq=4, hkv=2, block=128, ctx_lo=200, ctx_hi=700),
     synth.CAUSAL, False),
    ("bf16_d64_g4_b64_mixed_nc", 3, dict(bs=3, hq=8, hkv=2, d=64, block=64, n_causal=20,
                                         ctx_lo=100, ctx_hi=900), synth.MIXED, True),
    ("f32_d128_g8_b32_bidir", 1, dict(bs=2, hq=8, hkv=1, d=128, block=32, ctx_lo=100,
                                      ctx_hi=400), synth.BIDIR, False),
]


@pytest.mark.parametrize("name,cid,over,mode,nc_req", ROW_GROUPS, ids=[r[0] for r in ROW_GROUPS])
def test_row_groups_types_and_sizes(gpu_lib, name, cid, over, mode, nc_req):
    """Row groups under the split plan, a bound loose enough to split every
    unit many ways, and the balanced schedule, every row against the
    reference."""
    cfg = synth.config(cid, **over)
    print_case("block_attn row groups", name, cfg)
    assert (cfg.hq // cfg.hkv) * cfg.block > 128
    x = synth.make_attn_inputs(cfg, seed=51 + cid, n_causal_per_req=nc_req)
    case = AttnCase(x)
    outs = []
    for max_kv in (None, 20000, 65536 * 4):
        o, lse = run(case, mode, max_kv=max_kv, nc_per_req=nc_req)
        if nc_req:
            for b in range(cfg.bs):
                one = synth.AttnInputs(cfg, x.seq_lens[b:b + 1], x.page_table[b:b + 1],
                                       x.num_pages, x.q[b:b + 1], x.k_pool, x.v_pool,
                                       x.n_causal[b:b + 1])
                ro, rl = ref_dense(one, mode, int(x.n_causal[b]))
                assert np.max(np.abs(o[b:b + 1] - ro)) <= TOL[cfg.dtype]
                assert np.max(np.abs(lse[b:b + 1] - rl)) <= LSE_TOL[cfg.dtype]
        else:
            check_all(x, o, lse, mode, cfg.n_causal)
        outs.append(o)
    assert np.max(np.abs(outs[0] - outs[2])) <= (1e-5 if cfg.dtype == "f32" else 2 ** -7)


def test_single_token_block_modes_agree(gpu_lib):
    """B = 1 is single-token decode in every mask mode: the outputs agree bit
    for bit; with an empty context the output is the block's own V row."""
    cfg = synth.config(2, bs=4, block=1, ctx_lo=1, ctx_hi=300)
    print_case("block_attn single-token block, every mode", cfg)
    x = synth.make_attn_inputs(cfg, seed=61)
    x.seq_lens[0] = 0
    case = AttnCase(x)
    outs = [run(case, m) for m in (synth.BIDIR, synth.CAUSAL, synth.MIXED)]
    for o, lse in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(lse, outs[0][1])
    check_all(x, outs[0][0], outs[0][1], synth.CAUSAL, 0)
    v = x.as_f64("v_pool")[x.page_table[0, 0], :, :, 0]     # [Hkv, D]: key 0 of request 0
    g = cfg.hq // cfg.hkv
    for h in range(cfg.hq):
        assert np.array_equal(outs[0][0][0, 0, h], v[h // g]), h


@pytest.mark.parametrize("cid,over", [(5, dict(bs=3, ctx_lo=50, ctx_hi=600)),
                                      (3, dict(bs=2, hq=8, hkv=2, block=64, ctx_lo=10,
                                               ctx_hi=500))],
                         ids=["one_tile", "two_tiles_row_groups"])
def test_mixed_limits_are_bidir_and_causal(gpu_lib, cid, over):
    """MIXED with no clean row is BIDIR and with every row clean is CAUSAL,
    bit for bit."""
    cfg = synth.config(cid, **over)
    print_case("block_attn MIXED limits", cid, cfg)
    x = synth.make_attn_inputs(cfg, seed=71)
    case = AttnCase(x)

    def attn(mode, nc):
        lse = torch.empty((cfg.bs, cfg.block, cfg.hq), dtype=torch.float32, device="cuda")
        o = va.block_attn(mode, case.q, case.k, case.v, case.table, case.seq, case.max_kv,
                          n_causal=nc, lse=lse)
        torch.cuda.synchronize()
        return to_f64(o), lse.cpu().numpy()

    for nc, mode in ((0, synth.BIDIR), (cfg.block, synth.CAUSAL)):
        om, lm = attn(synth.MIXED, nc)
        oo, lo = attn(mode, 0)
        assert np.array_equal(om, oo) and np.array_equal(lm, lo), (nc, mode)


def test_page_permutation_changes_nothing(gpu_lib):
    """Moving the physical pages, with their page-table entries, changes no
    bit of the output (default plan and balanced schedule)."""
    cfg = synth.config(4, bs=6, ctx_lo=100, ctx_hi=1500)
    print_case("block_attn page permutation", cfg)
    x = synth.make_attn_inputs(cfg, seed=81)
    perm = np.random.default_rng(81).permutation(x.num_pages)
    k2 = np.empty_like(x.k_pool)
    v2 = np.empty_like(x.v_pool)
    k2[perm] = x.k_pool
    v2[perm] = x.v_pool
    t2 = np.where(x.page_table >= 0, perm[np.maximum(x.page_table, 0)], x.page_table)
    y = synth.AttnInputs(cfg, x.seq_lens, t2.astype(np.int32), x.num_pages, x.q, k2, v2,
                         x.n_causal)
    for max_kv in (None, 65536):
        o1, l1 = run(AttnCase(x), synth.CAUSAL, max_kv=max_kv)
        o2, l2 = run(AttnCase(y), synth.CAUSAL, max_kv=max_kv)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), max_kv


def test_last_block_row_is_the_same_in_causal_and_bidir(gpu_lib):
    """The block's last row sees the whole block under both masks: its output
    and LSE agree bit for bit."""
    cfg = synth.config(3, bs=3, ctx_lo=20, ctx_hi=700)
    print_case("block_attn last row, CAUSAL vs BIDIR", cfg)
    x = synth.make_attn_inputs(cfg, seed=93)
    case = AttnCase(x)
    oc, lc = run(case, synth.CAUSAL)
    ob, lb = run(case, synth.BIDIR)
    assert np.array_equal(oc[:, -1], ob[:, -1]) and np.array_equal(lc[:, -1], lb[:, -1])
    assert not np.array_equal(oc[:, 0], ob[:, 0])

