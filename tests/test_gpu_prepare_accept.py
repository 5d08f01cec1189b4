"""GPU parity of spec_prepare_block, spec_draft_argmax and spec_accept
against the float64 CPU reference. Integer outputs must match bit for bit.
The accept tests u * q < p are exact in double on both sides (the same float32
inputs), so requests with an accept tie (|u - min(1, p/q)| < 1e-6) are counted
and still compared; only a draw whose threshold lies within the derived
float64 band of an interval end (oracle.accept.sample_tie_band) is left out,
and at most 1 % of a test's requests may be."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import verify_attention_amd as va
from verify_attention_amd import synth
from _support import check_tie_share, print_case, to_dev

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ prepare_block
def test_prepare_golden(gpu_lib):
    fx = json.load(open(os.path.join(GOLDEN, "prepare_block_small.json")))
    print_case("prepare golden")
    t = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda")
    ids, pos, loc = va.prepare_block(t(fx["verified_id"]), t(fx["seq_lens"]), t(fx["page_table"]),
                                     fx["page_size"], fx["block"], fx["mask_token_id"], 16)
    e = fx["expect_draft_pass"]
    assert ids.cpu().tolist() == e["block_ids"]
    assert pos.cpu().tolist() == e["positions"]
    assert loc.cpu().tolist() == e["cache_loc"]
    ids, _, _ = va.prepare_block(t(fx["verified_id"]), t(fx["seq_lens"]), t(fx["page_table"]),
                                 fx["page_size"], fx["block"], fx["mask_token_id"], 16,
                                 t(fx["draft_tokens"]))
    assert ids.cpu().tolist() == fx["expect_verify_pass"]["block_ids"]


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("verify", [False, True])
def test_prepare_matches_reference(gpu_lib, cid, verify):
    cfg = synth.config(cid)
    print_case("prepare", cid, verify)
    seq = synth.context_lengths(cfg, cid)
    table, num_pages = synth.page_layout(cfg, seq, cid)
    verified, drafts = synth.make_round_state(cfg, cid)
    d = drafts if verify else None
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = va.prepare_block(to_dev(verified), to_dev(seq), to_dev(table), cfg.page, cfg.block,
                           123456, num_pages, None if d is None else to_dev(d), err=err)
    ref = oracle.prepare_block(verified, seq, table, cfg.page, cfg.block, 123456, d, num_pages)
    for g, r in zip(got, ref[:3]):
        assert np.array_equal(g.cpu().numpy(), r)
    assert int(err.item()) == ref[3] == 0


def test_prepare_error_flags(gpu_lib):
    print_case("prepare errors")
    seq = np.array([2, 5, -1, 0], np.int32)
    table = np.array([[3, -1], [3, 1], [0, 1], [9, 1]], np.int32)
    verified = np.arange(4, dtype=np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = va.prepare_block(to_dev(verified), to_dev(seq), to_dev(table), 4, 4, 0, 5, err=err)
    ref = oracle.prepare_block(verified, seq, table, 4, 4, 0, None, 5)
    for g, r in zip(got, ref[:3]):
        assert np.array_equal(g.cpu().numpy(), r)
    assert int(err.item()) == ref[3] == (va.ERR_SLOT | va.ERR_CAPACITY)


# ------------------------------------------------------------------ argmax
def test_argmax_with_planted_ties(gpu_lib):
    print_case("argmax ties")
    rng = np.random.default_rng(0)
    rows, V = 37, 5003  # odd V: unaligned rows take the scalar path
    x = rng.integers(-50, 50, size=(rows, V)).astype(np.float32)
    x[5, [7, 4000]] = 1000.0
    x[6, :] = 3.0
    x[7, [V - 1, V - 2]] = 999.0
    ref = np.array([oracle.argmax_lowest(r) for r in x])
    for dt in ("f32", "bf16"):
        t = to_dev(synth.bf16_bits(x)) if dt == "bf16" else to_dev(x)
        got = va.draft_argmax(t).cpu().numpy()
        assert np.array_equal(got, ref), dt


def test_argmax_aligned_rows_nan_inf_and_vector_ties(gpu_lib):
    # aligned rows take the vector path: ties inside one 16-byte vector and
    # across threads, rows of -inf and NaN (NaN never wins)
    print_case("argmax aligned edge rows")
    rng = np.random.default_rng(1)
    rows, V = 12, 8192
    x = rng.normal(0, 3, size=(rows, V)).astype(np.float32)
    x[0, [9, 11]] = 50.0                 # same float4 / bf16x8 vector
    x[1, [8, 8 + 4096]] = 50.0           # different threads
    x[2, :] = -np.inf
    x[3, :] = -np.inf
    x[3, 0] = np.nan                     # NaN, then -inf everywhere
    x[4, ::3] = np.nan
    x[5, :] = np.nan
    x[5, 7000] = -1.0
    x[6, :] = 2.0                        # all equal
    x[7, V - 1] = 99.0                   # the very last entry
    ref = np.array([oracle.argmax_lowest(r) for r in x])
    for dt in ("f32", "bf16"):
        t = to_dev(synth.bf16_bits(x)) if dt == "bf16" else to_dev(x)
        xv = synth.bf16_to_f32(synth.bf16_bits(x)) if dt == "bf16" else x
        want = np.array([oracle.argmax_lowest(r) for r in xv])
        got = va.draft_argmax(t).cpu().numpy()
        assert np.array_equal(got, want), (dt, got, want)
    assert ref[0] == 9 and ref[1] == 8 and ref[2] == 0 and ref[3] == 1 and ref[5] == 7000


def test_argmax_draft_pass_full_size(gpu_lib):
    cfg = synth.config(3)
    print_case("argmax full", cfg.name)
    logits = synth.make_argmax_logits(cfg, 3)
    got = va.draft_argmax(to_dev(logits)).cpu().numpy()
    f = synth.bf16_to_f32(logits)
    ref = np.array([oracle.argmax_lowest(r) for r in f])
    assert np.array_equal(got, ref)
    # bf16 logits of this size do tie: the lowest index must have won
    assert any((r == r.max()).sum() > 1 for r in f[:200])


# ------------------------------------------------------------------ accept
def run_accept(x, seq, greedy=False, err=None, ws=None):
    out = va.accept(to_dev(x.p), to_dev(x.q), to_dev(x.draft), to_dev(x.u), to_dev(seq),
                    greedy=greedy, err=err, ws=ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def compare_accept(got, ref, allow_ties=True):
    """Every request must match bit for bit except draws within the float64
    tie band of the sampling threshold (at most 1 % of the requests); accept
    ties are counted and reported, and compared like every other request."""
    tie = ref["tie_sample"] if allow_ties else np.zeros(len(ref["tie"]), bool)
    same = np.ones(len(tie), bool)
    for k_got, k_ref in (("accept_len", "accept_len"), ("commit_len", "commit_len"),
                         ("bonus", "bonus"), ("new_seq_lens", "new_seq_len"),
                         ("out_tokens", "out_tokens")):
        g, r = got[k_got], ref[k_ref]
        same &= (g == r).reshape(len(g), -1).all(-1)
    bad = np.flatnonzero(~same & ~tie)
    assert len(bad) == 0, f"requests differing without a tie: {bad}"
    n_tie = int(tie.sum())
    print(f"accept ties (compared): {int(ref['tie_accept'].sum())}; sampling ties excluded: "
          f"{n_tie}, of which matched anyway: {int((same & tie).sum())}")
    check_tie_share(n_tie, len(tie), "spec_accept")
    return n_tie, int((~same).sum())


@pytest.mark.parametrize("cid,bs", [(1, 64), (2, None), (5, None), (4, None)])
def test_accept_matches_reference(gpu_lib, cid, bs):
    cfg = synth.config(cid)
    print_case("accept", cid, bs)
    x = synth.make_accept_inputs(cfg, seed=cid, bs=bs)
    n = x.draft.shape[0]
    seq = synth.context_lengths(synth.config(cid, bs=n), cid)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = run_accept(x, seq, err=err)
    ref = oracle.accept_batch(x.p, x.q, x.draft, x.u, seq)
    ties, differ = compare_accept(got, ref)
    print(f"accept config {cid}: {n} requests, {ties} ties excluded, {differ} differ, "
          f"mean accept {ref['accept_len'].mean():.2f}")
    assert int(err.item()) == 0
    assert differ <= ties


def test_accept_at_the_largest_k(gpu_lib):
    """K = 63, the largest the call takes: half of the requests have q = p, so
    every test passes and the bonus comes from the 64th row of p; the others
    reject early."""
    cfg = synth.config(1, k_spec=63)
    print_case("accept K = 63")
    x = synth.make_accept_inputs(cfg, seed=63, bs=64)
    x.q[:32] = x.p[:32, :63]
    seq = synth.context_lengths(synth.config(1, bs=64), 63)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = run_accept(x, seq, err=err)
    ref = oracle.accept_batch(x.p, x.q, x.draft, x.u, seq)
    assert (ref["accept_len"][:32] == 63).all()
    ties, differ = compare_accept(got, ref)
    assert int(err.item()) == 0
    assert differ <= ties


def test_accept_all_accepted_and_workspace_reuse(gpu_lib):
    cfg = synth.config(2, bs=8)
    print_case("accept all accepted")
    x = synth.make_accept_inputs(cfg, seed=11, bs=8)
    x.q[:] = x.p[:, :-1]           # q == p: every draft passes, the bonus comes from row K
    seq = np.full(8, 1000, np.int32)
    ws = va.workspace(va.accept_workspace_bytes(8, cfg.k_spec, cfg.vocab))
    for _ in range(3):
        got = run_accept(x, seq, ws=ws)
        ref = oracle.accept_batch(x.p, x.q, x.draft, x.u, seq)
        compare_accept(got, ref)
        assert (got["accept_len"] == cfg.k_spec).all()


def test_accept_invalid_token_and_zero_residual(gpu_lib):
    cfg = synth.config(1, bs=4)
    print_case("accept error paths")
    x = synth.make_accept_inputs(cfg, seed=12, bs=4)
    x.draft[0, 0] = cfg.vocab + 3          # invalid token at the first position
    x.u[1, :] = 0.0                        # request 1: accept while p > 0 ...
    x.draft[1, 2] = -1                     # ... until the invalid token at position 2
    x.q[2, 0] = 2 * x.p[2, 0]              # request 2: q = 2p on row 0 -> residual is zero
    x.u[2, 0] = 0.9
    x.draft[2, 0] = int(np.argmax(x.q[2, 0]))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    seq = np.zeros(4, np.int32)
    got = run_accept(x, seq, err=err)
    ref = oracle.accept_batch(x.p, x.q, x.draft, x.u, seq)
    compare_accept(got, ref)
    assert got["accept_len"][0] == 0 and got["accept_len"][1] == 2 and got["accept_len"][2] == 0
    assert int(err.item()) == (va.ERR_TOKEN | va.ERR_ZERO_RESIDUAL)
    assert ref["err"][0] & oracle.accept.ERR_TOKEN and ref["err"][2] & oracle.accept.ERR_ZERO_RESIDUAL


def test_greedy_accept(gpu_lib):
    fx = json.load(open(os.path.join(GOLDEN, "greedy_accept_dflash.json")))
    print_case("accept greedy")
    V = fx["vocab"]
    cases = fx["cases"]
    K = len(cases[0]["drafts"])
    p = np.zeros((len(cases), K + 1, V), np.float32)
    for b, c in enumerate(cases):
        p[b, np.arange(K + 1), c["target_predict"]] = 1.0
    draft = np.array([c["drafts"] for c in cases], np.int32)
    seq = np.array([c["seq_len"] for c in cases], np.int32)
    out = va.accept(to_dev(p), None, to_dev(draft), None, to_dev(seq), greedy=True)
    for b, c in enumerate(cases):
        assert int(out["accept_len"][b]) == c["accept_len"]
        assert int(out["bonus"][b]) == c["bonus"]
        assert int(out["new_seq_lens"][b]) == c["new_seq_len"]
        assert out["out_tokens"][b].cpu().tolist() == c["out_tokens"]
    # a larger random greedy case against the reference (ties inside p rows)
    cfg = synth.config(1, bs=32)
    x = synth.make_accept_inputs(cfg, seed=13, bs=32)
    tgt = x.p.argmax(-1)
    x.draft[:] = np.where(np.random.default_rng(1).random(x.draft.shape) < 0.8, tgt[:, :-1], 3)
    s2 = np.arange(32, dtype=np.int32)
    got = run_accept(x, s2, greedy=True)
    ref = oracle.accept_batch(x.p, x.q, x.draft, x.u, s2, greedy=True)
    compare_accept(got, ref, allow_ties=False)


def test_one_hot_rejection_sampling_is_the_greedy_rule(gpu_lib):
    """With one-hot p and q (q at the drafted token) the rejection-sampling
    accept reproduces the greedy rule exactly, whatever the uniforms: a test
    passes iff the draft is p's token, and the residual (or the bonus row) is
    one-hot at p's token."""
    rng = np.random.default_rng(91)
    bs, K, V = 64, 15, 1000
    print_case("accept one-hot = greedy", bs, K, V)
    tgt = rng.integers(V, size=(bs, K + 1))
    draft = np.where(rng.random((bs, K)) < 0.7, tgt[:, :K],
                     rng.integers(V, size=(bs, K))).astype(np.int32)
    p = np.zeros((bs, K + 1, V), np.float32)
    p[np.arange(bs)[:, None], np.arange(K + 1), tgt] = 1.0
    q = np.zeros((bs, K, V), np.float32)
    q[np.arange(bs)[:, None], np.arange(K), draft] = 1.0
    u = rng.random((bs, K + 1), dtype=np.float32)
    seq = rng.integers(1, 500, size=bs).astype(np.int32)
    st = va.accept(to_dev(p), to_dev(q), to_dev(draft), to_dev(u), to_dev(seq))
    gr = va.accept(to_dev(p), None, to_dev(draft), None, to_dev(seq), greedy=True)
    torch.cuda.synchronize()
    for key in ("accept_len", "commit_len", "bonus", "out_tokens", "new_seq_lens"):
        assert torch.equal(st[key], gr[key]), key
    assert (st["accept_len"] < K).any() and (st["accept_len"] == K).any()

