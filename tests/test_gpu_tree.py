"""GPU parity of the tree verify path: spec_accept_tree against the float64
tree walk of the CPU reference: bit-exact outputs for every request except
ties, counted, reported and at most 1 % of a test's requests. A tie is a
child test within 1e-6 of its threshold (the tried mass T is a sum whose
order differs between the two sides) or a draw within the derived float64
band of an interval end."""
import numpy as np
import pytest
import torch

import oracle
import verify_attention_amd as va
from verify_attention_amd import synth
from _support import check_tie_share, print_case, to_dev

pytestmark = pytest.mark.gpu


def run_tree_accept(ti, seq, err=None, ws=None, out=None):
    dev = lambda a: to_dev(np.ascontiguousarray(a))
    res = va.accept_tree(dev(ti.parent), dev(ti.token), dev(ti.p), dev(ti.u), dev(seq), err=err,
                         ws=ws, out=out)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def compare(ti, seq, got):
    bs = ti.parent.shape[0]
    ties = differ = 0
    for b in range(bs):
        r = oracle.tree_accept_request(ti.parent[b], ti.token[b], ti.p[b], ti.u[b], seq[b])
        same = (got["accept_len"][b] == r["accept_len"] and got["bonus"][b] == r["bonus"] and
                got["commit_len"][b] == r["commit_len"] and
                got["new_seq_lens"][b] == r["new_seq_len"] and
                np.array_equal(got["out_tokens"][b], r["out_tokens"]) and
                np.array_equal(got["path_nodes"][b], r["path_nodes"]))
        if r["tie"]:
            ties += 1
            differ += not same
            continue
        assert same, (b, {k: got[k][b] for k in got}, r)
    print(f"ties {ties} of {bs} requests ({differ} of them differ)", flush=True)
    check_tie_share(ties, bs, "spec_accept_tree")
    return ties


def test_tree_accept_full_vocab(gpu_lib):
    cfg = synth.config(6, bs=16)
    print_case("spec_accept_tree full vocab", cfg.name, "bs", cfg.bs)
    par, _ = synth.make_trees(cfg, 41)
    ti = synth.make_tree_accept_inputs(cfg, 41, par)
    seq = np.full(cfg.bs, 1000, np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = run_tree_accept(ti, seq, err=err)
    assert int(err.item()) == 0
    compare(ti, seq, got)
    assert got["accept_len"].max() >= 1   # the workload does accept children


@pytest.mark.parametrize("N,V,depth,seed", [(16, 64, 6, 1), (64, 37, 12, 2), (1, 50, 1, 3),
                                            (33, 4099, 10, 4)])
def test_tree_accept_small_vocab_many_requests(gpu_lib, N, V, depth, seed):
    """Small vocabularies make deep acceptance common; N = 64 fills the wave,
    N = 1 is a root alone (bonus only), V = 4099 leaves a ragged last
    sub-block."""
    cfg = synth.config(6, bs=256, block=N, tree_depth=depth, vocab=V, logit_sigma=2.0)
    print_case("spec_accept_tree small vocab", N, V, depth)
    par, _ = synth.make_trees(cfg, seed)
    ti = synth.make_tree_accept_inputs(cfg, seed, par)
    seq = np.random.default_rng(seed).integers(0, 5000, size=cfg.bs).astype(np.int32)
    got = run_tree_accept(ti, seq)
    compare(ti, seq, got)
    if N > 1:
        assert got["accept_len"].max() >= 2


@pytest.mark.parametrize("N", [8, 150])
def test_tree_accept_workspace_reuse_and_error_paths(gpu_lib, N):
    """Invalid token ids, a parent that is not an earlier node and rows
    without mass, flagged and resolved as the reference does, in the
    one-chunk walk (8 nodes) and the chunked one (150 nodes)."""
    cfg = synth.config(6, bs=6, block=N, tree_depth=4 if N == 8 else 30, vocab=300,
                       logit_sigma=2.0)
    print_case("spec_accept_tree error paths", cfg)
    par, _ = synth.make_trees(cfg, 5)
    ti = synth.make_tree_accept_inputs(cfg, 5, par)
    ti.token[1, np.flatnonzero(ti.parent[1] == 0)[0]] = cfg.vocab + 3    # invalid token id
    ti.parent[2, 5] = 7 if N == 8 else 140                               # parent not earlier
    ti.p[3] = 0.0                                                        # rows without mass
    seq = np.arange(cfg.bs, dtype=np.int32) * 10
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = va.workspace(va.accept_tree_workspace_bytes(cfg.bs, cfg.block, cfg.vocab))
    first = run_tree_accept(ti, seq, err=err, ws=ws)
    e = int(err.item())
    assert e & va.ERR_TREE and e & va.ERR_ZERO_RESIDUAL and e & va.ERR_TOKEN
    compare(ti, seq, first)
    second = run_tree_accept(ti, seq, ws=ws)
    for k in first:
        assert np.array_equal(first[k], second[k])
    assert first["bonus"][3] == 0 and first["accept_len"][3] == 0


def test_linear_accept_zero_rows(gpu_lib):
    """A target row with no mass at all (not a distribution): both sides give
    token 0 and the zero-residual flag."""
    cfg = synth.config(2, bs=4, vocab=2000, k_spec=3)
    print_case("spec_accept zero rows", cfg)
    acc = synth.make_accept_inputs(cfg, 9)
    acc.p[2] = 0.0
    dev = lambda a: to_dev(np.ascontiguousarray(a))
    seq = np.zeros(cfg.bs, np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = va.accept(dev(acc.p), dev(acc.q), dev(acc.draft), dev(acc.u), dev(seq), err=err)
    torch.cuda.synchronize()
    r = oracle.accept_request(acc.p[2], acc.q[2], acc.draft[2], acc.u[2], 0)
    assert int(got["bonus"][2]) == r["bonus"] == 0 and int(got["accept_len"][2]) == r["accept_len"]
    assert int(err.item()) & va.ERR_ZERO_RESIDUAL


def test_chain_tree_matches_the_linear_accept(gpu_lib):
    """A chain tree through spec_accept_tree gives what spec_accept gives for
    the same block with one-hot draft rows (test uniforms u[1..K], final draw
    u[0]), bit for bit: a chain node has one child, so both kernels test
    u * 1 < p exactly; only draws within the float64 tie band are excluded
    (the two kernels sum the residual masses in different orders)."""
    rng = np.random.default_rng(97)
    bs, K, V = 32, 15, 4096
    print_case("chain tree = linear accept", bs, K, V)
    dev = lambda a: to_dev(np.ascontiguousarray(a))
    N = K + 1
    parent = np.tile(np.arange(-1, K, dtype=np.int32), (bs, 1))
    lg = rng.standard_normal((bs, N, V)) * 10.0
    p = np.exp(lg - lg.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    token = np.zeros((bs, N), np.int32)
    best = p[:, :K].argmax(-1)
    token[:, 1:] = np.where(rng.random((bs, K)) < 0.85, best, rng.integers(V, size=(bs, K)))
    u = rng.random((bs, N), dtype=np.float32)
    token[:8, 1:] = best[:8]        # the first requests accept every draft:
    u[:8, 1:] = 1e-4                # the bonus comes from the last row
    seq = rng.integers(1, 900, size=bs).astype(np.int32)
    tr = va.accept_tree(dev(parent), dev(token), dev(p), dev(u), dev(seq))
    q = np.zeros((bs, K, V), np.float32)
    q[np.arange(bs)[:, None], np.arange(K), token[:, 1:]] = 1.0
    ul = np.ascontiguousarray(np.concatenate([u[:, 1:], u[:, :1]], axis=1))
    draft = np.ascontiguousarray(token[:, 1:])
    lin = va.accept(dev(p), dev(q), dev(draft), dev(ul), dev(seq))
    torch.cuda.synchronize()
    ref = oracle.accept_batch(p, q, draft, ul, seq)
    keep = ~ref["tie_sample"]
    for key in ("accept_len", "commit_len", "bonus", "new_seq_lens", "out_tokens"):
        a, b = tr[key].cpu().numpy(), lin[key].cpu().numpy()
        assert np.array_equal(a[keep], b[keep]), key
    check_tie_share(int((~keep).sum()), bs, "chain tree vs linear accept")
    assert (ref["accept_len"][:8] == K).all() and (ref["accept_len"][8:] < K).all()
    assert (ref["accept_len"][8:] > 0).any()



@pytest.mark.parametrize("name,over,seed", [
    ("tree_sampler_481_v2000", dict(bs=24, vocab=2000), 5),
    ("tree_sampler_481_v4099_flat", dict(bs=16, vocab=4099, logit_sigma=2.0), 6),
])
def test_tree_sampler_shape_accept(gpu_lib, name, over, seed):
    """The Tree sampler's (16, 32, 32) tree (481 nodes in chunks of 64 per
    lane, the children of a node spread over several chunks) against the
    reference walk."""
    cfg = synth.config(10, **over)
    print_case("spec_accept_tree tree sampler", name, cfg.bs, cfg.vocab)
    par, _ = synth.make_trees(cfg, seed)
    ti = synth.make_tree_accept_inputs(cfg, seed, par)
    seq = np.random.default_rng(seed).integers(0, 5000, size=cfg.bs).astype(np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = run_tree_accept(ti, seq, err=err)
    assert int(err.item()) == 0
    compare(ti, seq, got)
    assert got["accept_len"].max() >= 1


def test_tree_sampler_workload_full_size(gpu_lib):
    """The Tree sampler's workload at its full size, in the bench's launch
    configuration: 8 requests, 481-node beam trees over the full vocabulary
    (151936), target rows N(0, 6^2)."""
    cfg = synth.config(10)
    print_case("spec_accept_tree full Tree sampler workload", cfg.bs, cfg.block, cfg.vocab)
    par, _ = synth.make_trees(cfg, 0)
    ti = synth.make_tree_accept_inputs(cfg, 0, par)
    seq = np.full(cfg.bs, 1024, np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = run_tree_accept(ti, seq, err=err)
    assert int(err.item()) == 0
    compare(ti, seq, got)
    print(f"accept lengths {got['accept_len'].tolist()}", flush=True)


@pytest.mark.parametrize("N", [65, 200, 512])
def test_wide_chain_tree_matches_the_reference(gpu_lib, N):
    """Chains of up to 512 nodes (walks across every 64-node chunk) with
    test uniforms small enough that most requests accept deep, and siblings
    placed in other chunks than their first brother: node 1's children are
    nodes 2 and N - 1 (a repeat of node 2's token and a fresh one)."""
    rng = np.random.default_rng(N)
    bs, V = 12, 300
    print_case("spec_accept_tree wide chain", N)
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (bs, 1))
    parent[:, N - 1] = 1
    lg = rng.standard_normal((bs, N, V)) * 4.0
    p = np.exp(lg - lg.max(-1, keepdims=True))
    p = (p / p.sum(-1, keepdims=True)).astype(np.float32)
    token = p.argmax(-1).astype(np.int32)
    token = np.concatenate([np.zeros((bs, 1), np.int32), token[:, :-1]], axis=1)  # child of n: argmax p_n
    token[:, N - 1] = token[:, 2]
    token[6:, N - 1] = np.argsort(-p[6:, 1], axis=-1, kind="stable")[:, 1]   # p_1's second best
    u = (rng.random((bs, N), dtype=np.float32) * np.float32(1e-3)).astype(np.float32)
    u[:, 0] = rng.random(bs, dtype=np.float32)
    u[3:6, 5 + (N // 3)] = np.float32(0.9999)     # an early stop at different depths
    u[0:2, 2] = u[6:9, 2] = np.float32(0.9999)    # node 2 rejected: its sibling N - 1 is tried
    u[6:9, N - 1] = 0.0
    tokdirty = token.copy()
    tokdirty[9, 7] = V + 5                          # an invalid token: a reject, flagged
    u[9, 1:7] = 0.0                                 # (reached: nodes 1..6 are accepted)
    ti = synth.TreeAcceptInputs(parent, tokdirty, p, u)
    seq = rng.integers(0, 900, size=bs).astype(np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = run_tree_accept(ti, seq, err=err)
    compare(ti, seq, got)
    assert int(err.item()) & va.ERR_TOKEN
    assert got["accept_len"].max() == N - 2        # the whole chain below node 1
    assert (got["accept_len"][0:2] == 1).all()          # the sibling repeats node 2's token
    assert (got["path_nodes"][6:9, 1] == N - 1).all()   # the fresh sibling is accepted
