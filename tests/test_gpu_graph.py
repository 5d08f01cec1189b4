"""Rounds captured in HIP graphs through the C ABI. The calls allocate
nothing, clear nothing and never synchronise with the host, so a round can be
recorded once and replayed: the linear verify round (the verify pass's block
preparation, block attention and the accept that also prepares the next
round's block), the tree round (the tree block's preparation, attention
under the tree masks, and the tree accept that commits its path into the K/V
pools), the quadratic round (attention under the layout's masks, then the
spine accept with the hand-off, the spine commit and the next block), the
draft pass round (MASK block, bidirectional attention, greedy draft argmax)
and the logits verify round (accept over logits with temperature, top-k and
top-p). Every replay is checked against the same calls run eagerly on the same
inputs, bit for bit, with eager work (new uniforms, new draft tokens, restored
pools) between the replays; the eager results are also checked against the
CPU reference."""
import numpy as np
import pytest
import torch

import oracle
import verify_attention_amd as va
from verify_attention_amd import synth
from _support import AttnCase, check_tie_share, print_case, to_dev

pytestmark = pytest.mark.gpu
MASK = 151669


def _round(case, x, cfg, dev_in, outs, stream=None):
    """The round's three calls, marshalled once (their enqueue closures)."""
    B = cfg.block
    max_kv = int(x.seq_lens.max()) + B
    e1, _ = va.prepare_block_call(dev_in["vid"], case.seq, case.table, cfg.page, B, MASK,
                                  x.num_pages, dev_in["drafts"], out=outs["prep"],
                                  err=outs["err"], stream=stream)
    e2, _ = va.block_attn_call(synth.CAUSAL, case.q, case.k, case.v, case.table, case.seq,
                               max_kv, out=outs["o"], ws=outs["ws_attn"], err=outs["err"],
                               stream=stream)
    e3, _ = va.accept_prepare_call(dev_in["p"], dev_in["q"], dev_in["draft"], dev_in["u"],
                                   case.seq, case.table, cfg.page, B, MASK, x.num_pages,
                                   out=outs["acc"], ws=outs["ws_acc"], err=outs["err"],
                                   stream=stream)
    return (e1, e2, e3)


def _outputs(cfg, case, x):
    bs, B = cfg.bs, cfg.block
    max_kv = int(x.seq_lens.max()) + B
    i32 = dict(dtype=torch.int32, device="cuda")
    acc = dict(accept_len=torch.empty(bs, **i32), commit_len=torch.empty(bs, **i32),
               bonus=torch.empty(bs, **i32), out_tokens=torch.empty((bs, cfg.k_spec + 1), **i32),
               new_seq_lens=torch.empty(bs, **i32), block_ids=torch.empty((bs, B), **i32),
               positions=torch.empty((bs, B), **i32), cache_loc=torch.empty((bs, B), **i32))
    return dict(prep=tuple(torch.empty((bs, B), **i32) for _ in range(3)),
                o=torch.empty_like(case.q),
                ws_attn=va.workspace(max(1, va.attn_workspace_bytes(bs, B, cfg.hq, cfg.hkv, cfg.d,
                                                                    max_kv))),
                ws_acc=va.workspace(va.accept_workspace_bytes(bs, cfg.k_spec, cfg.vocab)),
                acc=acc, err=torch.zeros(1, **i32))


def _snapshot(outs):
    snap = {f"prep{i}": t.clone() for i, t in enumerate(outs["prep"])}
    snap["o"] = outs["o"].clone()
    snap.update({k: v.clone() for k, v in outs["acc"].items()})
    return snap


def test_verify_round_replays_as_a_hip_graph(gpu_lib):
    cfg = synth.config(2, bs=8, vocab=6000)
    print_case("verify round as a HIP graph", cfg.bs, cfg.vocab)
    x = synth.make_attn_inputs(cfg, seed=6)
    case = AttnCase(x)
    acc = synth.make_accept_inputs(cfg, seed=6)
    verified, drafts = synth.make_round_state(cfg, 6)
    dev_in = dict(vid=to_dev(verified), drafts=to_dev(drafts), p=to_dev(acc.p), q=to_dev(acc.q),
                  draft=to_dev(acc.draft), u=to_dev(acc.u))
    g_out = _outputs(cfg, case, x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # one eager pass before the capture
        for e in _round(case, x, cfg, dev_in, g_out):
            e()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for e in _round(case, x, cfg, dev_in, g_out):
            e()
    rng = np.random.default_rng(60)
    e_out = _outputs(cfg, case, x)
    eager = _round(case, x, cfg, dev_in, e_out)
    for rep in range(3):
        # eager work between the replays: new uniforms and draft tokens
        u = rng.random(acc.u.shape, dtype=np.float32)
        dev_in["u"].copy_(torch.from_numpy(u))
        dev_in["drafts"].copy_(torch.from_numpy(
            rng.integers(0, cfg.vocab, size=drafts.shape).astype(np.int32)))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(g_out)
        for e in eager:
            e()
        torch.cuda.synchronize()
        want = _snapshot(e_out)
        for k in want:
            assert torch.equal(got[k], want[k]), (rep, k)
        assert int(g_out["err"].item()) == 0 and int(e_out["err"].item()) == 0
        # and the eager accept against the CPU reference
        ra = oracle.accept_batch(acc.p, acc.q, acc.draft, u, x.seq_lens)
        keep = ~ra["tie_sample"]
        check_tie_share(int((~keep).sum()), cfg.bs, "graph round accept")
        assert np.array_equal(want["accept_len"].cpu().numpy()[keep], ra["accept_len"][keep])
        assert np.array_equal(want["bonus"].cpu().numpy()[keep], ra["bonus"][keep])
        print(f"replay {rep}: accept lengths {want['accept_len'].tolist()}", flush=True)


def _tree_round(x, ti, case, tmask, dev_in, outs, pools, stream=None):
    """A tree round's three calls: the tree block's ids, positions and slots,
    the attention under the tree masks, the tree accept with the commit of its
    path into the pools (which it changes in place)."""
    cfg = x.cfg
    max_kv = int(x.seq_lens.max()) + cfg.block
    e1, _ = va.prepare_tree_call(dev_in["vid"], case.seq, case.table, cfg.page, dev_in["par"],
                                 MASK, x.num_pages, dev_in["tok"], out=outs["prep"],
                                 err=outs["err"], stream=stream)
    e2, _ = va.block_attn_tree_call(tmask, case.q, pools[0], pools[1], case.table, case.seq,
                                    max_kv, out=outs["o"], ws=outs["ws_attn"], err=outs["err"],
                                    stream=stream)
    e3, _ = va.accept_tree_commit_call(dev_in["par"], dev_in["tok"], dev_in["p"], dev_in["u"],
                                       case.seq, pools[0], pools[1], case.table, out=outs["acc"],
                                       ws=outs["ws_acc"], err=outs["err"], stream=stream)
    return (e1, e2, e3)


def _tree_outputs(x, case):
    cfg = x.cfg
    bs, N = cfg.bs, cfg.block
    max_kv = int(x.seq_lens.max()) + N
    i32 = dict(dtype=torch.int32, device="cuda")
    acc = dict(accept_len=torch.empty(bs, **i32), commit_len=torch.empty(bs, **i32),
               bonus=torch.empty(bs, **i32), out_tokens=torch.empty((bs, N), **i32),
               path_nodes=torch.empty((bs, N), **i32), new_seq_lens=torch.empty(bs, **i32),
               freed=torch.empty((bs, N), **i32))
    return dict(prep=tuple(torch.empty((bs, N), **i32) for _ in range(3)),
                o=torch.empty_like(case.q),
                ws_attn=va.workspace(max(1, va.attn_workspace_bytes(bs, N, cfg.hq, cfg.hkv, cfg.d,
                                                                    max_kv))),
                ws_acc=va.workspace(va.accept_tree_workspace_bytes(bs, N, cfg.vocab)),
                acc=acc, err=torch.zeros(1, **i32))


def test_tree_round_replays_as_a_hip_graph(gpu_lib):
    """The tree round, whose accept also commits the accepted path into the
    K/V pools, captured once and replayed: before every replay the pools are
    restored and the uniforms redrawn (eager work), and each replay's outputs
    and pools must equal the same calls run eagerly on their own copies."""
    cfg = synth.config(6, bs=8, vocab=4000)
    print_case("tree round as a HIP graph", cfg.bs, cfg.block, cfg.vocab)
    x = synth.make_attn_inputs(cfg, seed=8)
    case = AttnCase(x)
    par, masks = synth.make_trees(cfg, 8)
    ti = synth.make_tree_accept_inputs(cfg, 8, par)
    tmask = torch.from_numpy(np.ascontiguousarray(masks).view(np.int64)).to("cuda")
    verified = np.random.default_rng(80).integers(0, cfg.vocab, size=cfg.bs).astype(np.int32)
    dev_in = dict(vid=to_dev(verified), par=to_dev(ti.parent), tok=to_dev(ti.token),
                  p=to_dev(ti.p), u=to_dev(ti.u))
    k0, v0 = to_dev(x.k_pool), to_dev(x.v_pool)       # pristine pools
    g_pools = (k0.clone(), v0.clone())
    e_pools = (k0.clone(), v0.clone())
    g_out, e_out = _tree_outputs(x, case), _tree_outputs(x, case)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # one eager pass before the capture
        for e in _tree_round(x, ti, case, tmask, dev_in, g_out, g_pools):
            e()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for e in _tree_round(x, ti, case, tmask, dev_in, g_out, g_pools):
            e()
    eager = _tree_round(x, ti, case, tmask, dev_in, e_out, e_pools)
    rng = np.random.default_rng(81)
    for rep in range(3):
        u = rng.random(ti.u.shape, dtype=np.float32)
        dev_in["u"].copy_(torch.from_numpy(u))
        for pl in (g_pools, e_pools):
            pl[0].copy_(k0)
            pl[1].copy_(v0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for e in eager:
            e()
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(g_out["prep"][i], e_out["prep"][i]), (rep, "prep", i)
        assert torch.equal(g_out["o"], e_out["o"]), (rep, "o")
        for k in e_out["acc"]:
            assert torch.equal(g_out["acc"][k], e_out["acc"][k]), (rep, k)
        for a, b in zip(g_pools, e_pools):
            assert torch.equal(a, b), (rep, "pools")
        assert int(g_out["err"].item()) == 0 and int(e_out["err"].item()) == 0
        # the eager accept against the CPU reference
        depth = e_out["acc"]["accept_len"].cpu().numpy()
        bonus = e_out["acc"]["bonus"].cpu().numpy()
        for b in range(cfg.bs):
            ra = oracle.tree_accept_request(ti.parent[b], ti.token[b], ti.p[b], u[b],
                                            x.seq_lens[b])
            if ra.get("tie_sample") or ra.get("tie_accept"):
                continue
            assert depth[b] == ra["accept_len"] and bonus[b] == ra["bonus"], (rep, b)
        print(f"replay {rep}: tree depths {depth.tolist()}", flush=True)


def test_quadratic_round_replays_as_a_hip_graph(gpu_lib):
    """The quadratic round -- attention under the layout's masks, then the
    spine accept that also hands over the next drafts, commits the spine's
    K/V and prepares the next block -- captured once and replayed with pools
    restored and uniforms redrawn before every replay: outputs and pools equal
    the same calls run eagerly, and the accept equals the CPU reference."""
    cfg = synth.config(8, bs=8, vocab=3000)
    k, n, V = cfg.quad_k, cfg.block, cfg.vocab
    print_case("quadratic round as a HIP graph", cfg.bs, k, V)
    x = synth.make_attn_inputs(cfg, seed=10)
    case = AttnCase(x)
    _, masks = synth.quadratic_layout(k)
    tmask = torch.from_numpy(np.ascontiguousarray(masks).view(np.int64)).to("cuda")
    acc = synth.make_accept_inputs(cfg, seed=10)
    lg = np.random.default_rng(10).standard_normal((cfg.bs, n, V), dtype=np.float32) * 3
    logits = to_dev(synth.bf16_bits(lg))
    dev_in = dict(p=to_dev(acc.p), q=to_dev(acc.q), d=to_dev(acc.draft), u=to_dev(acc.u))
    max_kv = int(x.seq_lens.max()) + n
    k0, v0 = to_dev(x.k_pool), to_dev(x.v_pool)       # pristine pools

    def outputs(pools):
        o = torch.empty_like(case.q)
        ws_attn = va.workspace(max(1, va.attn_workspace_bytes(cfg.bs, n, cfg.hq, cfg.hkv, cfg.d,
                                                              max_kv)))
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        # marshalled once outside any capture, for its outputs and workspace
        _, acc_out = va.accept_quadratic_call(dev_in["p"], dev_in["q"], dev_in["d"], dev_in["u"],
                                              case.seq, logits, pools[0], pools[1], case.table,
                                              MASK, prepare_next=True, err=err)
        ws_q = va.workspace(va.accept_quadratic_workspace_bytes(cfg.bs, k, V))
        return dict(o=o, ws_attn=ws_attn, err=err, acc=acc_out, ws_q=ws_q)

    def round_calls(outs, pools):
        e1, _ = va.block_attn_tree_call(tmask, case.q, pools[0], pools[1], case.table, case.seq,
                                        max_kv, out=outs["o"], ws=outs["ws_attn"],
                                        err=outs["err"])
        e2, _ = va.accept_quadratic_call(dev_in["p"], dev_in["q"], dev_in["d"], dev_in["u"],
                                         case.seq, logits, pools[0], pools[1], case.table, MASK,
                                         prepare_next=True, out=outs["acc"], ws=outs["ws_q"],
                                         err=outs["err"])
        return (e1, e2)

    g_pools, e_pools = (k0.clone(), v0.clone()), (k0.clone(), v0.clone())
    g_out, e_out = outputs(g_pools), outputs(e_pools)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # one eager pass before the capture
        for e in round_calls(g_out, g_pools):
            e()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for e in round_calls(g_out, g_pools):
            e()
    eager = round_calls(e_out, e_pools)
    rng = np.random.default_rng(101)
    for rep in range(3):
        u = rng.random(acc.u.shape, dtype=np.float32)
        dev_in["u"].copy_(torch.from_numpy(u))
        for pl in (g_pools, e_pools):
            pl[0].copy_(k0)
            pl[1].copy_(v0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for e in eager:
            e()
        torch.cuda.synchronize()
        assert torch.equal(g_out["o"], e_out["o"]), (rep, "o")
        for key in e_out["acc"]:
            assert torch.equal(g_out["acc"][key], e_out["acc"][key]), (rep, key)
        for a, b in zip(g_pools, e_pools):
            assert torch.equal(a, b), (rep, "pools")
        assert int(g_out["err"].item()) == 0 and int(e_out["err"].item()) == 0
        ra = oracle.accept_batch(acc.p, acc.q, acc.draft, u, x.seq_lens)
        keep = ~ra["tie_sample"]
        check_tie_share(int((~keep).sum()), cfg.bs, "graph quadratic accept")
        got_len = e_out["acc"]["accept_len"].cpu().numpy()
        got_bonus = e_out["acc"]["bonus"].cpu().numpy()
        assert np.array_equal(got_len[keep], ra["accept_len"][keep])
        assert np.array_equal(got_bonus[keep], ra["bonus"][keep])
        print(f"replay {rep}: spine accept lengths {got_len.tolist()}", flush=True)


def _capture_and_compare(build, g_outs, e_outs, between, compare, reps=3):
    """Captures build(g_outs) (closures marshalled on the capture stream),
    then replays it `reps` times; before each replay between(rep) does eager
    work, after it the eager closures build(e_outs) run and compare(rep)
    checks both."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # one eager pass before the capture
        for e in build(g_outs):
            e()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for e in build(g_outs):
            e()
    eager = build(e_outs)
    for rep in range(reps):
        between(rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for e in eager:
            e()
        torch.cuda.synchronize()
        compare(rep)


def test_draft_round_replays_as_a_hip_graph(gpu_lib):
    """The draft pass round: its block (MASK fill), bidirectional block
    attention and the greedy draft argmax, replayed with new logits and
    verified ids written between replays; the drafts equal the lowest-index
    argmax of the bf16 rows."""
    cfg = synth.config(3, bs=8, argmax_vocab=20000)
    B = cfg.block
    print_case("draft round as a HIP graph", cfg.bs, B, cfg.argmax_vocab)
    x = synth.make_attn_inputs(cfg, seed=11)
    case = AttnCase(x)
    max_kv = int(x.seq_lens.max()) + B
    logits = to_dev(synth.make_argmax_logits(cfg, 11))
    vid = to_dev(np.zeros(cfg.bs, np.int32))
    i32 = dict(dtype=torch.int32, device="cuda")

    def outputs():
        return dict(prep=tuple(torch.empty((cfg.bs, B), **i32) for _ in range(3)),
                    o=torch.empty_like(case.q), tok=torch.empty(logits.shape[0], **i32),
                    ws=va.workspace(max(1, va.attn_workspace_bytes(cfg.bs, B, cfg.hq, cfg.hkv,
                                                                   cfg.d, max_kv))),
                    err=torch.zeros(1, **i32))

    def build(o):
        e1, _ = va.prepare_block_call(vid, case.seq, case.table, cfg.page, B, MASK, x.num_pages,
                                      None, out=o["prep"], err=o["err"])
        e2, _ = va.block_attn_call(synth.BIDIR, case.q, case.k, case.v, case.table, case.seq,
                                   max_kv, out=o["o"], ws=o["ws"], err=o["err"])
        e3, _ = va.draft_argmax_call(logits, out=o["tok"])
        return (e1, e2, e3)

    g, e = outputs(), outputs()
    rng = np.random.default_rng(111)
    state = {}

    def between(rep):
        bits = synth.bf16_bits(rng.standard_normal(tuple(logits.shape), dtype=np.float32) * 3)
        logits.copy_(to_dev(bits))
        vid.copy_(torch.from_numpy(rng.integers(0, 20000, cfg.bs).astype(np.int32)))
        state["bits"] = bits

    def compare(rep):
        for i in range(3):
            assert torch.equal(g["prep"][i], e["prep"][i]), (rep, "prep", i)
        assert torch.equal(g["o"], e["o"]) and torch.equal(g["tok"], e["tok"]), rep
        assert int(g["err"].item()) == 0 and int(e["err"].item()) == 0
        vals = synth.bf16_to_f32(state["bits"])
        want = np.array([oracle.argmax_lowest(r) for r in vals], np.int32)
        assert np.array_equal(e["tok"].cpu().numpy(), want), rep
        print(f"replay {rep}: drafts {e['tok'][:6].tolist()}...", flush=True)

    _capture_and_compare(build, g, e, between, compare)


def test_logits_round_replays_as_a_hip_graph(gpu_lib):
    """The logits verify round: the verify block, causal block attention and
    the accept over logits (temperature, top-k, top-p), replayed with new
    uniforms between replays; each replay equals the eager calls bit for
    bit."""
    cfg = synth.config(7, bs=6, vocab=20011)
    B, K = cfg.block, cfg.k_spec
    T, top_k, top_p = cfg.sampling
    print_case("logits round as a HIP graph", cfg.bs, B, cfg.vocab)
    x = synth.make_attn_inputs(cfg, seed=12)
    case = AttnCase(x)
    max_kv = int(x.seq_lens.max()) + B
    li = synth.make_logits_accept_inputs(cfg, seed=12)
    dev_in = dict(t=to_dev(li.target), dl=to_dev(li.draft_logits), d=to_dev(li.draft),
                  u=to_dev(li.u), vid=to_dev(np.zeros(cfg.bs, np.int32)))
    i32 = dict(dtype=torch.int32, device="cuda")

    def outputs():
        err = torch.zeros(1, **i32)
        _, acc = va.accept_logits_call(dev_in["t"], dev_in["dl"], dev_in["d"], dev_in["u"],
                                       case.seq, T, top_k, top_p, err=err)
        return dict(prep=tuple(torch.empty((cfg.bs, B), **i32) for _ in range(3)),
                    o=torch.empty_like(case.q), acc=acc, err=err,
                    ws=va.workspace(max(1, va.attn_workspace_bytes(cfg.bs, B, cfg.hq, cfg.hkv,
                                                                   cfg.d, max_kv))),
                    ws_acc=va.workspace(va.accept_logits_workspace_bytes(cfg.bs, K, cfg.vocab,
                                                                         top_k)))

    def build(o):
        e1, _ = va.prepare_block_call(dev_in["vid"], case.seq, case.table, cfg.page, B, MASK,
                                      x.num_pages, dev_in["d"], out=o["prep"], err=o["err"])
        e2, _ = va.block_attn_call(synth.CAUSAL, case.q, case.k, case.v, case.table, case.seq,
                                   max_kv, out=o["o"], ws=o["ws"], err=o["err"])
        e3, _ = va.accept_logits_call(dev_in["t"], dev_in["dl"], dev_in["d"], dev_in["u"],
                                      case.seq, T, top_k, top_p, out=o["acc"], ws=o["ws_acc"],
                                      err=o["err"])
        return (e1, e2, e3)

    g, e = outputs(), outputs()
    rng = np.random.default_rng(121)

    def between(rep):
        dev_in["u"].copy_(torch.from_numpy(rng.random(li.u.shape, dtype=np.float32)))

    def compare(rep):
        for i in range(3):
            assert torch.equal(g["prep"][i], e["prep"][i]), (rep, "prep", i)
        assert torch.equal(g["o"], e["o"]), rep
        for key in e["acc"]:
            assert torch.equal(g["acc"][key], e["acc"][key]), (rep, key)
        assert int(g["err"].item()) == 0 and int(e["err"].item()) == 0
        print(f"replay {rep}: accept lengths {e['acc']['accept_len'].tolist()}", flush=True)

    _capture_and_compare(build, g, e, between, compare)
