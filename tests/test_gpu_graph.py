"""One verify round captured in a HIP graph through the C ABI. The calls
allocate nothing, clear nothing and never synchronise with the host, so the
round — the verify pass's block preparation, block attention and the accept
that also prepares the next round's block — can be recorded once and replayed.
Every replay is checked against the same calls run eagerly on the same
inputs, bit for bit, with eager work (new uniforms, new draft tokens) between
the replays; the eager results are also checked against the CPU reference."""
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
