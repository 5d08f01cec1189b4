"""Benchmark of one self-speculative decoding round on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  verify workloads: block_attn -> spec_accept_prepare (the accept, then the
                    next round's block: the block preparation of every round
                    runs inside the previous round's accept call)
  draft workload:   spec_prepare_block (draft pass) -> block_attn -> spec_draft_argmax
  tree workload:    spec_prepare_tree -> block_attn_tree -> spec_accept_tree_commit
  logits workload:  spec_prepare_block (verify pass) -> block_attn -> spec_accept_logits
  quadratic layout: block_attn_tree -> spec_accept_quadratic (the spine
                    drafts' accept, the hand-off of the next drafts, the
                    spine's commit and the next round's block in one call)
Inputs are resident in HBM before the timed region. Several copies of the
per-step inputs are cycled so that every step reads its KV pages and target
rows from HBM rather than from the 256 MB last-level cache.

Prints ONE JSON line: verified tokens/s, the roofline position of the call
that dominates the step (algorithmic bytes over its average duration from
HIP events on the launch stream), the whole step against its own roofline,
and the float64 CPU reference timed on a bounded sample of requests (which
also re-checks the GPU's outputs for those requests and counts ties).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified tokens/s per round (attn+accept) and % HBM roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
F32_PEAK_TFLOPS = 157.3
DEFAULT_CONFIG = 4   # the high-concurrency ragged verify, the largest single-GPU workload
MASK_TOKEN = 151669  # any id works: the block's ids are outputs only


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG, help="round configuration 1..11")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="the warm-up runs at least this long (after the W steps)")
    ap.add_argument("--copies", type=int, default=0, help="input copies cycled (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU reference leg")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as HIP graph replays (one graph per input copy)")
    ap.add_argument("--event-steps", type=int, default=24,
                    help="steps at the end of the warm-up (right before the timed region) with "
                         "HIP events recorded on the launch stream around every call, for the "
                         "per-call average durations (at least 20; the timed steps carry no "
                         "events: an event record drains the stream)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="before warmup, run one plain device copy of this many MB (a known-size "
                         "kernel for scaling HBM byte counters)")
    return ap.parse_args()


def kernel_sources_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "verify_attention_amd", "csrc"))):
        h.update(open(os.path.join(ROOT, "verify_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, src_hash, call="block_attn"):
    """HBM bytes per launch of `call` from the committed counter runs
    (profiles/traffic.json: FETCH_SIZE and WRITE_SIZE summed over the call's
    kernels, each scaled by a plain copy of known size), or None when they
    were taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    key = workload if call == "block_attn" else f"{workload}/{call}"
    if t.get("kernel_src") != src_hash or key not in t.get("workloads", {}):
        return None
    return int(t["workloads"][key]["traffic_bytes"])


def attn_alg_bytes_flops(cfg, seq_lens, tree_masks=None):
    """Algorithmic bytes / flops of one block_attn launch: K and V of positions
    [0, L_b + B) read once per KV head, Q read and O written once; 4 * D flops
    per visible (query row, key) pair."""
    esz = 2 if cfg.dtype == "bf16" else 4
    keys = (seq_lens.astype(np.int64) + cfg.block).sum()
    kv = 2 * keys * cfg.hkv * cfg.d * esz
    qo = 2 * cfg.bs * cfg.block * cfg.hq * cfg.d * esz
    B = cfg.block
    i = np.arange(B)
    if cfg.modes[0] == 0:
        intra = cfg.bs * B * B
    elif cfg.modes[0] == 1:
        intra = cfg.bs * int((i + 1).sum())
    elif cfg.modes[0] == 2:
        nc = cfg.n_causal
        intra = cfg.bs * int(np.where(i < nc, i + 1, B).sum())
    else:
        m = np.asarray(tree_masks)
        shared = m.ndim == 1 or (m.ndim == 3 and len(m) == 1)   # one tree for the batch
        intra = sum(bin(int(v)).count("1") for v in m.ravel()) * (cfg.bs if shared else 1)
    pairs = (seq_lens.astype(np.int64) * B).sum() + intra
    flops = 4 * cfg.d * pairs * cfg.hq
    return int(kv + qo), int(flops)


def tree_accept_alg_bytes(cfg):
    """Tree accept: the final node's target row streamed once, plus one
    gathered float per node, per request."""
    return int(cfg.bs * (cfg.vocab + cfg.block) * 4)


def accept_alg_bytes(cfg, accept_len):
    """Target / draft rows streamed by spec_accept: the residual pair p_j, q_j
    (or the bonus row p_K alone) per request, plus 2K gathered floats."""
    V, K = cfg.vocab, cfg.k_spec
    rows = np.where(accept_len < K, 2, 1)
    return int((rows * V * 4).sum() + cfg.bs * (2 * K + 1) * 4)


def block_prep_bytes(bs, B):
    """Block preparation: block ids, positions and slots written (int32)."""
    return int(3 * bs * B * 4)


def logits_accept_alg_bytes(cfg, esz=4):
    """Logits accept: every target and draft logits row streamed once (the
    top-k needs each row whole); the candidate re-reads, kept sets and the
    gathered values are overhead."""
    return int(cfg.bs * (2 * cfg.k_spec + 1) * cfg.vocab * esz)


def handoff_alg_bytes(cfg, esz=2):
    """Quadratic hand-off: the k logits rows of the chosen group per request
    read once, the drafts and the next block's tokens written."""
    k, n = cfg.quad_k, (cfg.quad_k + 1) ** 2
    return int(cfg.bs * (k * cfg.vocab * esz + (k + n) * 4))


def commit_alg_bytes(cfg, accept_len):
    """Committed prefix: every moved row's K and V read once and written once."""
    esz = 2 if cfg.dtype == "bf16" else 4
    return int(accept_len.sum()) * cfg.hkv * cfg.d * 2 * 2 * esz


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _sample_inputs(x, reqs):
    """The attention inputs of requests `reqs` alone over a pool holding only
    their pages (page table renumbered), so that the float64 copies stay small
    at any batch size."""
    from verify_attention_amd import synth
    cfg = x.cfg
    need = [-(-(int(x.seq_lens[b]) + cfg.block) // cfg.page) for b in reqs]
    pages = np.unique(np.concatenate([x.page_table[b, :n] for b, n in zip(reqs, need)]))
    remap = np.full(x.num_pages, -1, dtype=np.int64)
    remap[pages] = np.arange(len(pages))
    table = np.full((len(reqs), x.max_pages), -1, dtype=np.int32)
    for r, (b, n) in enumerate(zip(reqs, need)):
        table[r, :n] = remap[x.page_table[b, :n]]
    return synth.AttnInputs(cfg, x.seq_lens[reqs], table, len(pages), x.q[reqs],
                            x.k_pool[pages], x.v_pool[pages], x.n_causal[reqs])


def cpu_baseline(cfg, x, seconds, gpu, masks=None, acc=None, tacc=None, lacc=None,
                 quad=None):
    """The float64 reference, as it stands, on the host cores, over a bounded
    sample of this workload: requests taken in a seeded random order, each one
    its dense attention over all query heads plus its accept (or tree /
    logits accept, or the quadratic hand-off), until `seconds` have elapsed.
    The same requests' GPU outputs from the last timed step (`gpu`) are
    compared with the reference's: integer outputs bit for bit except draws
    within the float64 tie band, attention to the workload's tolerance (not
    for workloads whose step commits into the pools it reads). Returns the
    baseline entry with that check and its tie counts."""
    import oracle
    from oracle import quadratic
    from threadpoolctl import threadpool_info
    order = np.random.default_rng(12345).permutation(cfg.bs)
    mode = cfg.modes[-1]
    tol = 1e-2 if cfg.dtype == "bf16" else 1e-5
    check = dict(requests=0, mismatched_requests=0, accept_ties=0, sampling_ties=0,
                 attn_max_abs_err=0.0, attn_checked=gpu.get("o") is not None)
    t0 = time.perf_counter()
    t_check = 0.0        # time spent checking the GPU's outputs, not counted
    done = 0
    while done < cfg.bs:
        b = int(order[done])
        one = _sample_inputs(x, [b])
        shared = masks is not None and (masks.ndim == 1 or (masks.ndim == 3 and len(masks) == 1))
        tree = None if masks is None else (masks if shared else masks[b:b + 1])
        ro, _ = oracle.block_attn_dense(one.as_f64("q"), one.as_f64("k_pool"),
                                        one.as_f64("v_pool"), one.page_table, one.seq_lens, mode,
                                        cfg.n_causal, tree=tree)
        r = None
        if acc is not None:
            r = oracle.accept_request(acc.p[b], acc.q[b], acc.draft[b], acc.u[b], x.seq_lens[b])
        elif tacc is not None:
            r = oracle.tree_accept_request(tacc.parent[b], tacc.token[b], tacc.p[b], tacc.u[b],
                                           x.seq_lens[b])
        elif lacc is not None:
            T, k, top_p = cfg.sampling
            r = oracle.accept_logits_request(lacc.target[b], lacc.draft_logits[b], lacc.draft[b],
                                             lacc.u[b], x.seq_lens[b], float(np.float32(T)), k,
                                             float(np.float32(top_p)))
        hand = None
        if quad is not None and r is not None:
            hand = quadratic.handoff(quad["logits_f32"](b), r["accept_len"], cfg.quad_k,
                                     r["bonus"], MASK_TOKEN)
        t1 = time.perf_counter()
        el = t1 - t0 - t_check
        done += 1
        # the check of the GPU's outputs (not timed)
        if gpu.get("o") is not None:
            e = float(np.max(np.abs(gpu["o"](b) - ro[0])))
            check["attn_max_abs_err"] = max(check["attn_max_abs_err"], e)
            bad = e > tol
        else:
            bad = False
        if r is not None:
            check["accept_ties"] += int(r["tie_accept"])
            check["sampling_ties"] += int(r["tie_sample"])
            if not r["tie_sample"]:
                got = gpu["accept"](b)
                bad |= got["accept_len"] != r["accept_len"] or got["bonus"] != r["bonus"]
                bad |= got["new_seq_lens"] != r["new_seq_len"]
                bad |= not np.array_equal(got["out_tokens"], r["out_tokens"])
                if hand is not None:
                    bad |= not np.array_equal(gpu["handoff"](b), hand[0])
        check["requests"] += 1
        check["mismatched_requests"] += int(bad)
        t_check += time.perf_counter() - t1
        if el >= seconds:
            break
    check["attn_max_abs_err"] = float(f"{check['attn_max_abs_err']:.3e}")
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    tok_per_req = cfg.quad_k + 1 if cfg.quad_k else cfg.block
    what = ("tree accept" if tacc is not None else "logits accept" if lacc is not None else
            "accept" + (" + hand-off" if quad is not None else "") if acc is not None else None)
    return dict(value=done * tok_per_req / el, unit="verified tokens/s", cores=int(threads),
                kind="oracle", cpu_model=cpu_model(),
                sample=f"{done} of the {cfg.bs} requests of this workload (seeded order): dense "
                       f"float64 attention over all {cfg.hq} query heads"
                       f"{' + ' + what if what else ''}, one request after another, {el:.1f} s; "
                       f"host has {len(os.sched_getaffinity(0))} cores",
                parity_sample=check)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the hot path runs on a single MI355X); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    import verify_attention_amd as va
    from verify_attention_amd import synth

    va.load()
    dev = torch.device("cuda:0")
    cfg = synth.config(args.config)
    mode = cfg.modes[-1]
    quad = cfg.quad_k > 0           # quadratic layout: bitmask attention + the linear accept
    tree = mode == synth.TREE and not quad
    x = synth.make_attn_inputs(cfg, seed=args.seed)
    parents = masks = tacc = acc = lacc = qlogits = None
    if tree:
        parents, masks = synth.make_trees(cfg, args.seed)
        tacc = synth.make_tree_accept_inputs(cfg, args.seed, parents)
    elif cfg.sampling:
        lacc = synth.make_logits_accept_inputs(cfg, args.seed)
    elif quad:
        _, masks = synth.quadratic_layout(cfg.quad_k)
        parents = synth.quadratic_parents(cfg.quad_k)
        acc = synth.make_accept_inputs(cfg, seed=args.seed)
        # the layout's logits rows (draft and verify in one forward), bf16
        qlogits = synth.make_argmax_logits(synth.config(args.config, argmax_vocab=cfg.vocab),
                                           args.seed, rows=cfg.bs * cfg.block).reshape(
            cfg.bs, cfg.block, cfg.vocab)
    elif cfg.vocab:
        acc = synth.make_accept_inputs(cfg, seed=args.seed)
    logits = synth.make_argmax_logits(cfg, seed=args.seed) if cfg.argmax_vocab else None
    verified, drafts = synth.make_round_state(cfg, args.seed)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # bytes one step streams (KV, Q, and the accept's rows or the logits):
    # enough input copies are cycled that a copy is not re-read before about
    # 768 MB have gone by, so no step finds its inputs in the 256 MB LLC
    step_bytes = x.k_pool.nbytes + x.v_pool.nbytes + x.q.nbytes
    if acc is not None:
        step_bytes += 2 * cfg.bs * cfg.vocab * 4
    if tacc is not None:
        step_bytes += tree_accept_alg_bytes(cfg)
    if lacc is not None:
        step_bytes += logits_accept_alg_bytes(cfg)
    if logits is not None:
        step_bytes += logits.nbytes
    if qlogits is not None:
        step_bytes += handoff_alg_bytes(cfg)
    copies = args.copies or max(2, int(np.ceil(768e6 / step_bytes)))
    sets = []
    for _ in range(copies):
        s = dict(q=up(x.q), k=up(x.k_pool), v=up(x.v_pool))
        if acc is not None:
            s.update(p=up(acc.p), qd=up(acc.q), u=up(acc.u), draft=up(acc.draft))
        if tacc is not None:
            s.update(p=up(tacc.p), u=up(tacc.u))
        if lacc is not None:
            s.update(tl=up(lacc.target), dl=up(lacc.draft_logits), u=up(lacc.u),
                     draft=up(lacc.draft))
        if logits is not None:
            s["logits"] = up(logits)
        if qlogits is not None:
            s["qlogits"] = up(qlogits)
        sets.append(s)
    table, seq = up(x.page_table), up(x.seq_lens)
    vid, dr = up(verified), up(drafts)
    max_kv = int(x.seq_lens.max()) + cfg.block
    bs, B = cfg.bs, cfg.block
    o = torch.empty_like(sets[0]["q"])
    ws_attn = va.workspace(va.attn_workspace_bytes(bs, B, cfg.hq, cfg.hkv, cfg.d, max_kv))
    prep_out = tuple(torch.empty((bs, B), dtype=torch.int32, device=dev) for _ in range(3))
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    if tree or quad:
        # one shared tree of mask words, [1, B, W], goes to the call as [B, W]
        shared_words = masks.ndim == 3 and len(masks) == 1 and bs > 1
        tmask = torch.from_numpy(np.ascontiguousarray(masks[0] if shared_words else masks)
                                 .view(np.int64)).to(dev)
        tpar = up(np.ascontiguousarray(parents, dtype=np.int32))
    if tree:
        ttok = up(tacc.token)
        ws_tacc = va.workspace(va.accept_tree_workspace_bytes(bs, B, cfg.vocab))
    if lacc is not None:
        ws_acc = va.workspace(va.accept_logits_workspace_bytes(bs, cfg.k_spec, cfg.vocab,
                                                               cfg.sampling[1]))
    if acc is not None:
        ws_acc = va.workspace(va.accept_workspace_bytes(bs, cfg.k_spec, cfg.vocab))
    # every call is checked once; the timed loop re-enqueues pre-marshalled
    # calls, all on one stream of their own (which a graph capture can use)
    rs = torch.cuda.Stream(device=dev)
    calls = []      # per step: list of (name, [enqueue per input copy])
    acc_out = None
    if tree or quad:
        if tree:  # a quadratic round's block is prepared by the previous round's accept
            calls.append(("spec_prepare_tree", [va.prepare_tree_call(
                vid, seq, table, cfg.page, tpar, MASK_TOKEN, x.num_pages, ttok,
                out=prep_out, err=err, stream=rs)[0]] * copies))
        calls.append(("block_attn_tree", [va.block_attn_tree_call(
            tmask, s["q"], s["k"], s["v"], table, seq, max_kv, out=o, ws=ws_attn,
            err=err, stream=rs)[0] for s in sets]))
    else:
        if acc is None:   # the draft pass and the logits verify prepare their own block
            calls.append(("spec_prepare_block", [va.prepare_block_call(
                vid, seq, table, cfg.page, B, MASK_TOKEN, x.num_pages,
                None if mode == synth.BIDIR else dr, out=prep_out, err=err,
                stream=rs)[0]] * copies))
        calls.append(("block_attn", [va.block_attn_call(
            mode, s["q"], s["k"], s["v"], table, seq, max_kv, n_causal=cfg.n_causal, out=o,
            ws=ws_attn, err=err, stream=rs)[0] for s in sets]))
    if tree:
        lst = []
        for s in sets:
            # the tree accept, whose accepted path becomes the committed
            # prefix of the cache in the same call
            c, acc_out = va.accept_tree_commit_call(tpar, ttok, s["p"], s["u"], seq, s["k"],
                                                    s["v"], table, out=acc_out, ws=ws_tacc,
                                                    err=err, stream=rs)
            lst.append(c)
        calls.append(("spec_accept_tree_commit", lst))
    elif quad:
        lst = []
        ws_q = va.workspace(va.accept_quadratic_workspace_bytes(bs, cfg.quad_k, cfg.vocab))
        for s in sets:
            c, acc_out = va.accept_quadratic_call(s["p"], s["qd"], s["draft"], s["u"], seq,
                                                  s["qlogits"], s["k"], s["v"], table,
                                                  MASK_TOKEN, prepare_next=True, out=acc_out,
                                                  ws=ws_q, err=err, stream=rs)
            lst.append(c)
        calls.append(("spec_accept_quadratic", lst))
    elif acc is not None:
        lst = []
        for s in sets:
            c, acc_out = va.accept_prepare_call(s["p"], s["qd"], s["draft"], s["u"], seq, table,
                                                cfg.page, B, MASK_TOKEN, x.num_pages,
                                                out=acc_out, ws=ws_acc, err=err, stream=rs)
            lst.append(c)
        calls.append(("spec_accept_prepare", lst))
    elif lacc is not None:
        lst = []
        for s in sets:
            c, acc_out = va.accept_logits_call(s["tl"], s["dl"], s["draft"], s["u"], seq,
                                               *cfg.sampling, out=acc_out, ws=ws_acc, err=err,
                                               stream=rs)
            lst.append(c)
        calls.append(("spec_accept_logits", lst))
    elif logits is not None:
        tokens = torch.empty(logits.shape[0], dtype=torch.int32, device=dev)
        calls.append(("spec_draft_argmax", [va.draft_argmax_call(s["logits"], out=tokens,
                                                                 stream=rs)[0]
                                            for s in sets]))
    stream = rs
    torch.cuda.synchronize()

    def step(i, ev=None):
        for c, (_, fns) in enumerate(calls):
            if ev is not None:
                ev[c].record(stream)
            fns[i % copies]()
        if ev is not None:
            ev[-1].record(stream)

    if args.copy_calib_mb:
        n = args.copy_calib_mb << 20
        src_c = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst_c = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        dst_c.copy_(src_c)
        torch.cuda.synchronize()
        del src_c, dst_c
    # W warm-up steps, continued until the warm-up has run for at least
    # --warmup-seconds of wall time: the first passes over a multi-GB KV pool
    # run measurably slower (clock and address-translation ramp-up), and the
    # number reported is the steady-state rate of a serving loop
    warm_steps, t_w = 0, time.perf_counter()
    while warm_steps < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        step(warm_steps)
        warm_steps += 1
        if warm_steps % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # per-call durations: the last --event-steps warm-up steps carry HIP events
    # around every call (recorded on the launch stream), right before the
    # timed region and in the same steady state; an event's time includes the
    # dispatch that follows it
    n_ev = max(20, args.event_steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
           for _ in range(n_ev)]
    for i in range(n_ev):
        step(warm_steps + i, evs[i])
    torch.cuda.synchronize()
    per_call_us = {}
    for c, (name, _) in enumerate(calls):
        per_call_us[name] = float(np.mean([e[c].elapsed_time(e[c + 1]) for e in evs]) * 1e3)
    torch.cuda.synchronize()
    graphs = []
    if args.graph:
        # one HIP graph per input copy, captured on the calls' own stream (the
        # library allocates, clears and synchronises nothing), then replayed
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=rs):
                for _, fns in calls:
                    fns[c]()
            graphs.append(g)
        for i in range(2 * copies):
            graphs[i % copies].replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if graphs:
            graphs[i % copies].replay()
        else:
            step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if int(err.item()) != 0:
        raise RuntimeError(f"kernels reported data errors: {int(err.item())}")
    # outputs of the last timed step, for the CPU leg's check
    gpu = {}
    if not (tree or quad):
        o_last = o.float().cpu().numpy().astype(np.float64)
    else:
        # the step's commit moved rows inside the cycled pools: the check's
        # attention runs once more, untimed, over a fresh copy of the inputs
        o_chk = va.block_attn_tree(tmask, sets[0]["q"], up(x.k_pool), up(x.v_pool), table, seq,
                                   max_kv)
        o_last = o_chk.float().cpu().numpy().astype(np.float64)
    gpu["o"] = lambda b: o_last[b]
    if acc_out is not None:
        snap = {k: v.cpu().numpy() for k, v in acc_out.items()}
        gpu["accept"] = lambda b: {k: v[b] for k, v in snap.items()}
    if quad:
        hsnap = acc_out["next_draft"].cpu().numpy()
        gpu["handoff"] = lambda b: hsnap[b]
    al = acc_out["accept_len"].cpu().numpy() if acc_out is not None else None
    cl = acc_out["commit_len"].cpu().numpy() if acc_out is not None else None

    # algorithmic bytes per call
    alg_bytes, alg_flops = attn_alg_bytes_flops(cfg, x.seq_lens, masks)
    esz = 2 if cfg.dtype == "bf16" else 4
    call_bytes = {"block_attn": alg_bytes, "block_attn_tree": alg_bytes,
                  "spec_prepare_block": block_prep_bytes(bs, B),
                  "spec_prepare_tree": block_prep_bytes(bs, B)}
    if al is not None:
        if tree:
            call_bytes["spec_accept_tree_commit"] = tree_accept_alg_bytes(cfg) + \
                int(al.sum()) * cfg.hkv * cfg.d * 2 * 2 * esz
        elif lacc is not None:
            call_bytes["spec_accept_logits"] = logits_accept_alg_bytes(cfg)
        elif quad:
            call_bytes["spec_accept_quadratic"] = (accept_alg_bytes(cfg, al) +
                                                   handoff_alg_bytes(cfg) +
                                                   commit_alg_bytes(cfg, al) +
                                                   2 * bs * B * 4)
        else:
            call_bytes["spec_accept_prepare"] = accept_alg_bytes(cfg, al) + block_prep_bytes(bs, B)
    if logits is not None:
        call_bytes["spec_draft_argmax"] = int(logits.nbytes)
    src_hash = kernel_sources_hash()
    mfma_peak = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else F32_PEAK_TFLOPS

    def roofline(name):
        us = per_call_us[name]
        ab = call_bytes[name]
        gbs = ab / (us * 1e-6) / 1e9
        rl = {"kernel": name, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
              "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
              "traffic": measured_traffic(cfg.name, src_hash,
                                          "block_attn" if name.startswith("block_attn") else name),
              "traffic_unit": "bytes per launch", "alg_bytes_per_launch": int(ab),
              "avg_us": round(us, 2), "event_samples": n_ev}
        if name.startswith("block_attn"):
            tflops = alg_flops / (us * 1e-6) / 1e12
            rl["mfma_frac"] = round(tflops / mfma_peak, 4)
            if alg_flops / alg_bytes > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9):
                # flops per byte above the ridge: the matrix cores bound the kernel
                rl.update(bound="mfma", achieved=round(tflops, 1), peak=mfma_peak,
                          unit="TFLOP/s", frac=round(tflops / mfma_peak, 4),
                          alg_flops_per_launch=alg_flops, hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
        return rl

    dominant = max(per_call_us, key=per_call_us.get)
    tokens_per_step = bs * (cfg.quad_k + 1 if quad else B)
    value = tokens_per_step * args.steps / wall
    step_bytes_alg = sum(call_bytes[n] for n, _ in calls)
    step_roof_us = max(step_bytes_alg / (HBM_PEAK_GBS * 1e9),
                       alg_flops / (mfma_peak * 1e12)) * 1e6
    ms = wall / args.steps * 1e3
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "verified tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps + n_ev,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": ("synthetic (seeded N(0,1) Q/K/V, normal target logits, draft logits = target "
                 "+ normal noise)" if lacc is not None else
                 "synthetic (seeded N(0,1) Q/K/V, softmax-of-normal target/draft rows"
                 + (", N(0, 3^2) bf16 layout logits)" if quad else ")")
                 if acc is not None or tree else
                 "synthetic (seeded N(0,1) Q/K/V, N(0, 3^2) bf16 draft logits)"
                 if logits is not None else "synthetic (seeded N(0,1) Q/K/V)"),
        "config": {"workload": cfg.name, "bs": bs, "block": B, "hq": cfg.hq, "hkv": cfg.hkv,
                   "head_dim": cfg.d, "page": cfg.page, "mode": synth.MODE_NAMES[mode],
                   "ctx": [cfg.ctx_lo, cfg.ctx_hi], "vocab": cfg.vocab or cfg.argmax_vocab,
                   "k_spec": cfg.k_spec, "input_copies": copies,
                   "step": [n for n, _ in calls], "launch": "hip_graph" if graphs else "eager",
                   **({"layout": f"quadratic, k = {cfg.quad_k}",
                       "verified_tokens_per_request": cfg.quad_k + 1} if quad else {})},
        "roofline": roofline(dominant),
        "step_roofline": {"alg_bytes": int(step_bytes_alg), "roofline_us": round(step_roof_us, 2),
                          "measured_us": round(ms * 1e3, 2),
                          "frac": round(step_roof_us / (ms * 1e3), 4)},
        "calls": {n: roofline(n) for n, _ in calls if n != dominant},
        "kernel_src": src_hash,
    }
    if cl is not None:
        line["committed_tokens_per_s"] = round(float(cl.sum() * args.steps / wall), 1)
        line["mean_commit_len"] = float(cl.mean())
    if not args.no_cpu:
        quad_in = None
        if quad:
            qf = lambda b: synth.bf16_to_f32(qlogits[b])
            quad_in = {"logits_f32": qf}
        line["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_seconds, gpu, masks,
                                            acc if acc is not None else None, tacc, lacc,
                                            quad_in)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
