"""Benchmark of one self-speculative decoding round on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  verify workloads: spec_prepare_block (verify pass) -> block_attn -> spec_accept
  draft workload:   spec_prepare_block (draft pass)  -> block_attn -> spec_draft_argmax
  tree workload:    block_attn_tree -> spec_accept_tree -> spec_commit_kv
  logits workload:  spec_prepare_block (verify pass) -> block_attn -> spec_accept_logits
  quadratic layout: block_attn_tree (draft groups + verify spine) -> spec_accept
Inputs are resident in HBM before the timed region. Several copies of the
per-step inputs are cycled so that every step reads its KV pages and target
rows from HBM rather than from the 256 MB last-level cache.

Prints ONE JSON line: verified tokens/s (bs * B per step), the roofline
position of the call that dominates the step (block_attn, or the accept /
argmax call when it takes longer: algorithmic bytes over its event-timed
average duration) and the float64 CPU reference timed on a bounded sample.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="round configuration 1..9")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="the warm-up runs at least this long (after the W steps)")
    ap.add_argument("--copies", type=int, default=0, help="input copies cycled (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU reference leg")
    ap.add_argument("--event-every", type=int, default=8,
                    help="HIP events bracket the calls of every n-th timed step (an event "
                         "record drains the stream: on every step they would slow it)")
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
        intra = sum(bin(int(v)).count("1") for v in m.ravel()) * (cfg.bs if m.ndim == 1 else 1)
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


def logits_accept_alg_bytes(cfg, esz=4):
    """Logits accept: every target and draft logits row streamed once (the
    top-k needs each row whole); the candidate re-reads, kept sets and the
    gathered values are overhead."""
    return int(cfg.bs * (2 * cfg.k_spec + 1) * cfg.vocab * esz)


def cpu_baseline(cfg, x, acc, seconds, masks=None, tacc=None, lacc=None):
    """The float64 reference, as it stands, on the host cores: dense attention
    per (request, KV head) plus the sequential accept (or tree accept),
    request after request, until `seconds` have elapsed (at least one
    request)."""
    import oracle
    from threadpoolctl import threadpool_info
    q, kp, vp = x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool")
    mode = cfg.modes[0]
    t0 = time.perf_counter()
    done = 0
    while True:
        b = done % cfg.bs
        sl = slice(b, b + 1)
        oracle.block_attn_dense(q[sl], kp, vp, x.page_table[sl], x.seq_lens[sl], mode,
                                cfg.n_causal,
                                tree=None if masks is None else (masks if masks.ndim == 1 else masks[sl]))
        if acc is not None:
            oracle.accept_request(acc.p[b], acc.q[b], acc.draft[b], acc.u[b], x.seq_lens[b])
        if tacc is not None:
            oracle.tree_accept_request(tacc.parent[b], tacc.token[b], tacc.p[b], tacc.u[b],
                                       x.seq_lens[b])
        if lacc is not None:
            T, k, top_p = cfg.sampling
            oracle.accept_logits_request(lacc.target[b], lacc.draft_logits[b], lacc.draft[b],
                                         lacc.u[b], x.seq_lens[b], float(np.float32(T)), k,
                                         float(np.float32(top_p)))
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    return dict(value=done * cfg.block / el, unit="verified tokens/s", cores=int(threads),
                kind="oracle",
                sample=f"{done} requests of this workload (attention over all {cfg.hq} query "
                       f"heads{' + accept' if acc is not None or tacc is not None or lacc is not None else ''}"
                       f"), one after another, {el:.1f} s; host has "
                       f"{len(os.sched_getaffinity(0))} cores")


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
    parents = masks = tacc = acc = lacc = None
    if tree:
        parents, masks = synth.make_trees(cfg, args.seed)
        tacc = synth.make_tree_accept_inputs(cfg, args.seed, parents)
    elif cfg.sampling:
        lacc = synth.make_logits_accept_inputs(cfg, args.seed)
    elif quad:
        _, masks = synth.quadratic_layout(cfg.quad_k)
        acc = synth.make_accept_inputs(cfg, seed=args.seed)
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
        tmask = torch.from_numpy(masks.view(np.int64)).to(dev)
    if tree:
        tpar, ttok = up(tacc.parent), up(tacc.token)
        ws_tacc = va.workspace(va.accept_tree_workspace_bytes(bs, B, cfg.vocab))
    if lacc is not None:
        ws_acc = va.workspace(va.accept_logits_workspace_bytes(bs, cfg.k_spec, cfg.vocab,
                                                               cfg.sampling[1]))
    if acc is not None or lacc is not None:
        if acc is not None:
            ws_acc = va.workspace(va.accept_workspace_bytes(bs, cfg.k_spec, cfg.vocab))
        acc_out = dict(accept_len=torch.empty(bs, dtype=torch.int32, device=dev),
                       commit_len=torch.empty(bs, dtype=torch.int32, device=dev),
                       bonus=torch.empty(bs, dtype=torch.int32, device=dev),
                       out_tokens=torch.empty((bs, cfg.k_spec + 1), dtype=torch.int32, device=dev),
                       new_seq_lens=torch.empty(bs, dtype=torch.int32, device=dev))
    elif not tree and logits is not None:
        tokens = torch.empty(logits.shape[0], dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    # every call is checked once; the timed loop re-enqueues pre-marshalled calls
    # a tree round has no linear block to prepare (node positions follow the
    # tree depths): its step is the tree attention and the tree accept
    prep_call = None if (tree or quad) else va.prepare_block_call(
        vid, seq, table, cfg.page, B, 0, x.num_pages, None if mode == synth.BIDIR else dr,
        out=prep_out, err=err)[0]
    if tree:
        attn_calls = [va.block_attn_tree_call(tmask, s["q"], s["k"], s["v"], table, seq, max_kv,
                                              out=o, ws=ws_attn, err=err)[0] for s in sets]
        acc_out = None
        tail_calls = []
        for s in sets:
            # the tree accept, whose accepted path becomes the committed
            # prefix of the cache in the same call
            acc_call, acc_out = va.accept_tree_commit_call(tpar, ttok, s["p"], s["u"], seq,
                                                           s["k"], s["v"], table, out=acc_out,
                                                           ws=ws_tacc, err=err)
            tail_calls.append(acc_call)
    elif quad:
        attn_calls = [va.block_attn_tree_call(tmask, s["q"], s["k"], s["v"], table, seq, max_kv,
                                              out=o, ws=ws_attn, err=err)[0] for s in sets]
    else:
        attn_calls = [va.block_attn_call(mode, s["q"], s["k"], s["v"], table, seq, max_kv,
                                         n_causal=cfg.n_causal, out=o, ws=ws_attn, err=err)[0]
                      for s in sets]
    if acc is not None:
        tail_calls = [va.accept_call(s["p"], s["qd"], s["draft"], s["u"], seq, out=acc_out,
                                     ws=ws_acc, err=err)[0] for s in sets]
    elif lacc is not None:
        tail_calls = [va.accept_logits_call(s["tl"], s["dl"], s["draft"], s["u"], seq,
                                            *cfg.sampling, out=acc_out, ws=ws_acc, err=err)[0]
                      for s in sets]
    elif logits is not None:
        tail_calls = [va.draft_argmax_call(s["logits"], out=tokens)[0] for s in sets]
    elif not tree:
        tail_calls = [lambda: None] * copies  # attention-only workload

    def step(i, ev=None):
        if prep_call is not None:
            prep_call()
        if ev is not None:
            ev[0].record(stream)
        attn_calls[i % copies]()
        if ev is not None:
            ev[1].record(stream)
        tail_calls[i % copies]()
        if ev is not None:
            ev[2].record(stream)

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
    # per-call durations: events around the calls of every n-th timed step
    every = max(1, args.event_every)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] if i % every == 0 else None
           for i in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if int(err.item()) != 0:
        raise RuntimeError(f"kernels reported data errors: {int(err.item())}")

    evs = [e for e in evs if e is not None]
    attn_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    tail_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    alg_bytes, alg_flops = attn_alg_bytes_flops(cfg, x.seq_lens, masks)
    attn_s = attn_ms.mean() / 1e3
    achieved = alg_bytes / attn_s / 1e9
    mfma_peak = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else F32_PEAK_TFLOPS
    tokens_per_step = bs * B
    value = tokens_per_step * args.steps / wall
    extra = {}
    if acc is not None or tree or lacc is not None:
        al = acc_out["accept_len"].cpu().numpy()
        cl = acc_out["commit_len"].cpu().numpy()
        if tree:
            # plus the committed rows' K and V, read once and written once
            esz = 2 if cfg.dtype == "bf16" else 4
            ab = tree_accept_alg_bytes(cfg) + int(al.sum()) * cfg.hkv * cfg.d * 2 * 2 * esz
        elif lacc is not None:
            ab = logits_accept_alg_bytes(cfg)
        else:
            ab = accept_alg_bytes(cfg, al)
        extra["accept"] = dict(avg_us=round(tail_ms.mean() * 1e3, 2),
                               alg_bytes=ab, achieved_gbs=round(ab / (tail_ms.mean() / 1e3) / 1e9, 1),
                               mean_commit_len=float(cl.mean()))
        extra["committed_tokens_per_s"] = float(cl.sum() * args.steps / wall)
    elif logits is not None:
        ab = logits.nbytes
        extra["draft_argmax"] = dict(avg_us=round(tail_ms.mean() * 1e3, 2), alg_bytes=int(ab),
                                     achieved_gbs=round(ab / (tail_ms.mean() / 1e3) / 1e9, 1))
    attn_rl = {"kernel": "block_attn", "bound": "hbm",
               "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(achieved / HBM_PEAK_GBS, 4),
               "traffic": measured_traffic(cfg.name, kernel_sources_hash()),
               "traffic_unit": "bytes per launch",
               "alg_bytes_per_launch": alg_bytes, "avg_us": round(attn_ms.mean() * 1e3, 2),
               "mfma_frac": round(alg_flops / attn_s / 1e12 / mfma_peak, 4)}
    if alg_flops / alg_bytes > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        # flops per byte above the ridge: the matrix cores bound the kernel
        tflops = alg_flops / attn_s / 1e12
        attn_rl.update(bound="mfma", achieved=round(tflops, 1), peak=mfma_peak, unit="TFLOP/s",
                       frac=round(tflops / mfma_peak, 4), alg_flops_per_launch=alg_flops,
                       hbm_frac=round(achieved / HBM_PEAK_GBS, 4))
    tail_rl = None
    if acc is not None or tree or lacc is not None or logits is not None:
        tail_name = ("spec_accept_tree_commit" if tree else "spec_accept_logits"
                     if lacc is not None else "spec_accept" if acc is not None else
                     "spec_draft_argmax")
        tail_s = tail_ms.mean() / 1e3
        tail_rl = {"kernel": tail_name, "bound": "hbm", "achieved": round(ab / tail_s / 1e9, 1),
                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": round(ab / tail_s / 1e9 / HBM_PEAK_GBS, 4),
                   "traffic": measured_traffic(cfg.name, kernel_sources_hash(), tail_name),
                   "traffic_unit": "bytes per launch", "alg_bytes_per_launch": int(ab),
                   "avg_us": round(tail_ms.mean() * 1e3, 2)}
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "verified tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "event_steps": len(evs),
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": ("synthetic (seeded N(0,1) Q/K/V, normal target logits, draft logits = target "
                 "+ normal noise)" if lacc is not None else
                 "synthetic (seeded N(0,1) Q/K/V, softmax-of-normal target/draft rows)"
                 if acc is not None or tree else
                 "synthetic (seeded N(0,1) Q/K/V, N(0, 3^2) bf16 draft logits)"
                 if logits is not None else "synthetic (seeded N(0,1) Q/K/V)"),
        "config": {"workload": cfg.name, "bs": bs, "block": B, "hq": cfg.hq, "hkv": cfg.hkv,
                   "head_dim": cfg.d, "page": cfg.page, "mode": synth.MODE_NAMES[mode],
                   "ctx": [cfg.ctx_lo, cfg.ctx_hi], "vocab": cfg.vocab or cfg.argmax_vocab,
                   "k_spec": cfg.k_spec, "input_copies": copies,
                   **({"layout": f"quadratic, k = {cfg.quad_k}"} if quad else {})},
        "roofline": attn_rl,
        "kernel_src": kernel_sources_hash(),
        **extra,
    }
    if tail_rl is not None and tail_rl["avg_us"] > attn_rl["avg_us"]:
        # the call that dominates the step carries the roofline
        line["roofline"], line["attn_roofline"] = tail_rl, attn_rl
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(cfg, x, acc, args.cpu_seconds, masks, tacc, lacc)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
