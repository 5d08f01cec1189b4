"""Seeded synthetic inputs for one self-speculative decoding round.

This module only draws random numbers and lays them out in the library's
buffer formats. It holds none of the method's arithmetic (no masking, no
attention, no acceptance test, no residual sampling): the tests, the bench and
the CPU reference all take their inputs from here, and nothing here imports
either side.

Workload shapes follow the five round configurations of the DFlash / I-DLM /
block-diffusion pages (SGLang Spec V2 verify block, I-DLM Block-N mixed layout,
LLaDA-style draft block). Where a page leaves a distribution open the choice is
stated next to the field.

Buffer formats (the library's contract):
  q        [bs, B, Hq, D]              query rows of the block (bf16 or fp32)
  k_pool   [num_pages, Hkv, P, D]      K pages, token-major inside a page
  v_pool   [num_pages, Hkv, D, P]      V pages, dim-major inside a page
  page_table [bs, max_pages] int32     physical page of logical page n; -1 unused
  seq_lens [bs] int32                  committed context length L_b; the block
                                       occupies positions L_b .. L_b+B-1 and its
                                       K/V are already in the pages
  p [bs, K+1, V] f32, q_probs [bs, K, V] f32, draft [bs, K] i32, u [bs, K+1] f32
"""
from __future__ import annotations

import dataclasses
import numpy as np

BIDIR, CAUSAL, MIXED, TREE = 0, 1, 2, 3
MODE_NAMES = {BIDIR: "BIDIR", CAUSAL: "CAUSAL", MIXED: "MIXED", TREE: "TREE"}


@dataclasses.dataclass(frozen=True)
class RoundConfig:
    """One round's shapes. `ctx_lo/ctx_hi` give the committed-context range;
    `commit_hi` > 0 adds the previous round's commit length ~ U{1..commit_hi}."""
    name: str
    bs: int
    hq: int
    hkv: int
    d: int
    page: int
    block: int
    modes: tuple
    dtype: str                 # "bf16" | "f32"
    ctx_lo: int
    ctx_hi: int
    commit_hi: int = 0
    n_causal: int = 0          # MIXED: clean (causal) positions at the block head
    vocab: int = 0             # 0: no accept step in this round
    k_spec: int = 0            # draft tokens checked by the accept step
    logit_sigma: float = 3.0
    q_noise_sigma: float = 0.0  # >0: q-logits = p-logits + N(0, s^2); 0: independent
    argmax_vocab: int = 0      # draft pass: argmax of bf16 logits over this vocab
    tree_depth: int = 0        # TREE: the block is a token tree of this many levels at most
    tree_width: int = 0        # TREE: >0: a beam-shaped tree, tree_depth levels of this many nodes
    # accept from logits under (temperature, top_k, top_p); () = accept from
    # stored probability rows
    sampling: tuple = ()
    quad_k: int = 0            # >0: the block is the quadratic layout of quad_k drafts


# The five round configurations. Sizes are the workloads the pages describe:
#  1 tiny fp32 correctness round (both intra-block masks, vocab 512)
#  2 Qwen3-8B-shaped verify at concurrency 32 (page size 16, block 16)
#  3 block-diffusion draft pass, ragged contexts, block 32, greedy draft ids
#  4 high-concurrency ragged verify (batch 256)
#  5 I-DLM style mixed layout: 8 clean causal + 8 MASK bidirectional positions
#  7 the verify of 2 with the accept taking logits under the sampling
#    parameters of the Uno evaluation protocol (temperature 1, top-k 50,
#    top-p 0.95): target logits N(0, 3^2), draft logits = target + N(0, 0.5^2)
#  8 quadratic layout: the verify of 2 with k = 4 drafts and a group of k
#    MASK tokens after the root and after every draft (25 positions), draft
#    and verify in one forward; the accept checks the k drafts
#  9 the draft pass of 3 with a 128-position block: g * B = 512 query rows
#    per KV head put the attention's flops per KV byte (about 470) above the
#    MI355X ridge (2.5 PFLOP/s / 8 TB/s = 312.5), the matrix-core-bound
#    shape; attention only (no argmax tail)
#  6 tree verify: the Qwen3-8B-shaped verify of 2 with a 32-node token tree
#    (at most 16 levels) as the block, one tree per request; target logits
#    N(0, 6^2), peaked enough (top-4 mass about 2/3 at this vocabulary) that
#    top-candidate children are accepted at useful rates
# 10 the Tree sampler's own setting, (B, K, V) = (16, 32, 32): 15 drafted
#    positions, top-32 candidates per position, the best 32 prefixes kept per
#    length, so a beam-shaped tree of 1 + 15 * 32 = 481 nodes (8 mask words a
#    row; g * B = 1924 query rows per KV head); the Qwen3-8B-shaped verify of
#    6 otherwise, at 8 requests
# 11 the quadratic layout of 8 at the verify's own block of 16: k = 15
#    drafts and a group of 15 MASK tokens after the root and after every
#    draft, 256 positions (4 mask words a row, g * B = 1024 query rows per KV
#    head)
CONFIGS = {
    1: RoundConfig("tiny_f32", bs=1, hq=2, hkv=1, d=64, page=16, block=8,
                   modes=(BIDIR, CAUSAL), dtype="f32", ctx_lo=256, ctx_hi=256,
                   vocab=512, k_spec=7, logit_sigma=2.0, q_noise_sigma=0.0),
    2: RoundConfig("qwen3_8b_verify_bs32", bs=32, hq=32, hkv=8, d=128, page=16,
                   block=16, modes=(CAUSAL,), dtype="bf16", ctx_lo=1024,
                   ctx_hi=1024, vocab=151936, k_spec=15, logit_sigma=3.0,
                   q_noise_sigma=0.5),
    3: RoundConfig("draft_bidir_bs64", bs=64, hq=16, hkv=4, d=128, page=32,
                   block=32, modes=(BIDIR,), dtype="bf16", ctx_lo=1024,
                   ctx_hi=9216, argmax_vocab=157184, logit_sigma=3.0),
    4: RoundConfig("ragged_verify_bs256", bs=256, hq=32, hkv=8, d=128, page=16,
                   block=16, modes=(CAUSAL,), dtype="bf16", ctx_lo=1024,
                   ctx_hi=9216, commit_hi=16, vocab=151936, k_spec=15,
                   logit_sigma=3.0, q_noise_sigma=0.5),
    5: RoundConfig("idlm_mixed_bs128", bs=128, hq=32, hkv=8, d=128, page=16,
                   block=16, modes=(MIXED,), dtype="bf16", ctx_lo=4096,
                   ctx_hi=4096, n_causal=8, vocab=151936, k_spec=8,
                   logit_sigma=3.0, q_noise_sigma=0.5),
    6: RoundConfig("tree_verify_bs32", bs=32, hq=32, hkv=8, d=128, page=16,
                   block=32, modes=(TREE,), dtype="bf16", ctx_lo=1024,
                   ctx_hi=1024, tree_depth=16, vocab=151936, k_spec=31,
                   logit_sigma=6.0, q_noise_sigma=0.5),
    8: RoundConfig("quadratic_verify_bs32", bs=32, hq=32, hkv=8, d=128, page=16,
                   block=25, modes=(TREE,), dtype="bf16", ctx_lo=1024, ctx_hi=1024,
                   vocab=151936, k_spec=4, logit_sigma=3.0, q_noise_sigma=0.5, quad_k=4),
    7: RoundConfig("qwen3_8b_verify_bs32_logits", bs=32, hq=32, hkv=8, d=128, page=16,
                   block=16, modes=(CAUSAL,), dtype="bf16", ctx_lo=1024,
                   ctx_hi=1024, vocab=151936, k_spec=15, logit_sigma=3.0,
                   q_noise_sigma=0.5, sampling=(1.0, 50, 0.95)),
    10: RoundConfig("tree_sampler_b481_bs8", bs=8, hq=32, hkv=8, d=128, page=16,
                    block=481, modes=(TREE,), dtype="bf16", ctx_lo=1024, ctx_hi=1024,
                    tree_depth=15, tree_width=32, vocab=151936, k_spec=480,
                    logit_sigma=6.0, q_noise_sigma=0.5),
    11: RoundConfig("quadratic_k15_verify_bs32", bs=32, hq=32, hkv=8, d=128, page=16,
                    block=256, modes=(TREE,), dtype="bf16", ctx_lo=1024, ctx_hi=1024,
                    vocab=151936, k_spec=15, logit_sigma=3.0, q_noise_sigma=0.5, quad_k=15),
    9: RoundConfig("draft_bidir_b128_bs64", bs=64, hq=16, hkv=4, d=128, page=32,
                   block=128, modes=(BIDIR,), dtype="bf16", ctx_lo=1024, ctx_hi=9216),
}


def config(cid: int, **overrides) -> RoundConfig:
    """A round configuration, optionally with fields replaced (smaller test
    variants keep the shape family but shrink bs, vocab or contexts)."""
    return dataclasses.replace(CONFIGS[cid], **overrides)


# Independent child streams, one per drawn item, so that resizing one item
# never shifts the numbers of another.
_STREAMS = dict(pages=1, ctx=2, commit=3, q=4, k=5, v=6, plogit=7, qnoise=8,
                draft=9, uniform=10, argmax=11, ncausal=12, poison=13, tree=14)


def rng_for(seed: int, item: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), _STREAMS[item]])


# ---------------------------------------------------------------- bf16 values
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even) and return the
    16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bf16 bit patterns."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng, shape, sigma=1.0, chunk=1 << 26):
    """N(0, sigma^2) drawn in float32 and rounded once to bf16 -> uint16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        out[s:e] = bf16_bits(x)
    return out.reshape(shape)


def _normal_f32(rng, shape, sigma=1.0):
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


# ------------------------------------------------------------ attention round
@dataclasses.dataclass
class AttnInputs:
    cfg: RoundConfig
    seq_lens: np.ndarray       # [bs] int32
    page_table: np.ndarray     # [bs, max_pages] int32
    num_pages: int
    q: np.ndarray              # [bs, B, Hq, D] uint16 (bf16 bits) or float32
    k_pool: np.ndarray         # [num_pages, Hkv, P, D]
    v_pool: np.ndarray         # [num_pages, Hkv, D, P]
    n_causal: np.ndarray       # [bs] int32 (MIXED clean-prefix lengths)

    @property
    def max_pages(self):
        return self.page_table.shape[1]

    def as_f64(self, name):
        """Exact float64 values of a stored tensor."""
        a = getattr(self, name)
        if a.dtype == np.uint16:
            return bf16_to_f32(a).astype(np.float64)
        return a.astype(np.float64)


def context_lengths(cfg: RoundConfig, seed: int) -> np.ndarray:
    """Committed lengths L_b: context ~ U{ctx_lo..ctx_hi}, plus the previous
    round's commit ~ U{1..commit_hi} when the workload has one."""
    ctx = rng_for(seed, "ctx").integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=cfg.bs)
    if cfg.commit_hi:
        ctx = ctx + rng_for(seed, "commit").integers(1, cfg.commit_hi + 1, size=cfg.bs)
    return ctx.astype(np.int32)


def page_layout(cfg: RoundConfig, seq_lens: np.ndarray, seed: int, shuffle=True,
                spare_pages: int = 0):
    """Each request owns ceil((L_b + 2B) / P) pages (the over-allocation rule
    of the Spec V2 page: reserved = committed + 2 * block). Physical page ids
    come from a random permutation of the pool; unused table entries are -1."""
    P, B = cfg.page, cfg.block
    need = (seq_lens.astype(np.int64) + 2 * B + P - 1) // P
    total = int(need.sum()) + spare_pages
    max_pages = int(need.max())
    ids = np.arange(total, dtype=np.int32)
    if shuffle:
        ids = rng_for(seed, "pages").permutation(total).astype(np.int32)
    table = np.full((cfg.bs, max_pages), -1, dtype=np.int32)
    o = 0
    for b in range(cfg.bs):
        n = int(need[b])
        table[b, :n] = ids[o:o + n]
        o += n
    return table, total


def make_attn_inputs(cfg: RoundConfig, seed: int, shuffle=True,
                     n_causal_per_req=False, poison_tail=False) -> AttnInputs:
    """Q/K/V ~ N(0,1) (bf16: drawn in float32, rounded once). Every pool slot
    holds a value, including slots past a request's end. With `poison_tail`,
    slots at positions >= L_b + B are overwritten with NaN so that any read
    of them shows up in the output."""
    seq = context_lengths(cfg, seed)
    table, num_pages = page_layout(cfg, seq, seed, shuffle=shuffle)
    shp_q = (cfg.bs, cfg.block, cfg.hq, cfg.d)
    shp_k = (num_pages, cfg.hkv, cfg.page, cfg.d)
    shp_v = (num_pages, cfg.hkv, cfg.d, cfg.page)
    if cfg.dtype == "bf16":
        q = _normal_bf16(rng_for(seed, "q"), shp_q)
        k = _normal_bf16(rng_for(seed, "k"), shp_k)
        v = _normal_bf16(rng_for(seed, "v"), shp_v)
        nan = np.uint16(0x7FC0)
    else:
        q = _normal_f32(rng_for(seed, "q"), shp_q)
        k = _normal_f32(rng_for(seed, "k"), shp_k)
        v = _normal_f32(rng_for(seed, "v"), shp_v)
        nan = np.float32(np.nan)
    if poison_tail:
        P = cfg.page
        for b in range(cfg.bs):
            end = int(seq[b]) + cfg.block
            for n in range(table.shape[1]):
                pg = table[b, n]
                if pg < 0:
                    continue
                lo = max(end - n * P, 0)
                if lo < P:
                    k[pg, :, lo:, :] = nan
                    v[pg, :, :, lo:] = nan
    if n_causal_per_req:
        nc = rng_for(seed, "ncausal").integers(0, cfg.block + 1, size=cfg.bs)
    else:
        nc = np.full(cfg.bs, cfg.n_causal, dtype=np.int64)
    return AttnInputs(cfg, seq, table, num_pages, q, k, v, nc.astype(np.int32))


# -------------------------------------------------------------- token trees
def random_tree_parents(rng, n_nodes: int, max_depth: int) -> np.ndarray:
    """parent[n] of a random token tree in topological order: node 0 is the
    root (depth 0); every other node extends the previous node with
    probability 1/2 (a main path with side branches, as a top-candidate tree
    has) and otherwise picks a uniformly random earlier node; parents are
    limited to depth below max_depth - 1."""
    parent = np.full(n_nodes, -1, dtype=np.int32)
    depth = np.zeros(n_nodes, dtype=np.int32)
    for n in range(1, n_nodes):
        ok = np.flatnonzero(depth[:n] < max_depth - 1)
        chain = rng.random() < 0.5 and depth[n - 1] < max_depth - 1
        parent[n] = n - 1 if chain else ok[rng.integers(len(ok))]
        depth[n] = depth[parent[n]] + 1
    return parent


def _node_logits(cfg: "RoundConfig", rp, N: int) -> np.ndarray:
    """Target logits of one request's N nodes, l ~ N(0, sigma^2) (one row per
    node, drawn in node order from the request's share of the stream)."""
    return rp.standard_normal((N, cfg.vocab)) * cfg.logit_sigma


def _draft_logits(cfg: "RoundConfig", lp_row: np.ndarray, rq) -> np.ndarray:
    """The drafter's logits for the token after a node: its target logits
    plus N(0, s^2) noise."""
    return lp_row + rq.standard_normal(len(lp_row)) * max(cfg.q_noise_sigma, 1e-3)


def beam_tree_parents(cfg: "RoundConfig", lp: np.ndarray, rq) -> np.ndarray:
    """parent[n] of the tree the Tree sampler keeps: per position the top
    tree_width candidates of the drafter, and of all extensions of the kept
    prefixes the tree_width with the largest summed draft log-probability
    (ties: earlier prefix, then the higher-ranked candidate), for tree_depth
    positions: the root, then tree_depth levels of tree_width nodes, a level's
    nodes grouped by parent in level order and, under one parent, by rank.
    The drafter's distribution is taken per prefix (node x's children are
    candidates of softmax(_draft_logits(lp[x]))). One draft row is drawn per
    node in node order, leaves included, as make_tree_accept_inputs draws
    them."""
    W, N = cfg.tree_width, cfg.block
    parent = np.full(N, -1, dtype=np.int32)
    score = np.zeros(N)
    level = [0]
    nxt = 1
    for _ in range(cfg.tree_depth):
        cands = []                        # (-score, prefix order, rank, prefix)
        for order, x in enumerate(level):
            lq = _draft_logits(cfg, lp[x], rq)
            m = lq.max()
            logq = lq - (m + np.log(np.exp(lq - m).sum()))
            top = _top_indices(lq, W)
            cands += [(-(score[x] + logq[t]), order, r, x) for r, t in enumerate(top)]
        kept = sorted(sorted(cands)[:W], key=lambda c: (c[1], c[2]))
        level = []
        for negs, _, _, x in kept:
            parent[nxt], score[nxt] = x, -negs
            level.append(nxt)
            nxt += 1
    for _ in level:                       # the last level's draft rows (unused here)
        rq.standard_normal(cfg.vocab)
    return parent


def tree_row_masks(parent: np.ndarray) -> np.ndarray:
    """uint64 row masks of a tree of at most 64 nodes in topological order:
    bit j of row n is set iff node j is node n or one of its ancestors."""
    if len(parent) > 64:
        raise ValueError("one word per row holds at most 64 nodes; use tree_row_words")
    return tree_row_words(parent)[:, 0].copy()


def tree_row_words(parent: np.ndarray) -> np.ndarray:
    """The same row masks for a tree of any size as W = ceil(N / 64) uint64
    words per row, [N, W]: bit j of the mask is bit j % 64 of word j // 64."""
    n_nodes = len(parent)
    W = (n_nodes + 63) // 64
    rows = [0] * n_nodes
    for n in range(n_nodes):
        rows[n] = 1 << n
        if parent[n] >= 0:
            rows[n] |= rows[parent[n]]
    out = np.zeros((n_nodes, W), dtype=np.uint64)
    for n in range(n_nodes):
        for w in range(W):
            out[n, w] = np.uint64((rows[n] >> (64 * w)) & ((1 << 64) - 1))
    return out


def quadratic_layout(k: int):
    """The quadratic layout of k drafts as block rows: the spine (the root,
    then drafts s_1 .. s_k) at positions i * (k + 1), and after spine token j
    a group G_j of k MASK positions j * (k + 1) + 1 .. j * (k + 1) + k, which
    proposes the continuation if exactly s_1 .. s_j are accepted. Returns
    (role [n] as (kind, j, m) tuples, row masks) with n = (k + 1)^2: spine
    token i sees spine tokens 0 .. i (causal); a member of G_j sees spine
    tokens 0 .. j and every member of G_j (bidirectional inside the group).
    The masks are [n] uint64 for n <= 64, else W = ceil(n / 64) words per row
    of the one shared layout, [1, n, W] (bit j of a row is bit j % 64 of word
    j // 64); n <= 512."""
    n = (k + 1) * (k + 1)
    if n > 512:
        raise ValueError("the layout needs (k + 1)^2 <= 512 positions")
    role, rows = [], []
    for pos in range(n):
        j, m = divmod(pos, k + 1)
        spine = sum(1 << (t * (k + 1)) for t in range(j + 1))
        if m == 0:
            role.append(("spine", j, 0))
            rows.append(spine)
        else:
            group = sum(1 << (j * (k + 1) + 1 + t) for t in range(k))
            role.append(("mask", j, m - 1))
            rows.append(spine | group)
    W = (n + 63) // 64
    words = np.array([[(r >> (64 * w)) & ((1 << 64) - 1) for w in range(W)] for r in rows],
                     dtype=np.uint64)
    return role, (words[:, 0].copy() if W == 1 else words[None])


def quadratic_parents(k: int) -> np.ndarray:
    """Position order of the quadratic layout as parents: spine token i
    follows spine token i - 1; member 0 of group G_j follows spine token j and
    member m follows member m - 1 (the layout's tokens after spine token j).
    Only the positions come from this; the attention masks are those of
    quadratic_layout."""
    n = (k + 1) * (k + 1)
    parent = np.full(n, -1, dtype=np.int32)
    for pos in range(1, n):
        j, m = divmod(pos, k + 1)
        if m == 0:
            parent[pos] = (j - 1) * (k + 1)
        else:
            parent[pos] = j * (k + 1) if m == 1 else pos - 1
    return parent


def make_trees(cfg: RoundConfig, seed: int, per_request=True):
    """Token trees for a TREE round: parents [bs, B] and row masks [bs, B]
    (per_request), or one tree shared by the batch ([B] each). Blocks of more
    than 64 nodes get their masks as words: [bs, B, W] (or [1, B, W] for one
    shared tree)."""
    r = rng_for(seed, "tree")
    depth = cfg.tree_depth or cfg.block
    wide = cfg.block > 64
    masks = tree_row_words if wide else tree_row_masks
    if cfg.tree_width:
        if 1 + depth * cfg.tree_width != cfg.block:
            raise ValueError("a beam tree has 1 + tree_depth * tree_width nodes")
        # the beam follows the round's own target and draft rows (the streams
        # of make_tree_accept_inputs, request by request)
        rp, rq = rng_for(seed, "plogit"), rng_for(seed, "qnoise")
        draw = lambda: beam_tree_parents(cfg, _node_logits(cfg, rp, cfg.block), rq)
    else:
        draw = lambda: random_tree_parents(r, cfg.block, depth)
    if not per_request:
        par = draw()
        return par, (masks(par)[None] if wide else masks(par))
    par = np.stack([draw() for _ in range(cfg.bs)])
    return par, np.stack([masks(p) for p in par])


# --------------------------------------------------------------- accept step
@dataclasses.dataclass
class AcceptInputs:
    p: np.ndarray       # [bs, K+1, V] float32 target rows (row i scores block token i+1)
    q: np.ndarray       # [bs, K, V]   float32 draft rows
    draft: np.ndarray   # [bs, K] int32 draft tokens, d_i ~ q_i
    u: np.ndarray       # [bs, K+1] float32 uniforms in [0, 1)


def _softmax_rows64(x):
    x = x.astype(np.float64)
    x -= x.max(axis=-1, keepdims=True)
    np.exp(x, out=x)
    x /= x.sum(axis=-1, keepdims=True)
    return x


def make_accept_inputs(cfg: RoundConfig, seed: int, bs: int | None = None) -> AcceptInputs:
    """p = softmax(l), l ~ N(0, sigma^2) per row. q = softmax(l + N(0, s^2))
    when the workload ties the draft to the target (the verify configs), or
    softmax of independent logits (the tiny config). Distributions are built in
    float64 one request at a time and stored as float32. Draft tokens are drawn
    from the stored q rows with numpy's categorical sampler; the accept step's
    own uniforms come from a separate stream."""
    bs = cfg.bs if bs is None else bs
    K, V = cfg.k_spec, cfg.vocab
    p = np.empty((bs, K + 1, V), np.float32)
    q = np.empty((bs, K, V), np.float32)
    draft = np.empty((bs, K), np.int32)
    rp, rq, rd = rng_for(seed, "plogit"), rng_for(seed, "qnoise"), rng_for(seed, "draft")
    for b in range(bs):
        lp = rp.standard_normal((K + 1, V)) * cfg.logit_sigma
        p[b] = _softmax_rows64(lp)
        if cfg.q_noise_sigma > 0:
            lq = lp[:K] + rq.standard_normal((K, V)) * cfg.q_noise_sigma
        else:
            lq = rq.standard_normal((K, V)) * cfg.logit_sigma
        q[b] = _softmax_rows64(lq)
        for i in range(K):
            w = q[b, i].astype(np.float64)
            draft[b, i] = rd.choice(V, p=w / w.sum())
    u = rng_for(seed, "uniform").random((bs, K + 1), dtype=np.float32)
    return AcceptInputs(p, q, draft, u)


@dataclasses.dataclass
class TreeAcceptInputs:
    parent: np.ndarray  # [bs, N] int32, parent[:, 0] = -1
    token: np.ndarray   # [bs, N] int32 candidate token of each node (node 0 unused)
    p: np.ndarray       # [bs, N, V] float32 target rows (row n: the token after node n)
    u: np.ndarray       # [bs, N] float32 uniforms in [0, 1)


def _top_indices(x: np.ndarray, k: int) -> np.ndarray:
    """The indices of the k largest entries of x, largest first, the lower
    index first among equal values (a stable descending sort's first k)."""
    if k >= len(x):
        return np.argsort(-x, kind="stable")
    cand = np.argpartition(-x, k - 1)[:k]
    kth = x[cand].min()
    cand = np.flatnonzero(x >= kth)            # every entry tied with the k-th
    return cand[np.lexsort((cand, -x[cand]))][:k]


def make_tree_accept_inputs(cfg: RoundConfig, seed: int, parents: np.ndarray,
                            bs: int | None = None) -> TreeAcceptInputs:
    """Target rows p = softmax(l), l ~ N(0, sigma^2), one per node. The
    children of node x take the top tokens of a draft distribution q_x =
    softmax(l_x + N(0, s^2)) (largest first, as a top-candidate tree keeps
    them), so siblings carry distinct tokens and the first child is the
    draft's most likely token."""
    bs = cfg.bs if bs is None else bs
    N, V = parents.shape[-1], cfg.vocab
    par = np.broadcast_to(parents, (bs, N)).astype(np.int32)
    p = np.empty((bs, N, V), np.float32)
    token = np.zeros((bs, N), np.int32)
    rp, rq = rng_for(seed, "plogit"), rng_for(seed, "qnoise")
    for b in range(bs):
        lp = _node_logits(cfg, rp, N)
        p[b] = _softmax_rows64(lp)
        for x in range(N):
            kids = np.flatnonzero(par[b] == x)
            if len(kids) == 0 and not cfg.tree_width:
                continue      # (a beam tree's rows are drawn for every node)
            lq = _draft_logits(cfg, lp[x], rq)
            if len(kids):
                token[b, kids] = _top_indices(lq, len(kids))
    u = rng_for(seed, "uniform").random((bs, N), dtype=np.float32)
    return TreeAcceptInputs(par.copy(), token, p, u)


@dataclasses.dataclass
class LogitsAcceptInputs:
    target: np.ndarray  # [bs, K+1, V] target logits (row i scores block token i+1)
    draft_logits: np.ndarray  # [bs, K, V] draft logits
    draft: np.ndarray   # [bs, K] int32 draft tokens
    u: np.ndarray       # [bs, K+1] float32 uniforms in [0, 1)


def make_logits_accept_inputs(cfg: RoundConfig, seed: int, bs: int | None = None,
                              dtype: str = "f32") -> LogitsAcceptInputs:
    """Target logits l ~ N(0, sigma^2) per row and draft logits l + N(0, s^2)
    (float32, or bf16 bits when dtype is "bf16"). Draft token i is the token at
    rank R of draft row i (largest logit first, lower index first on ties),
    R ~ Geometric(0.35) - 1 capped at 39, so drafts sit among the drafter's
    top candidates as a sampler with top-k truncation draws them. The accept
    step's uniforms come from a separate stream."""
    bs = cfg.bs if bs is None else bs
    K, V = cfg.k_spec, cfg.vocab
    tl = np.empty((bs, K + 1, V), np.float32)
    dl = np.empty((bs, K, V), np.float32)
    draft = np.empty((bs, K), np.int32)
    rp, rq, rd = rng_for(seed, "plogit"), rng_for(seed, "qnoise"), rng_for(seed, "draft")
    for b in range(bs):
        tl[b] = rp.standard_normal((K + 1, V), dtype=np.float32) * np.float32(cfg.logit_sigma)
        dl[b] = tl[b, :K] + rq.standard_normal((K, V), dtype=np.float32) * np.float32(
            cfg.q_noise_sigma)
        if dtype == "bf16":  # the drafts are ranked on the stored values
            tl[b] = bf16_to_f32(bf16_bits(tl[b]))
            dl[b] = bf16_to_f32(bf16_bits(dl[b]))
        ranks = np.minimum(rd.geometric(0.35, size=K) - 1, 39)
        for i in range(K):
            draft[b, i] = np.argsort(-dl[b, i], kind="stable")[ranks[i]]
    u = rng_for(seed, "uniform").random((bs, K + 1), dtype=np.float32)
    if dtype == "bf16":
        return LogitsAcceptInputs(bf16_bits(tl), bf16_bits(dl), draft, u)
    return LogitsAcceptInputs(tl, dl, draft, u)


def make_argmax_logits(cfg: RoundConfig, seed: int, rows: int | None = None) -> np.ndarray:
    """Draft-pass logits [bs * (B-1), V] as bf16 bits, N(0, sigma^2) rounded to
    bf16 (equal maxima occur; the lowest index is the defined winner)."""
    rows = cfg.bs * (cfg.block - 1) if rows is None else rows
    return _normal_bf16(rng_for(seed, "argmax"), (rows, cfg.argmax_vocab), cfg.logit_sigma)


def make_round_state(cfg: RoundConfig, seed: int, vocab: int | None = None):
    """verified_id [bs] (previous round's bonus token) and the verify pass's
    draft tokens [bs, B-1], uniform over the vocabulary."""
    vocab = vocab or cfg.vocab or cfg.argmax_vocab or 32000
    r = rng_for(seed, "draft")
    verified = r.integers(0, vocab, size=cfg.bs).astype(np.int32)
    drafts = r.integers(0, vocab, size=(cfg.bs, cfg.block - 1)).astype(np.int32)
    return verified, drafts
