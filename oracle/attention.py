"""Block-query attention over a paged KV cache (reference form, float64).

What is computed (the pages' definition, written out):

* "SGLang strengthens diffusion LLMs: LLaDA 2.0", section "Attention Mask":
  one block-diffusion forward is a context query (the block's queries attend
  to all cached KV, exactly as chunked prefill) plus an intra-block query over
  the block's own KV, bidirectional (a rectangular mask) for block diffusion
  and causal (a triangular mask) for AR chunked prefill.
* "From DFlash to dLLM Self-Spec (4)", sections 4.4 / 4.4.1: the draft pass
  uses the bidirectional view and the verify pass switches to the causal view
  of the same block.
* "From DFlash to dLLM Self-Spec (4)", section 4.3.1 (I-DLM Block-N layout):
  clean/spec positions followed by MASK positions in one forward. MIXED mode
  makes the first n_c block rows causal and lets the MASK rows (i >= n_c) see
  the whole context, every clean position and every MASK position.
* "Unlocking Lossless Speedups in LLMs via Discrete Diffusion", method steps
  (the Tree sampler verified with tree attention): the block is a token tree;
  TREE mode gives each block row its own visibility bitmask over the block
  (bit j of row i set: row i sees block key j), which the caller fills with
  the node's ancestors and the node itself, so that a node attends exactly to
  the context and its own root path.

Readings where the pages are silent: scale 1/sqrt(D); query head h uses KV
head h // (Hq / Hkv); no positional term inside attention; the block's own K/V
sit in the cache at positions L_b .. L_b+B-1 before the attention runs.

Cache format: k_pool [num_pages, Hkv, P, D]; v_pool [num_pages, Hkv, D, P];
logical position n of request b lives in physical page page_table[b, n // P]
at offset n % P.
"""
import numpy as np

BIDIR, CAUSAL, MIXED, TREE = 0, 1, 2, 3


def visible(mode, i, jb, n_causal, tree_row=0):
    """May block row i see block key jb (both 0-based inside the block)?
    Context keys (before the block) are always visible. In TREE mode
    `tree_row` is row i's bitmask over the block keys."""
    if mode == BIDIR:
        return True
    if mode == CAUSAL:
        return jb <= i
    if mode == MIXED:
        return i >= n_causal or jb <= i
    if mode == TREE:
        return (int(tree_row) >> jb) & 1 == 1
    raise ValueError(mode)


def _tree_rows(tree, bs, B):
    """Per-request row masks [bs][B] (Python ints of B bits) from uint64 mask
    words: [B] (one tree, one word per row), [bs, B] (one tree per request),
    or, for blocks of any size, [bs, B, W] / [1, B, W] with W = ceil(B / 64)
    words per row, word w holding bits 64 w .. 64 w + 63 (or None)."""
    if tree is None:
        return [[0] * B for _ in range(bs)]
    t = np.asarray(tree, dtype=np.uint64)
    if t.ndim == 1:
        t = np.broadcast_to(t, (bs, B))
    if t.ndim == 2:
        t = t[:, :, None]
    t = np.broadcast_to(t, (bs, B, t.shape[-1]))
    return [[sum(int(w) << (64 * k) for k, w in enumerate(t[b, i])) for i in range(B)]
            for b in range(bs)]


def unpage_kv(k_pool, v_pool, page_table_row, n_tokens, kvh):
    """Logical K rows [n, D] and V rows [n, D] of one request and KV head,
    read one token at a time through the page table."""
    P = k_pool.shape[2]
    D = k_pool.shape[3]
    K = np.empty((n_tokens, D), np.float64)
    V = np.empty((n_tokens, D), np.float64)
    for n in range(n_tokens):
        page = int(page_table_row[n // P])
        off = n % P
        K[n] = k_pool[page, kvh, off, :]
        V[n] = v_pool[page, kvh, :, off]
    return K, V


def attn_row(qrow, K, V, L, B, i, mode, n_causal, scale, tree_row=0):
    """One query row: block row i of a request with committed length L.
    Returns (o [D], lse) with lse = max + ln(sum of exp(s - max))."""
    n = L + B
    vis = np.array([j < L or visible(mode, i, j - L, n_causal, tree_row) for j in range(n)])
    s = (K[:n] @ qrow) * scale
    s = s[vis]
    m = s.max()
    w = np.exp(s - m)
    tot = w.sum()
    o = (w @ V[:n][vis]) / tot
    return o, m + np.log(tot)


def block_attn_rows(q, k_pool, v_pool, page_table, seq_lens, mode, n_causal, scale=None,
                    rows=None, tree=None):
    """Per-row loop form. q [bs, B, Hq, D] float64. Returns o [bs, B, Hq, D]
    and lse [bs, B, Hq]; with `rows` (an iterable of (b, i, h)) only those rows
    are computed and the rest stay NaN. `tree`: TREE-mode row masks, [B]
    shared or [bs, B] per request (one word per row), or [bs or 1, B, W]
    words per row for any block size."""
    bs, B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    g = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    nc = np.broadcast_to(np.asarray(n_causal), (bs,))
    trow = _tree_rows(tree, bs, B)
    o = np.full(q.shape, np.nan)
    lse = np.full((bs, B, Hq), np.nan)
    if rows is None:
        rows = [(b, i, h) for b in range(bs) for i in range(B) for h in range(Hq)]
    cache = {}
    for b, i, h in rows:
        kvh = h // g
        L = int(seq_lens[b])
        if (b, kvh) not in cache:
            cache = {(b, kvh): unpage_kv(k_pool, v_pool, page_table[b], L + B, kvh)}
        K, V = cache[(b, kvh)]
        o[b, i, h], lse[b, i, h] = attn_row(q[b, i, h], K, V, L, B, i, mode, int(nc[b]), scale,
                                            trow[b][i])
    return o, lse


def mask_matrix(L, B, mode, n_causal, tree_rows=None):
    """Dense [B, L+B] visibility matrix: a block of ones over the context,
    then the intra-block rectangle (BIDIR), triangle (CAUSAL), the mixed
    layout (causal clean rows, all-visible MASK rows) or the rows' tree
    bitmasks (TREE)."""
    M = np.zeros((B, L + B), bool)
    M[:, :L] = True
    r = np.arange(B)[:, None]
    c = np.arange(B)[None, :]
    if mode == BIDIR:
        intra = np.ones((B, B), bool)
    elif mode == CAUSAL:
        intra = c <= r
    elif mode == MIXED:
        intra = (r >= n_causal) | (c <= r)
    else:
        bits = np.array([[(int(tree_rows[i]) >> j) & 1 for j in range(B)] for i in range(B)])
        intra = bits.astype(bool)
    M[:, L:] = intra
    return M


def block_attn_dense(q, k_pool, v_pool, page_table, seq_lens, mode, n_causal, scale=None,
                     tree=None):
    """Dense matrix form: per (request, KV head) the g query heads' [B, L+B]
    score matrices, masked to -inf, softmax along keys, times V."""
    bs, B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    g = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    nc = np.broadcast_to(np.asarray(n_causal), (bs,))
    trow = _tree_rows(tree, bs, B)
    o = np.empty(q.shape)
    lse = np.empty((bs, B, Hq))
    for b in range(bs):
        L = int(seq_lens[b])
        M = mask_matrix(L, B, mode, int(nc[b]), trow[b])
        for kvh in range(Hkv):
            K, V = unpage_kv(k_pool, v_pool, page_table[b], L + B, kvh)
            for hl in range(g):
                h = kvh * g + hl
                S = (q[b, :, h, :] @ K.T) * scale
                S = np.where(M, S, -np.inf)
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                tot = E.sum(axis=1, keepdims=True)
                o[b, :, h, :] = (E / tot) @ V
                lse[b, :, h] = (m + np.log(tot))[:, 0]
    return o, lse
