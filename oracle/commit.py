"""Committed-prefix KV after the accept (reference form).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed:

* "From DFlash to dLLM Self-Spec (4)", section 4.6 (KV lifecycle): after a
  round the runtime needs to know which KV slots to release (the speculative
  suffix that was not accepted) and how far each request advances; section
  4.4.1: the LinearSpec verify crops the cache to the committed length; and
  the recursive dynamic compaction note of the same page: the committable
  path is fixed inside the candidate block, then the accepted tokens are
  written out and the rejected suffix released.
* "Unlocking Lossless Speedups in LLMs via Discrete Diffusion", the Tree
  sampler: the accepted tokens form a root path of the token tree, so after
  the verify their K/V must become a contiguous prefix for the next round's
  causal view.

Readings where the pages are silent:
* The block occupies positions L .. L + B - 1 with node n (node 0 the root,
  the last committed token) at position L + n, as the tree verify lays it
  out. An accept with depth d and path p_1 .. p_d (node ids, p_k >= k) commits
  positions L .. L + d: position L + k (k >= 1) must hold the K and V of node
  p_k, which is copied there from position L + p_k (every KV head). A linear
  verify is the chain tree p_k = k, for which nothing moves.
* The released slots are those of positions L + d + 1 .. L + B - 1, listed in
  position order, then -1 up to B entries.
"""
import numpy as np


def slot_of(page_table_row, P, pos):
    """Cache slot of logical position pos: page * P + offset."""
    return int(page_table_row[pos // P]) * P + pos % P


def dest_position(L, k):
    """Position that receives the k-th accepted node (k = 0 .. d - 1)."""
    return L + 1 + k


def commit_kv(k_pool, v_pool, page_table, seq_lens, accept_len, path_nodes, B):
    """Returns (k_pool', v_pool', freed [bs, B]) after committing every
    request's accepted path. k_pool [num_pages, Hkv, P, D], v_pool
    [num_pages, Hkv, D, P]; path_nodes [bs, >= max depth] node ids or None
    (the chain)."""
    k = k_pool.copy()
    v = v_pool.copy()
    P = k_pool.shape[2]
    bs = len(seq_lens)
    freed = np.full((bs, B), -1, np.int64)
    for b in range(bs):
        L, d = int(seq_lens[b]), int(accept_len[b])
        path = [k_ + 1 for k_ in range(d)] if path_nodes is None else [int(x) for x in path_nodes[b][:d]]
        # read every source row before writing any destination
        src = [(k_pool[int(page_table[b][(L + n) // P]), :, (L + n) % P, :].copy(),
                v_pool[int(page_table[b][(L + n) // P]), :, :, (L + n) % P].copy()) for n in path]
        for idx, (kr, vr) in enumerate(src):
            pos = dest_position(L, idx)
            pg, off = int(page_table[b][pos // P]), pos % P
            k[pg, :, off, :] = kr
            v[pg, :, :, off] = vr
        for i, pos in enumerate(range(L + d + 1, L + B)):
            freed[b, i] = slot_of(page_table[b], P, pos)
    return k, v, freed
