"""Block preparation for one decode round (reference form).

Follows "From DFlash to dLLM Self-Spec (2): SGLang Spec V2", section 2.2.2
(decode step 1, preparing the DFlash block): token 0 of the block is the
previous round's verified token and the remaining block slots hold the mask
token; the same step produces each block token's position and its KV slot.
The verify pass of the same page (section 2.2.4) feeds the draft tokens in
place of the mask token. The capacity rule is the over-allocation of section
2.3.5 (a request reserves committed + 2 * block slots).

A KV slot is page * page_size + offset, where page is the request's page-table
entry for logical page position // page_size (the request -> token-slot map of
section 2.3.5).
"""
import numpy as np

ERR_SLOT = 1        # a page-table entry needed by the block is out of range
ERR_CAPACITY = 2    # L_b + B exceeds the request's page-table row


def prepare_block(verified_id, seq_lens, page_table, page_size, block, mask_token_id,
                  draft_tokens=None, num_pages=None):
    """Returns (block_ids, positions, cache_loc, err) for every request.

    block_ids[b, 0] = verified_id[b]; block_ids[b, i>=1] = mask token (draft
    pass) or draft_tokens[b, i-1] (verify pass). positions[b, i] = L_b + i.
    cache_loc[b, i] = page_table[b, pos // P] * P + pos % P, or -1 with an
    error bit set when the slot cannot be formed."""
    bs = len(seq_lens)
    max_pages = page_table.shape[1]
    block_ids = np.zeros((bs, block), np.int64)
    positions = np.zeros((bs, block), np.int64)
    cache_loc = np.zeros((bs, block), np.int64)
    err = 0
    for b in range(bs):
        L = int(seq_lens[b])
        if L < 0 or L + block > max_pages * page_size:
            err |= ERR_CAPACITY
        for i in range(block):
            if i == 0:
                block_ids[b, i] = verified_id[b]
            elif draft_tokens is None:
                block_ids[b, i] = mask_token_id
            else:
                block_ids[b, i] = draft_tokens[b, i - 1]
            pos = L + i
            positions[b, i] = pos
            n = pos // page_size
            page = int(page_table[b, n]) if 0 <= pos and n < max_pages else -1
            if page < 0 or (num_pages is not None and page >= num_pages):
                err |= ERR_SLOT
                cache_loc[b, i] = -1
            else:
                cache_loc[b, i] = page * page_size + pos % page_size
    return block_ids, positions, cache_loc, err


ERR_TREE = 16       # a node's parent is not an earlier node


def tree_depths(parent):
    """Depth of every node of a block given as parents in topological order:
    depth(0) = 0 (the root), depth(n) = depth(parent[n]) + 1. A node whose
    parent is not an earlier node, or that descends from such a node, has no
    depth (None)."""
    depth = [None] * len(parent)
    depth[0] = 0
    for n in range(1, len(parent)):
        p = int(parent[n])
        if 0 <= p < n and depth[p] is not None:
            depth[n] = depth[p] + 1
    return depth


def prepare_tree(verified_id, seq_lens, page_table, page_size, parent, mask_token_id,
                 node_tokens=None, num_pages=None):
    """Block preparation for a block whose tokens form a tree (or any layout
    described by parents in position order), following the same step of
    section 2.2.2 of the Spec V2 page: ids, positions and KV slots of the
    block in one pass.

    parent [N] (one layout for the batch) or [bs, N]; node 0 is the root.
    block_ids[b, 0] = verified_id[b]; block_ids[b, n>=1] = node_tokens[b, n]
    (or the mask token when node_tokens is None). positions[b, n] = L_b +
    depth(n): a node continues its parent's sequence, so siblings share a
    position (-1, with ERR_TREE, for a node without a depth). cache_loc[b, n]
    = the slot of position L_b + n: node n's K/V occupy the n-th slot after
    the committed prefix, as block row n of a linear block does (-1 with
    ERR_SLOT when the page is missing or out of range). ERR_CAPACITY when
    L_b + N does not fit the request's page-table row."""
    bs = len(seq_lens)
    par = np.asarray(parent)
    N = par.shape[-1]
    max_pages = page_table.shape[1]
    block_ids = np.zeros((bs, N), np.int64)
    positions = np.zeros((bs, N), np.int64)
    cache_loc = np.zeros((bs, N), np.int64)
    err = 0
    for b in range(bs):
        pb = par if par.ndim == 1 else par[b]
        depth = tree_depths(pb)
        L = int(seq_lens[b])
        if L < 0 or L + N > max_pages * page_size:
            err |= ERR_CAPACITY
        for n in range(N):
            if n == 0:
                block_ids[b, n] = verified_id[b]
            elif node_tokens is None:
                block_ids[b, n] = mask_token_id
            else:
                block_ids[b, n] = node_tokens[b, n]
            if depth[n] is None:
                err |= ERR_TREE
                positions[b, n] = -1
            else:
                positions[b, n] = L + depth[n]
            pos = L + n
            page_idx = pos // page_size
            page = int(page_table[b, page_idx]) if 0 <= pos and page_idx < max_pages else -1
            if page < 0 or (num_pages is not None and page >= num_pages):
                err |= ERR_SLOT
                cache_loc[b, n] = -1
            else:
                cache_loc[b, n] = page * page_size + pos % page_size
    return block_ids, positions, cache_loc, err
