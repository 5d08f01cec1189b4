"""Plain, slow, float64 CPU reference for one self-speculative decoding round.

TEST INFRASTRUCTURE ONLY. Nothing in the library path imports, calls or links
this package; only the tests, the package's smoke check and the bench's
CPU-baseline leg use it. It shares no code with the HIP path: it re-implements
paging from the page table, the intra-block masks, the softmax and the
acceptance rule from the pages' definitions, in float64 NumPy.

Modules:
  prepare   -- block ids / positions / cache slots of one round's block
  attention -- block-query attention over a paged KV cache (BIDIR, CAUSAL,
               MIXED and TREE masks), two forms: a per-row loop and a dense
               masked-softmax matrix form
  accept    -- speculative accept: p/q rejection test, longest accepted
               prefix, residual (or bonus) sample, committed length; the greedy
               special case; argmax with the lowest index winning; the tree
               walk (recursive rejection over deterministic candidates)
  sampling  -- temperature / top-k / top-p processing of logits rows, and the
               accept on processed target and draft rows
  commit    -- the committed prefix's K/V after an accept (the accepted tree
               path moved to contiguous positions) and the released slots
  quadratic -- the quadratic layout's hand-off: the next round's drafts from
               the MASK group after the last accepted spine token

Parity status: every function here is pinned by CPU tests against closed
forms, library routines, brute force or exact enumeration (see the tests
named test_oracle_*). None is "parity unpinned".
"""
from .prepare import prepare_block, prepare_tree, tree_depths
from .attention import (BIDIR, CAUSAL, MIXED, TREE, visible, block_attn_rows,
                        block_attn_dense, attn_row, unpage_kv, mask_matrix)
from .accept import (accept_request, accept_batch, greedy_accept_request, argmax_lowest,
                     tree_accept_request, tree_children)
from .sampling import (sampling_filter, rank_order, accept_logits_request,
                       accept_logits_batch)
from .commit import commit_kv, slot_of
from . import quadratic

__all__ = [
    "prepare_block", "prepare_tree", "tree_depths", "quadratic", "BIDIR", "CAUSAL", "MIXED", "TREE", "visible", "block_attn_rows",
    "block_attn_dense", "attn_row", "unpage_kv", "mask_matrix", "accept_request", "accept_batch",
    "greedy_accept_request", "argmax_lowest", "tree_accept_request", "tree_children",
    "sampling_filter", "rank_order", "accept_logits_request", "accept_logits_batch",
    "commit_kv", "slot_of",
]
