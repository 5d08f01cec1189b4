"""The quadratic layout's hand-off between rounds (reference form).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed: "From DFlash to dLLM Self-Spec (4)", section 4.4.1 (the
paragraph comparing recursive compaction with Quadratic Decoding): the layout
inserts a quadratic number of MASK tokens among the speculative tokens, so
that when a speculative position fails verification, the MASK branch after
the last accepted position still supplies the speculative tokens of the next
step; "Unlocking Lossless Speedups in LLMs via Discrete Diffusion",
limitations (4) and future work (2): with this layout, draft and verify merge
into one forward.

Readings where the pages are silent (the layout's shape only is given):
* The block of k drafts has n = (k + 1)^2 positions: the spine (the root,
  then drafts s_1 .. s_k) at block positions i * (k + 1), and after spine
  token j a group G_j of k MASK positions j * (k + 1) + 1 + m (m = 0 .. k-1).
* Spine token j's own row predicts the token right after it (the target's
  next-token view, which the accept uses); member m of G_j occupies the m-th
  position after spine token j + 1 and proposes the token one further on, so
  when exactly s_1 .. s_a are accepted, the correction (bonus) takes position
  L + a + 1 and G_a's k members propose the k tokens after it: the next
  round's drafts.
* The drafts are the greedy choice (lowest index among equal maxima, NaN
  never wins) of each member row's logits, as the DFlash draft pass takes its
  drafts.
* After the accept, the spine's accepted tokens move to contiguous positions
  (the committed-prefix rule of oracle.commit with path p_i = i * (k + 1)).
"""
import numpy as np

from .accept import argmax_lowest


def spine_path(k):
    """Block positions of the spine drafts s_1 .. s_k: p_i = i * (k + 1)."""
    return [i * (k + 1) for i in range(1, k + 1)]


def group_rows(k, j):
    """Block positions of the members of group G_j, in member order."""
    return [j * (k + 1) + 1 + m for m in range(k)]


def handoff(logits, accept_len, k, bonus, mask_token_id):
    """The next round from one request's quadratic block.

    logits [n, V]: the rows of the n = (k + 1)^2 block positions. accept_len:
    drafts accepted by this round's accept (0 .. k); bonus: its correction
    token. Returns (next_draft [k], next_block [n]): next_draft[m] = the
    greedy token of member m of G_accept_len; next_block = the next round's
    quadratic block tokens (position 0: the bonus, its root; spine position
    (m + 1) * (k + 1): next_draft[m]; every group position: the mask token).
    An accept_len outside 0 .. k gives drafts of -1 (and no block)."""
    n = (k + 1) * (k + 1)
    if logits.shape[0] != n:
        raise ValueError("logits must hold the (k + 1)^2 block rows")
    a = int(accept_len)
    if not 0 <= a <= k:
        return np.full(k, -1, np.int64), None
    nxt = np.array([argmax_lowest(logits[r]) for r in group_rows(k, a)], np.int64)
    block = np.full(n, mask_token_id, np.int64)
    block[0] = bonus
    for m, p in enumerate(spine_path(k)):
        block[p] = nxt[m]
    return nxt, block
