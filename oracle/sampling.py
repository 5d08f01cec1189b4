"""Sampling parameters in front of the accept (reference form, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed:

* "Unlocking Lossless Speedups in LLMs via Discrete Diffusion", reproduction
  section: the evaluation samples with temperature 1, top-p 0.95 and top-k
  50. The lossless rule keeps the output distribution equal to the target's,
  so with sampling parameters the target is the processed distribution of the
  verifier's logits, and the draft distribution is the processed
  distribution of the drafter's logits.
* "From DFlash to dLLM Self-Spec (4)", section 4.3.1: the I-DLM verify
  consumes the logits (gather, softmax / top-k, correction); p and q are
  the probabilities of the speculative token under the two views.

Readings where the pages are silent (the plainest ones, as common serving
stacks apply them):
* One row of logits l [V] becomes a distribution in this order:
  1. rank the tokens by logit, largest first; among equal logits (-0 and
     +0 are equal) the lower index ranks first; NaN logits are never kept;
  2. top-k: keep the first top_k ranks;
  3. temperature: e_r = exp((l_r - l_max) / T) over the kept ranks (float64),
     P_r = e_r / sum e;
  4. top-p: keep rank r iff sum_{s < r} P_s < top_p, i.e. the shortest
     prefix of ranks whose mass reaches top_p; top_p >= 1 keeps every rank
     (no nucleus truncation, rather than a decision left to rounding);
  5. p(v) = e_v / sum_{kept} e for every kept v, 0 elsewhere.
* Every target row and every draft row is processed with the same
  parameters, then the linear accept rule (oracle.accept.accept_request) runs
  on the processed rows: tests u_i * q_i(d_i) < p_i(d_i), residual
  max(p_j - q_j, 0) or the processed bonus row, drawn in vocabulary order.
* A top-p decision whose prefix mass lies within 1e-9 of top_p is a tie: a
  request that uses such a row is excluded from bit-exact comparisons, like
  the accept and sampling ties of accept_request.
* Two correct evaluations of a processed row agree to PROB_REL_ERR relative
  per probability (exponentials and sums in float64, in different orders),
  so the residual entries of the two sides differ by at most
  PROB_REL_ERR * (p + q) each, 2 * PROB_REL_ERR in total; the draw's tie band
  widens by that (accept.sample_tie_band's resid_abs_err).
"""
import math

import numpy as np

from .accept import accept_request

TOPP_TIE_EPS = 1e-9
PROB_REL_ERR = 1e-12


def rank_order(logits):
    """Token ids by logit, largest first, lower index first among equal
    logits (-0 and +0 are equal); NaN logits are left out. A stable library
    sort on (-logit, id)."""
    l = np.asarray(logits, np.float64)
    ids = np.flatnonzero(~np.isnan(l))
    return [int(v) for v in ids[np.lexsort((ids, -l[ids]))]]


def mass_before(e, r, z_k):
    """Mass of ranks 0 .. r-1 relative to the top-k normaliser (step 4)."""
    return math.fsum(e[:r]) / z_k


def sampling_filter(logits, temperature, top_k, top_p):
    """Processed distribution of one row of logits (steps 1-5 above).

    Returns (p [V] float64, kept ids in rank order, tie)."""
    V = len(logits)
    ranked = rank_order(logits)[:top_k]
    if not ranked or not math.isfinite(float(logits[ranked[0]])):
        raise ValueError("a row needs at least one finite logit")
    l_max = np.float64(logits[ranked[0]])
    e = [np.exp((np.float64(logits[v]) - l_max) / np.float64(temperature)) for v in ranked]
    z_k = math.fsum(e)
    kept, tie = [], False
    for r in range(len(ranked)):
        if top_p >= 1.0:  # top-p 1 means no nucleus truncation
            kept.append(r)
            continue
        before = mass_before(e, r, z_k)
        if abs(before - top_p) < TOPP_TIE_EPS:
            tie = True
        if not before < top_p:
            break
        kept.append(r)
    z_s = math.fsum(e[r] for r in kept)
    p = np.zeros(V, np.float64)
    for r in kept:
        p[ranked[r]] = e[r] / z_s
    return p, [ranked[r] for r in kept], tie


def accept_logits_request(target_logits, draft_logits, draft, u, seq_len, temperature, top_k,
                          top_p):
    """One request of the logits-input accept. target_logits [K+1, V],
    draft_logits [K, V], draft [K], u [K+1].

    Returns accept_request's dict on the processed rows; tie also covers a
    top-p tie in any row the accept used (rows 0..accept_len of the draft and
    target, and the target's bonus row when every draft was accepted)."""
    K = len(draft)
    p, tp = zip(*[sampling_filter(target_logits[i], temperature, top_k, top_p)[::2]
                  for i in range(K + 1)])
    q, tq = zip(*[sampling_filter(draft_logits[i], temperature, top_k, top_p)[::2]
                  for i in range(K)])
    res = accept_request(np.stack(p), np.stack(q), draft, u, seq_len,
                         resid_abs_err=2.0 * PROB_REL_ERR)
    j = res["accept_len"]
    used = any(tp[: j + 1]) or any(tq[: min(j + 1, K)])
    res["tie_topp"] = bool(used)
    res["tie"] = res["tie"] or bool(used)
    return res


def accept_logits_batch(target_logits, draft_logits, draft, u, seq_lens, temperature, top_k,
                        top_p, requests=None):
    """Every request (or the listed ones); stacked outputs and tie flags."""
    bs = draft.shape[0]
    reqs = range(bs) if requests is None else requests
    keys = ("accept_len", "commit_len", "bonus", "out_tokens", "new_seq_len", "err", "tie",
            "tie_accept", "tie_sample", "tie_topp")
    res = {k: [] for k in keys}
    for b in reqs:
        r = accept_logits_request(target_logits[b], draft_logits[b], draft[b], u[b],
                                  seq_lens[b], temperature, top_k, top_p)
        for k in keys:
            res[k].append(r[k])
    return {k: np.array(v) for k, v in res.items()}
