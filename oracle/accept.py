"""Speculative accept / bonus epilogue (reference form, float64).

What is computed:

* "Unlocking Lossless Speedups in LLMs via Discrete Diffusion", prerequisite
  "speculative decoding and rejection sampling" and the Psi-Spec Linear
  sampler: a block of draft tokens is scored by the target in one pass; the
  longest prefix that passes rejection sampling is kept and the rejected slot
  is re-drawn from the residual distribution, which leaves the output
  distribution equal to the target's.
* "From DFlash to dLLM Self-Spec (4)", section 4.3 / 4.3.1 (I-DLM p/q verify):
  q is the draft probability of the speculative token, p the anchor (causal
  view) probability; a token is accepted with probability min(1, p/q), and a
  reject emits a correction from the anchor side.
* "From DFlash to dLLM Self-Spec (2)", section 2.2.5: the greedy rule (accept
  while the draft equals the target's argmax at the previous position; bonus =
  target argmax at the accept length; commit = accept + 1) and the outputs
  accept_len, commit_len, bonus, out_tokens, new_seq_lens.
* "From DFlash to dLLM Self-Spec (4)", section 4.4.1 (LinearSpec verify):
  count matching positions, add one, crop the cache to length + accepted, and
  carry the last emitted token into the next round.
* "Unlocking Lossless Speedups in LLMs via Discrete Diffusion", method steps
  (the Tree sampler: top candidates per position kept as a tree of prefixes,
  verified in parallel, losslessness from rejection sampling):
  tree_accept_request walks the tree from the root with the recursive
  rejection rule for deterministic candidates (see its docstring).

Readings where the pages are silent:
* Row alignment: target row i (0-based, i = 0..K) scores block token i+1, so
  test i uses p[i, d_i], q[i, d_i] with d_i = draft[i]; row K is the bonus row.
* The test is u_i * q < p in float64 (exact for float32 inputs), which is
  u_i < min(1, p/q) without a division; p = 0 is never accepted.
* u[0..K-1] drive the tests, u[K] drives the one final draw.
* Residual r = max(p_j - q_j, 0) (float64, one rounding per entry) after a
  reject at j, else r = p_K; S = sum r; the token is the smallest t with
  C_t > u_K * S (C = running sum in vocabulary order). If S <= 0 the draw
  falls back to p_j and flags it; if rounding leaves no C_t above the
  threshold the last index with r > 0 is taken; a row with no positive entry
  at all (not a distribution) yields token 0.
"""
import numpy as np

ERR_TOKEN = 4          # a draft token id is outside [0, V)
ERR_ZERO_RESIDUAL = 8  # residual mass was zero; the draw used p_j instead
TIE_EPS = 1e-6         # accept-test ties: |u - min(1, p/q)| below this


def sample_tie_band(V, S, resid_abs_err=0.0):
    """Half-width of the band around the draw's threshold inside which two
    correct float64 evaluations of the inverse CDF may pick different tokens.

    Both sides hold the same float64 residual entries (each is a float32
    value, or the difference of two float32 values, rounded once, a
    deterministic operation) and differ only in the order of their sums. A
    running sum of n non-negative terms is within (n - 1) * 2^-53 * S of its
    exact value (first-order bound; S = the total), this reference's running
    sum has n <= V, and a summation tree or scan of depth below 256 (the
    kernels' sub-block sums and scans) stays within 256 * 2^-53 * S. The
    threshold u * S moves with S and adds one rounding. Together the running
    sum at the chosen boundary and the threshold differ between the two
    sides by at most (2V + 512) * 2^-53 * S = (V + 256) * 2^-52 * S.
    resid_abs_err bounds sum_v |r_v - r'_v| when the two sides compute the
    residual entries themselves (the logits accept); it moves both the
    running sum and S, so it counts twice."""
    return (V + 256) * 2.0 ** -52 * S + 2.0 * resid_abs_err


def draw_is_tie(thr, C, t, band):
    """Whether the draw's threshold thr lies strictly inside the tie band of
    an end of the chosen token's interval (C[t-1], C[t]]. A zero threshold
    (u = 0) is not a tie: it is exactly 0 on both sides and every running sum
    before the first entry with mass is a sum of zeros, exact in any order,
    so both pick the first entry with mass."""
    if thr == 0.0:
        return False
    lo = C[t - 1] if t > 0 else 0.0
    return bool(abs(thr - C[t]) < band or abs(thr - lo) < band)


def argmax_lowest(x):
    """Index of the maximum; the lowest index wins among equal maxima; NaN
    never wins (a row without a non-NaN entry gives 0)."""
    x = np.asarray(x)
    ok = ~np.isnan(x)
    if not ok.any():
        return 0
    m = x[ok].max()
    return int(np.flatnonzero(x == m)[0])


def _inverse_cdf(r, u):
    """Smallest t with C_t > u * S, C the running sum of r. Returns
    (t, S, thr, C) with a fallback to the last positive entry (token 0 when
    the row holds no positive entry at all)."""
    C = np.cumsum(r)
    S = C[-1]
    thr = np.float64(u) * S
    t = int(np.searchsorted(C, thr, side="right"))
    if t >= len(r):
        pos = np.flatnonzero(r > 0)
        t = int(pos[-1]) if len(pos) else 0
    return t, S, thr, C


def accept_request(p, q, draft, u, seq_len, resid_abs_err=0.0):
    """One request. p [K+1, V], q [K, V] float32 rows; draft [K]; u [K+1].

    Returns a dict with accept_len, commit_len, bonus, out_tokens [K+1]
    (accepted drafts, then the bonus, then -1), new_seq_len, err, and the
    tie flags: tie_accept when a reached test has |u - min(1, p/q)| < 1e-6,
    tie_sample when u_K * S lies within sample_tie_band(V, S, resid_abs_err)
    of the chosen token's interval ends (draw_is_tie), tie = either."""
    K, V = q.shape
    err = 0
    tie_accept = False
    n_acc = 0
    for i in range(K):
        d = int(draft[i])
        if d < 0 or d >= V:
            err |= ERR_TOKEN
            break
        pd = np.float64(p[i, d])
        qd = np.float64(q[i, d])
        ui = np.float64(u[i])
        if qd > 0 and abs(ui - min(1.0, pd / qd)) < TIE_EPS:
            tie_accept = True
        if ui * qd < pd:
            n_acc += 1
        else:
            break
    j = n_acc
    if j < K:
        r = np.maximum(p[j].astype(np.float64) - q[j].astype(np.float64), 0.0)
    else:
        r = p[K].astype(np.float64)
    if not r.sum() > 0:
        err |= ERR_ZERO_RESIDUAL
        r = p[j].astype(np.float64)
    t, S, thr, C = _inverse_cdf(r, u[K])
    tie_sample = draw_is_tie(thr, C, t, sample_tie_band(V, S, resid_abs_err))
    out = np.full(K + 1, -1, np.int64)
    out[:n_acc] = draft[:n_acc]
    out[n_acc] = t
    return dict(accept_len=n_acc, commit_len=n_acc + 1, bonus=t, out_tokens=out,
                new_seq_len=int(seq_len) + n_acc + 1, err=err, tie=tie_accept or tie_sample,
                tie_accept=tie_accept, tie_sample=tie_sample)


def greedy_accept_request(p, draft, seq_len):
    """Greedy special case: accept while draft[i] == argmax p[i]; the bonus is
    argmax p[accept_len]; commit = accept_len + 1."""
    K = len(draft)
    n_acc = 0
    while n_acc < K and int(draft[n_acc]) == argmax_lowest(p[n_acc]):
        n_acc += 1
    bonus = argmax_lowest(p[n_acc])
    out = np.full(K + 1, -1, np.int64)
    out[:n_acc] = draft[:n_acc]
    out[n_acc] = bonus
    return dict(accept_len=n_acc, commit_len=n_acc + 1, bonus=bonus, out_tokens=out,
                new_seq_len=int(seq_len) + n_acc + 1, err=0, tie=False, tie_accept=False,
                tie_sample=False)


ERR_TREE = 16  # a node's parent is not an earlier node (the node is ignored)


def tree_children(parent, x):
    """Children of node x in increasing node order (nodes whose parent is x;
    a node n is only a child when 0 <= parent[n] < n)."""
    return [n for n in range(1, len(parent)) if int(parent[n]) == x and 0 <= x < n]


def tree_accept_request(parent, token, p, u, seq_len):
    """Tree verification of one request by recursive rejection sampling.

    The tree's candidates are deterministic (top candidates), so each child
    is a draft with a one-hot draft distribution: at node x (starting at the
    root, node 0) the children c are tried in increasing node order; with T
    the target mass p_x of the distinct tokens already tried at x, child c is
    accepted iff u[c] * (1 - T) < p_x(token[c]) (the probability p_x(t) / (1 -
    T) of the normalised residual; a token already tried has residual 0, an
    id outside [0, V) is a reject and is flagged). An accepted child becomes
    the next node. When no child of x is accepted (or x is a leaf) the bonus
    is drawn from r = p_x with the tried tokens set to 0: the smallest t with
    C_t > u[0] * S, C the running sum of r in vocabulary order, S = sum r
    (S <= 0: drawn from p_x itself and flagged).

    parent [N] (parent[0] = -1), token [N] (token[0], the root, is not read),
    p [N, V] float32 (row n: the target distribution of the token after
    node n's path), u [N] float32. Returns accept_len (accepted nodes),
    path_nodes [N] (accepted node ids, then -1), out_tokens [N] (their
    tokens, then the bonus, then -1), bonus, commit_len, new_seq_len, err and
    tie flags as accept_request (tie_accept: a test with |u - p/(1 - T)| <
    1e-6, T being a sum whose order may differ; tie_sample: the final
    threshold within sample_tie_band(V, S) of an interval end).
    """
    N, V = p.shape
    err = 0
    for n in range(1, N):
        if not 0 <= int(parent[n]) < n:
            err |= ERR_TREE
    path = []
    tie_accept = False
    x = 0
    while True:
        tried = []
        nxt = -1
        T = np.float64(0.0)
        for c in tree_children(parent, x):
            d = int(token[c])
            if d < 0 or d >= V:
                err |= ERR_TOKEN
                continue
            pr = np.float64(0.0) if d in tried else np.float64(p[x, d])
            uc = np.float64(u[c])
            if 1.0 - T > 0 and abs(uc - pr / (1.0 - T)) < TIE_EPS:
                tie_accept = True
            if uc * (1.0 - T) < pr:
                nxt = c
                break
            if d not in tried:
                tried.append(d)
                T += pr
        if nxt < 0:
            break
        path.append(nxt)
        x = nxt
    r = p[x].astype(np.float64)
    for d in tried:
        r[d] = 0.0
    if not r.sum() > 0:
        err |= ERR_ZERO_RESIDUAL
        r = p[x].astype(np.float64)
    t, S, thr, C = _inverse_cdf(r, u[0])
    tie_sample = draw_is_tie(thr, C, t, sample_tie_band(V, S))
    k = len(path)
    nodes = np.full(N, -1, np.int64)
    nodes[:k] = path
    out = np.full(N, -1, np.int64)
    out[:k] = [int(token[c]) for c in path]
    out[k] = t
    return dict(accept_len=k, commit_len=k + 1, bonus=t, out_tokens=out, path_nodes=nodes,
                new_seq_len=int(seq_len) + k + 1, err=err, tie=tie_accept or tie_sample,
                tie_accept=tie_accept, tie_sample=tie_sample)


def accept_batch(p, q, draft, u, seq_lens, greedy=False, requests=None):
    """Every request (or the listed ones) of a batch; returns stacked arrays
    plus the per-request tie flags."""
    bs, K = draft.shape
    reqs = range(bs) if requests is None else requests
    res = dict(accept_len=[], commit_len=[], bonus=[], out_tokens=[], new_seq_len=[],
               err=[], tie=[], tie_accept=[], tie_sample=[])
    for b in reqs:
        if greedy:
            r = greedy_accept_request(p[b], draft[b], seq_lens[b])
        else:
            r = accept_request(p[b], q[b], draft[b], u[b], seq_lens[b])
        for key in res:
            res[key].append(r[key])
    return {k: np.array(v) for k, v in res.items()}
