"""GPU parity of the sampling-parameter path through the C ABI:
spec_sampling_filter against the float64 processed rows of the CPU reference
(kept ids in rank order bit-exact, probabilities to 1e-12 relative; rows with
a top-p decision within 1e-9 of top_p are counted and excluded), and
spec_accept_logits against the reference accept on processed rows (every
output bit-exact for requests without a tie)."""
import numpy as np
import pytest
import torch

import oracle
import verify_attention_amd as va
from verify_attention_amd import synth
from _support import check_tie_share, print_case, to_dev

pytestmark = pytest.mark.gpu


def _values(a):
    """Exact float32 values of stored logits (bf16 bits or float32)."""
    return synth.bf16_to_f32(a) if a.dtype == np.uint16 else a


def _f32(x):
    """temperature and top_p cross the C ABI as float32: the reference takes
    the same float32 values."""
    return float(np.float32(x))


def run_filter(logits, T, k, top_p):
    got = va.sampling_filter(to_dev(logits), T, k, top_p)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in got.items()}


def check_filter(logits, got, T, k, top_p):
    vals = _values(logits)
    ties = 0
    for r in range(vals.shape[0]):
        p, kept, tie = oracle.sampling_filter(vals[r], _f32(T), k, _f32(top_p))
        if tie:
            ties += 1
            continue
        n = int(got["n_kept"][r])
        assert n == len(kept), (r, n, len(kept))
        assert list(got["kept_ids"][r, :n]) == kept, r
        assert (got["kept_ids"][r, n:] == -1).all() and (got["kept_probs"][r, n:] == 0).all()
        np.testing.assert_allclose(got["kept_probs"][r, :n], p[kept], rtol=oracle.sampling.PROB_REL_ERR, atol=0)
    print(f"filter rows {vals.shape[0]}: top-p ties excluded {ties}", flush=True)
    return ties


PARAMS = [(1.0, 50, 0.95), (0.7, 64, 0.9), (1.3, 1, 0.5), (1.0, 20, 1.0), (2.0, 37, 0.99)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [524288, 151936, 5003, 64, 30])
def test_filter_matches_reference(V, dtype):
    rng = np.random.default_rng(V)
    rows = 12
    x = (rng.standard_normal((rows, V), dtype=np.float32) * 3).astype(np.float32)
    if dtype == "bf16":
        x = synth.bf16_bits(x)
    for T, k, top_p in PARAMS:
        print_case("sampling_filter", V, dtype, T, k, top_p)
        check_filter(x, run_filter(x, T, k, top_p), T, k, top_p)


def test_filter_ties_nan_and_inf():
    rng = np.random.default_rng(7)
    V = 20000
    x = rng.integers(-40, 8, size=(10, V)).astype(np.float32)   # many equal logits
    x[1, ::97] = np.nan
    x[2, :] = -np.inf
    x[2, 5000:5040] = rng.normal(0, 1, 40).astype(np.float32)     # fewer finite than top_k
    x[3, 100:200] = 7.0                                           # 100 equal maxima
    x[4, ::2] = -0.0
    x[4, 1::2] = 0.0                                              # signed zeros only
    for T, k, top_p in PARAMS:
        print_case("sampling_filter ties", T, k, top_p)
        check_filter(x, run_filter(x, T, k, top_p), T, k, top_p)


@pytest.mark.parametrize("V", [5003, 151936])
def test_filter_constant_rows_take_the_exact_slow_path(V):
    # every tile maximum ties, so the candidates overflow LDS: the exact
    # round-by-round path must still return the lowest indices
    x = np.zeros((3, V), np.float32)
    x[1] = 2.5
    x[2, 4000] = 3.0
    print_case("sampling_filter constant rows", V)
    got = run_filter(x, 1.0, 50, 0.95)
    check_filter(x, got, 1.0, 50, 0.95)
    assert list(got["kept_ids"][0, :3]) == [0, 1, 2]


def run_accept_logits(x, seq, T, k, top_p, err=None):
    out = va.accept_logits(to_dev(x.target), to_dev(x.draft_logits), to_dev(x.draft),
                           to_dev(x.u), to_dev(seq), T, k, top_p, err=err)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in out.items()}


def compare_accept_logits(x, seq, got, T, k, top_p):
    ref = oracle.accept_logits_batch(_values(x.target), _values(x.draft_logits), x.draft, x.u,
                                     seq, _f32(T), k, _f32(top_p))
    same = np.ones(len(seq), bool)
    for kg, kr in (("accept_len", "accept_len"), ("commit_len", "commit_len"),
                   ("bonus", "bonus"), ("new_seq_lens", "new_seq_len"),
                   ("out_tokens", "out_tokens")):
        same &= (got[kg] == ref[kr]).reshape(len(seq), -1).all(-1)
    bad = np.flatnonzero(~same & ~ref["tie"])
    assert len(bad) == 0, f"requests differing without a tie: {bad}"
    print(f"accept_logits: {len(seq)} requests, ties excluded {int(ref['tie'].sum())} "
          f"(accept {int(ref['tie_accept'].sum())}, sampling {int(ref['tie_sample'].sum())}, "
          f"top-p {int(ref['tie_topp'].sum())}), tied that matched {int((same & ref['tie']).sum())}, "
          f"mean accept {ref['accept_len'].mean():.2f}", flush=True)
    check_tie_share(int(ref["tie"].sum()), len(seq), "spec_accept_logits")
    return ref


@pytest.mark.parametrize("dtype,bs", [("f32", None), ("bf16", 8)])
def test_accept_logits_matches_reference(dtype, bs):
    # the logits verify workload (Qwen3-8B-shaped, bs 32, K = 15, V = 151936,
    # temperature 1, top-k 50, top-p 0.95); bf16 logits at bs 8
    cfg = synth.config(7)
    T, k, top_p = cfg.sampling
    print_case("accept_logits", dtype, bs or cfg.bs)
    x = synth.make_logits_accept_inputs(cfg, seed=3, bs=bs, dtype=dtype)
    n = x.draft.shape[0]
    seq = synth.context_lengths(synth.config(7, bs=n), 3)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = run_accept_logits(x, seq, T, k, top_p, err=err)
    compare_accept_logits(x, seq, got, T, k, top_p)
    assert int(err.item()) == 0


@pytest.mark.parametrize("T,k,top_p", [(0.8, 64, 0.9), (1.5, 8, 1.0), (1.0, 1, 0.95)])
def test_accept_logits_other_parameters(T, k, top_p):
    cfg = synth.config(7, bs=6, vocab=20011, k_spec=9)
    print_case("accept_logits params", T, k, top_p)
    x = synth.make_logits_accept_inputs(cfg, seed=4)
    seq = np.arange(6, dtype=np.int32) * 7
    compare_accept_logits(x, seq, run_accept_logits(x, seq, T, k, top_p), T, k, top_p)


def test_accept_logits_error_paths():
    cfg = synth.config(7, bs=4, vocab=3001, k_spec=5)
    print_case("accept_logits error paths")
    x = synth.make_logits_accept_inputs(cfg, seed=5)
    x.draft[0, 0] = cfg.vocab + 2            # invalid id: a reject, flagged
    x.draft_logits[1] = x.target[1, :5]      # q == p on every row of request 1:
    x.draft[1, :2] = [oracle.argmax_lowest(x.target[1, i]) for i in range(2)]  # accepted,
    x.draft[1, 2] = np.argsort(x.target[1, 2])[0]  # then a draft outside both kept sets:
    x.u[1, :2] = 0.5                               # rejected with zero residual
    seq = np.full(4, 100, np.int32)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = run_accept_logits(x, seq, 1.0, 50, 0.95, err=err)
    ref = compare_accept_logits(x, seq, got, 1.0, 50, 0.95)
    e = int(err.item())
    assert e & va.ERR_TOKEN and e & va.ERR_ZERO_RESIDUAL
    assert got["accept_len"][0] == 0 and got["accept_len"][1] == 2
    assert ref["err"][1] & va.ERR_ZERO_RESIDUAL


def test_untruncated_logits_accept_is_the_accept_on_softmax_rows():
    """With nothing truncated (V = top-k = 64, top-p 1, temperature 1) the
    logits accept equals spec_accept fed the softmax rows (float32), request by
    request; ties of either reference are excluded (the two paths round the
    probabilities differently)."""
    rng = np.random.default_rng(101)
    bs, K, V = 48, 7, 64
    print_case("accept_logits untruncated = accept", bs, K, V)
    tl = (rng.standard_normal((bs, K + 1, V)) * 2.0).astype(np.float32)
    dl = (tl[:, :K] + rng.standard_normal((bs, K, V)) * 0.5).astype(np.float32)

    def softmax(a):
        e = np.exp(a.astype(np.float64) - a.max(-1, keepdims=True))
        return e / e.sum(-1, keepdims=True)

    q64 = softmax(dl)
    draft = np.array([[rng.choice(V, p=q64[b, i]) for i in range(K)] for b in range(bs)], np.int32)
    u = rng.random((bs, K + 1), dtype=np.float32)
    seq = rng.integers(1, 900, size=bs).astype(np.int32)
    got_l = va.accept_logits(to_dev(tl), to_dev(dl), to_dev(draft), to_dev(u), to_dev(seq),
                             1.0, V, 1.0)
    p32, q32 = softmax(tl).astype(np.float32), q64.astype(np.float32)
    got_a = va.accept(to_dev(p32), to_dev(q32), to_dev(draft), to_dev(u), to_dev(seq))
    torch.cuda.synchronize()
    ref_l = oracle.accept_logits_batch(tl, dl, draft, u, seq, np.float32(1.0), V, np.float32(1.0))
    ref_a = oracle.accept_batch(p32, q32, draft, u, seq)
    keep = ~(ref_l["tie"] | ref_a["tie"])
    for key in ("accept_len", "commit_len", "bonus", "new_seq_lens", "out_tokens"):
        a, b = got_l[key].cpu().numpy(), got_a[key].cpu().numpy()
        assert np.array_equal(a[keep], b[keep]), key
    check_tie_share(int((~keep).sum()), bs, "untruncated logits accept vs accept")
    assert (ref_a["accept_len"] > 0).any()

