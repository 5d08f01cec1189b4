"""The bench's host logic (CPU only): the one-GPU contract and the algorithmic
byte and flop counts its roofline divides by, checked against counts written
out by hand for small shapes."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from verify_attention_amd import synth  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr


def test_attention_bytes_and_flops_by_hand():
    cfg = synth.config(2, bs=2, block=4, hq=4, hkv=2, d=8, ctx_lo=3, ctx_hi=3)
    seq = np.array([3, 5])
    kv_bytes = 2 * ((3 + 4) + (5 + 4)) * 2 * 8 * 2      # K and V, 2 KV heads, D 8, bf16
    qo_bytes = 2 * 2 * 4 * 4 * 8 * 2                    # Q read + O written
    # CAUSAL: row i sees L keys of context and i + 1 block keys
    pairs = sum(L * 4 + (1 + 2 + 3 + 4) for L in (3, 5))
    b, f = bench.attn_alg_bytes_flops(cfg, seq)
    assert b == kv_bytes + qo_bytes
    assert f == 4 * 8 * pairs * 4
    # BIDIR and MIXED (2 clean rows, then rows that see the whole block)
    cb = synth.config(2, bs=2, block=4, hq=4, hkv=2, d=8, modes=(synth.BIDIR,))
    assert bench.attn_alg_bytes_flops(cb, seq)[1] == 4 * 8 * sum(L * 4 + 16 for L in (3, 5)) * 4
    cm = synth.config(2, bs=2, block=4, hq=4, hkv=2, d=8, modes=(synth.MIXED,), n_causal=2)
    assert bench.attn_alg_bytes_flops(cm, seq)[1] == 4 * 8 * sum(L * 4 + (1 + 2 + 4 + 4)
                                                                   for L in (3, 5)) * 4
    # TREE: the set bits of the row masks
    ct = synth.config(2, bs=2, block=4, hq=4, hkv=2, d=8, modes=(synth.TREE,))
    masks = np.array([0b1, 0b11, 0b101, 0b1011], dtype=np.uint64)
    assert bench.attn_alg_bytes_flops(ct, seq, masks)[1] == \
        4 * 8 * sum(L * 4 + 1 + 2 + 2 + 3 for L in (3, 5)) * 4
    # trees past 64 nodes: mask words per row ([bs, B, W]); a 70-node chain
    # per request sees 1 + 2 + ... + 70 block pairs
    cw = synth.config(2, bs=2, block=70, hq=4, hkv=2, d=8, modes=(synth.TREE,))
    chain = synth.tree_row_words(np.arange(-1, 69, dtype=np.int32))
    words = np.stack([chain, chain])
    assert words.shape == (2, 70, 2)
    assert bench.attn_alg_bytes_flops(cw, seq, words)[1] == \
        4 * 8 * sum(L * 70 + 70 * 71 // 2 for L in (3, 5)) * 4


def test_accept_bytes_by_hand():
    cfg = synth.config(2, bs=3, vocab=100, k_spec=5)
    al = np.array([0, 5, 2])         # the all-accepted request streams the bonus row only
    assert bench.accept_alg_bytes(cfg, al) == (2 + 1 + 2) * 100 * 4 + 3 * (2 * 5 + 1) * 4
    assert bench.logits_accept_alg_bytes(cfg) == 3 * 11 * 100 * 4
    assert bench.tree_accept_alg_bytes(synth.config(6, bs=2, vocab=100, block=8)) == \
        2 * (100 + 8) * 4


def test_traffic_table_matches_its_sources():
    t = bench.measured_traffic("qwen3_8b_verify_bs32", "not-these-sources")
    assert t is None
    import json
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(path):
        tj = json.load(open(path))
        for key, w in tj["workloads"].items():
            name, _, call = key.partition("/")
            got = bench.measured_traffic(name, tj["kernel_src"], call or "block_attn")
            assert got == int(w["traffic_bytes"])


def test_cpu_leg_sample_inputs_keep_each_requests_attention():
    """The CPU leg runs the reference on one request at a time over a pool
    holding only that request's pages (page table renumbered): the result
    must equal the reference on the whole batch for that request, bit for
    bit, whatever the page shuffle."""
    import oracle
    cfg = synth.config(4, bs=5, hq=4, hkv=2, d=16, ctx_lo=20, ctx_hi=90)
    x = synth.make_attn_inputs(cfg, seed=3)
    mode = cfg.modes[-1]
    full, _ = oracle.block_attn_dense(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                      x.page_table, x.seq_lens, mode, cfg.n_causal)
    for b in (0, 3, 4):
        one = bench._sample_inputs(x, [b])
        assert one.num_pages < x.num_pages
        assert np.all(one.page_table[0][one.page_table[0] >= 0] < one.num_pages)
        got, _ = oracle.block_attn_dense(one.as_f64("q"), one.as_f64("k_pool"),
                                         one.as_f64("v_pool"), one.page_table, one.seq_lens,
                                         mode, cfg.n_causal)
        assert np.array_equal(got[0], full[b]), b


def test_cpu_leg_counts_a_planted_mismatch():
    """The bench line's parity sample is not vacuous: GPU outputs equal to
    the reference give no mismatch; one request's bonus or attention row
    changed gives exactly one."""
    import oracle
    cfg = synth.config(1, bs=3)
    x = synth.make_attn_inputs(cfg, seed=4)
    acc = synth.make_accept_inputs(cfg, seed=4)
    ro, _ = oracle.block_attn_dense(x.as_f64("q"), x.as_f64("k_pool"), x.as_f64("v_pool"),
                                    x.page_table, x.seq_lens, cfg.modes[-1], cfg.n_causal)
    ra = oracle.accept_batch(acc.p, acc.q, acc.draft, acc.u, x.seq_lens)

    def gpu(bad_bonus=None, bad_attn=None):
        def o(b):
            return ro[b] + (0.5 if b == bad_attn else 0.0)

        def accept(b):
            return dict(accept_len=ra["accept_len"][b],
                        bonus=ra["bonus"][b] + (1 if b == bad_bonus else 0),
                        new_seq_lens=ra["new_seq_len"][b], out_tokens=ra["out_tokens"][b])
        return {"o": o, "accept": accept}

    for g, want in ((gpu(), 0), (gpu(bad_bonus=1), 1), (gpu(bad_attn=2), 1)):
        r = bench.cpu_baseline(cfg, x, 60.0, g, acc=acc)
        ps = r["parity_sample"]
        assert ps["requests"] == cfg.bs and ps["sampling_ties"] == 0
        assert ps["mismatched_requests"] == want, (want, ps)
