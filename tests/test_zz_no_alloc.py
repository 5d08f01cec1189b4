"""The allocation-free accept (spec_accept_static) against spec_accept,
through the C ABI: identical outputs, bit for bit, on two calls in a row (the
second smaller, so the shared scratch holds the first call's contents), in
the stochastic and the greedy form. Run in a fresh process and after the
other GPU tests."""
import numpy as np
import pytest
import torch

import verify_attention_amd as va
from verify_attention_amd import synth
from _support import print_case, to_dev

pytestmark = pytest.mark.gpu

KEYS = ("accept_len", "commit_len", "bonus", "out_tokens", "new_seq_lens")


def _inputs(cid, bs, seed, **over):
    cfg = synth.config(cid, bs=bs, **over)
    x = synth.make_accept_inputs(cfg, seed=seed)
    seq = synth.context_lengths(cfg, seed)
    return x, seq


@pytest.mark.parametrize("greedy", [False, True])
def test_static_accept_equals_workspace_accept(gpu_lib, greedy):
    cases = [(2, 32, 5, {}), (1, 9, 6, dict(vocab=3001, k_spec=11))]  # second call smaller
    for cid, bs, seed, over in cases:
        print_case("spec_accept_static", "greedy" if greedy else "stochastic", cid, bs, over)
        x, seq = _inputs(cid, bs, seed, **over)
        p, q, d, u, s = (to_dev(a) for a in (x.p, x.q, x.draft, x.u, seq))
        e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
        e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
        ref = va.accept(p, q, d, u, s, greedy=greedy, err=e1)
        got = va.accept_static(p, q, d, u, s, greedy=greedy, err=e2)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(got[k], ref[k]), (cid, k)
        assert int(e1.item()) == int(e2.item())
        assert (ref["accept_len"] > 0).any() or greedy


def test_static_accept_rejects_sizes_beyond_its_scratch(gpu_lib):
    print_case("spec_accept_static limit")
    bs, K, V = 1024, 15, 151936
    assert va.accept_workspace_bytes(bs, K, V) > va.ACCEPT_STATIC_SCRATCH_BYTES
    lib = va.load()
    fake = torch.zeros(16, dtype=torch.int32, device="cuda")
    ptr = fake.data_ptr()
    st = lib.spec_accept_static(bs, K, V, 0, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                                None, None)
    assert st == va.SPEC_ESCRATCH        # checked on the host, nothing launched
