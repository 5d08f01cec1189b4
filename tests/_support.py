"""Helpers shared by the GPU tests: upload seeded synthetic inputs and
compare against the float64 CPU reference."""
import numpy as np
import torch

from verify_attention_amd import synth


def to_dev(a, dev="cuda"):
    """numpy -> torch on the GPU; uint16 arrays hold bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_f64(t):
    """torch (bf16 / fp32) -> exact float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


class AttnCase:
    """Device copies of one attention workload."""

    def __init__(self, x: synth.AttnInputs, dev="cuda"):
        self.x = x
        self.q = to_dev(x.q, dev)
        self.k = to_dev(x.k_pool, dev)
        self.v = to_dev(x.v_pool, dev)
        self.table = to_dev(x.page_table, dev)
        self.seq = to_dev(x.seq_lens, dev)
        self.nc = to_dev(x.n_causal, dev)
        self.max_kv = int(x.seq_lens.max()) + x.cfg.block


def print_case(*parts):
    print("CASE", *parts, flush=True)


# Share of a test's requests that may be left out of a bit-exact comparison
# as ties (a decision within the tie band of its threshold, where two correct
# float64 evaluations may differ).
MAX_TIE_SHARE = 0.01


def check_tie_share(n_excluded, n, what=""):
    """Report the tie count and fail if more than 1 % of the requests were
    left out of the bit-exact comparison."""
    print(f"TIES {what}: {n_excluded} of {n} requests excluded", flush=True)
    assert n_excluded <= MAX_TIE_SHARE * n, (
        f"{n_excluded} of {n} requests excluded as ties (more than {MAX_TIE_SHARE:.0%})")
