"""CPU checks of the C ABI: the library loads, exports exactly the functions
include/specattn.h declares, and rejects bad arguments on the host before
any launch (no compute calls here; this container has no GPU)."""
import ctypes
import os
import subprocess

import pytest

import verify_attention_amd as va
from verify_attention_amd import binding as b

FAKE = ctypes.c_void_p(4096)  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(b.lib_path()):
        from verify_attention_amd import build
        build.build()
    return va.load()


def test_exports_match_header(lib):
    declared = set(b.header_functions())
    out = subprocess.run(["nm", "-D", "--defined-only", b.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[2] for ln in out.splitlines() if len(ln.split()) == 3 and ln.split()[1] == "T"}
    assert exported == declared
    for name in declared:
        assert getattr(lib, name) is not None


def test_version_and_status_strings(lib):
    assert lib.spec_version() == 100
    for s in (0, -1, -2, -3, -4):
        assert len(lib.spec_status_string(s)) > 0
    assert lib.spec_status_string(-99) == b"unknown status"


def _prep(lib, **kw):
    args = dict(bs=2, B=4, P=16, max_pages=4, num_pages=8, mask=0, vid=FAKE, seq=FAKE, tab=FAKE,
                draft=None, ids=FAKE, pos=FAKE, loc=FAKE, err=None)
    args.update(kw)
    return lib.spec_prepare_block(args["bs"], args["B"], args["P"], args["max_pages"],
                                  args["num_pages"], args["mask"], args["vid"], args["seq"],
                                  args["tab"], args["draft"], args["ids"], args["pos"],
                                  args["loc"], args["err"], None)


def test_prepare_block_rejects_bad_arguments(lib):
    assert _prep(lib, bs=0) == b.SPEC_EINVAL
    assert _prep(lib, B=0) == b.SPEC_EINVAL
    assert _prep(lib, P=0) == b.SPEC_EINVAL
    assert _prep(lib, max_pages=0) == b.SPEC_EINVAL
    assert _prep(lib, num_pages=0) == b.SPEC_EINVAL
    assert _prep(lib, vid=None) == b.SPEC_EINVAL
    assert _prep(lib, loc=None) == b.SPEC_EINVAL


def _attn(lib, **kw):
    a = dict(mode=1, nc=0, ncr=None, dt=1, bs=2, B=16, hq=32, hkv=8, d=128, P=16, max_pages=80,
             num_pages=200, max_kv=1040, q=FAKE, k=FAKE, v=FAKE, tab=FAKE, seq=FAKE, scale=0.0,
             o=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30, err=None)
    a.update(kw)
    return lib.block_attn(a["mode"], a["nc"], a["ncr"], a["dt"], a["bs"], a["B"], a["hq"],
                          a["hkv"], a["d"], a["P"], a["max_pages"], a["num_pages"], a["max_kv"],
                          a["q"], a["k"], a["v"], a["tab"], a["seq"], a["scale"], a["o"],
                          a["lse"], a["ws"], a["ws_bytes"], a["err"], None)


def test_block_attn_rejects_bad_arguments(lib):
    assert _attn(lib, d=96) == b.SPEC_ENOTSUP
    assert _attn(lib, P=8) == b.SPEC_ENOTSUP
    assert _attn(lib, dt=7) == b.SPEC_ENOTSUP
    assert _attn(lib, mode=3) == b.SPEC_EINVAL
    assert _attn(lib, hq=30) == b.SPEC_EINVAL           # Hq % Hkv != 0
    assert _attn(lib, B=513, max_pages=200) == b.SPEC_EINVAL  # g * B = 2052 > 2048
    assert _attn(lib, bs=0) == b.SPEC_EINVAL
    assert _attn(lib, max_pages=0) == b.SPEC_EINVAL
    assert _attn(lib, mode=2, nc=17) == b.SPEC_EINVAL   # n_causal > B
    assert _attn(lib, mode=2, nc=-1) == b.SPEC_EINVAL
    assert _attn(lib, q=None) == b.SPEC_EINVAL
    assert _attn(lib, o=None) == b.SPEC_EINVAL
    assert _attn(lib, scale=float("nan")) == b.SPEC_EINVAL
    assert _attn(lib, max_pages=1, B=32, hq=8, hkv=8) == b.SPEC_EINVAL  # table shorter than B


def test_block_attn_tree_rejects_bad_arguments(lib):
    def tree(**kw):
        a = dict(tm=FAKE, per=1, dt=1, bs=2, B=32, hq=8, hkv=2, d=128, P=16, max_pages=80,
                 num_pages=200, max_kv=1040, q=FAKE, k=FAKE, v=FAKE, tab=FAKE, seq=FAKE,
                 scale=0.0, o=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 30, err=None)
        a.update(kw)
        return lib.block_attn_tree(a["tm"], a["per"], a["dt"], a["bs"], a["B"], a["hq"], a["hkv"],
                                   a["d"], a["P"], a["max_pages"], a["num_pages"], a["max_kv"],
                                   a["q"], a["k"], a["v"], a["tab"], a["seq"], a["scale"], a["o"],
                                   a["lse"], a["ws"], a["ws_bytes"], a["err"], None)
    assert tree(tm=None) == b.SPEC_EINVAL
    assert tree(B=513, hq=2, hkv=2) == b.SPEC_EINVAL      # more nodes than 8 mask words
    assert tree(B=64, hq=64, hkv=1) == b.SPEC_EINVAL      # g * B = 4096 > 2048
    assert tree(d=96) == b.SPEC_ENOTSUP
    assert tree(q=None) == b.SPEC_EINVAL
    # the mode argument of block_attn itself does not take TREE (no mask pointer)
    assert _attn(lib, mode=3) == b.SPEC_EINVAL


def test_block_attn_workspace_planning(lib):
    # few (request, KV head) units and a long context -> split-KV workspace
    small = lib.block_attn_workspace_bytes(2, 16, 32, 8, 128, 8192)
    assert small > 0
    assert _attn(lib, bs=2, max_kv=8192, ws_bytes=small - 1) == b.SPEC_ENOSPC
    assert _attn(lib, bs=2, max_kv=8192, ws=None, ws_bytes=small) == b.SPEC_ENOSPC
    # enough units to fill the chip, short contexts -> one workgroup per unit,
    # no workspace at all
    assert lib.block_attn_workspace_bytes(32, 16, 32, 8, 128, 1040) == 0
    # large batches take the balanced schedule: two partial slots of M x (D + 2)
    # floats per workgroup (256), whatever the batch size
    bal = 2 * 256 * 64 * (128 + 2) * 4
    assert bal <= lib.block_attn_workspace_bytes(256, 16, 32, 8, 128, 9232) <= bal + 256
    assert lib.block_attn_workspace_bytes(128, 16, 32, 8, 128, 4112) == \
        lib.block_attn_workspace_bytes(256, 16, 32, 8, 128, 9232)
    assert lib.block_attn_workspace_bytes(0, 16, 32, 8, 128, 9232) == 0
    # 512 rows per KV head run as 4 row groups of 128: the plan (and so the
    # workspace) of 4 KV heads x 128 rows equals that of 16 KV heads x 128 rows
    for kv in (8192, 2 ** 18):
        assert lib.block_attn_workspace_bytes(2, 128, 16, 4, 128, kv) == \
            lib.block_attn_workspace_bytes(2, 32, 64, 16, 128, kv) > 0


def _acc(lib, **kw):
    a = dict(bs=4, K=15, V=151936, greedy=0, p=FAKE, q=FAKE, d=FAKE, u=FAKE, seq=FAKE, al=FAKE,
             cl=FAKE, bon=FAKE, out=FAKE, nsl=FAKE, ws=FAKE, ws_bytes=1 << 30, err=None)
    a.update(kw)
    return lib.spec_accept(a["bs"], a["K"], a["V"], a["greedy"], a["p"], a["q"], a["d"], a["u"],
                           a["seq"], a["al"], a["cl"], a["bon"], a["out"], a["nsl"], a["ws"],
                           a["ws_bytes"], a["err"], None)


def test_accept_rejects_bad_arguments(lib):
    assert _acc(lib, bs=0) == b.SPEC_EINVAL
    assert _acc(lib, K=0) == b.SPEC_EINVAL
    assert _acc(lib, K=64) == b.SPEC_EINVAL
    assert _acc(lib, V=0) == b.SPEC_EINVAL
    assert _acc(lib, q=None) == b.SPEC_EINVAL
    assert _acc(lib, u=None) == b.SPEC_EINVAL
    assert _acc(lib, out=None) == b.SPEC_EINVAL
    assert _acc(lib, V=524289) == b.SPEC_ENOTSUP              # stochastic accept vocabulary cap
    need = lib.spec_accept_workspace_bytes(4, 15, 151936, 0)
    assert need > 0
    assert _acc(lib, ws_bytes=need - 1) == b.SPEC_ENOSPC
    assert _acc(lib, ws=None) == b.SPEC_ENOSPC
    assert lib.spec_accept_workspace_bytes(4, 15, 151936, 1) == 4 * 16 * 4


def test_accept_tree_rejects_bad_arguments(lib):
    def acc(**kw):
        a = dict(bs=4, N=32, V=151936, par=FAKE, tok=FAKE, p=FAKE, u=FAKE, seq=FAKE, al=FAKE,
                 cl=FAKE, bon=FAKE, out=FAKE, path=FAKE, nsl=FAKE, ws=FAKE, ws_bytes=1 << 30,
                 err=None)
        a.update(kw)
        return lib.spec_accept_tree(a["bs"], a["N"], a["V"], a["par"], a["tok"], a["p"], a["u"],
                                    a["seq"], a["al"], a["cl"], a["bon"], a["out"], a["path"],
                                    a["nsl"], a["ws"], a["ws_bytes"], a["err"], None)
    assert acc(bs=0) == b.SPEC_EINVAL
    assert acc(N=0) == b.SPEC_EINVAL
    assert acc(N=513) == b.SPEC_EINVAL
    assert acc(par=None) == b.SPEC_EINVAL
    assert acc(path=None) == b.SPEC_EINVAL
    assert acc(V=524289) == b.SPEC_ENOTSUP
    need = lib.spec_accept_tree_workspace_bytes(4, 32, 151936)
    assert need > lib.spec_accept_workspace_bytes(4, 31, 151936, 0)   # + the node ids
    assert acc(ws_bytes=need - 1) == b.SPEC_ENOSPC


def test_argmax_rejects_bad_arguments(lib):
    assert lib.spec_draft_argmax(0, 10, 1, FAKE, FAKE, None) == b.SPEC_EINVAL
    assert lib.spec_draft_argmax(4, 0, 1, FAKE, FAKE, None) == b.SPEC_EINVAL
    assert lib.spec_draft_argmax(4, 10, 5, FAKE, FAKE, None) == b.SPEC_ENOTSUP
    assert lib.spec_draft_argmax(4, 10, 1, None, FAKE, None) == b.SPEC_EINVAL


def test_binding_fails_loudly_without_gpu_tensors(lib):
    import torch
    x = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(b.SpecError):
        va.prepare_block(x, x, torch.zeros((3, 2), dtype=torch.int32), 16, 4, 0, 8)


def test_sampling_filter_rejects_bad_arguments(lib):
    def filt(**kw):
        a = dict(rows=8, V=151936, dt=b.F32, x=FAKE, T=1.0, k=50, p=0.95, ids=FAKE, probs=FAKE,
                 n=FAKE, ws=FAKE, ws_bytes=1 << 30)
        a.update(kw)
        return lib.spec_sampling_filter(a["rows"], a["V"], a["dt"], a["x"], a["T"], a["k"], a["p"],
                                        a["ids"], a["probs"], a["n"], a["ws"], a["ws_bytes"], None)
    assert filt(rows=0) == b.SPEC_EINVAL
    assert filt(V=0) == b.SPEC_EINVAL
    assert filt(x=None) == b.SPEC_EINVAL
    assert filt(n=None) == b.SPEC_EINVAL
    assert filt(T=0.0) == b.SPEC_EINVAL
    assert filt(T=float("inf")) == b.SPEC_EINVAL
    assert filt(k=0) == b.SPEC_EINVAL
    assert filt(k=65) == b.SPEC_EINVAL
    assert filt(p=0.0) == b.SPEC_EINVAL
    assert filt(p=float("nan")) == b.SPEC_EINVAL
    assert filt(dt=7) == b.SPEC_ENOTSUP
    assert filt(V=524289) == b.SPEC_ENOTSUP
    need = lib.spec_sampling_filter_workspace_bytes(8, 151936)
    assert need >= 8 * 2374 * 4
    assert filt(ws_bytes=need - 1) == b.SPEC_ENOSPC
    assert filt(ws=None) == b.SPEC_ENOSPC


def test_accept_logits_rejects_bad_arguments(lib):
    def acc(**kw):
        a = dict(bs=4, K=15, V=151936, dt=b.F32, T=1.0, k=50, p=0.95, tl=FAKE, dl=FAKE, dr=FAKE,
                 u=FAKE, seq=FAKE, al=FAKE, cl=FAKE, bon=FAKE, out=FAKE, nsl=FAKE, ws=FAKE,
                 ws_bytes=1 << 30, err=None)
        a.update(kw)
        return lib.spec_accept_logits(a["bs"], a["K"], a["V"], a["dt"], a["T"], a["k"], a["p"],
                                      a["tl"], a["dl"], a["dr"], a["u"], a["seq"], a["al"],
                                      a["cl"], a["bon"], a["out"], a["nsl"], a["ws"],
                                      a["ws_bytes"], a["err"], None)
    assert acc(bs=0) == b.SPEC_EINVAL
    assert acc(K=0) == b.SPEC_EINVAL
    assert acc(K=64) == b.SPEC_EINVAL
    assert acc(dl=None) == b.SPEC_EINVAL
    assert acc(u=None) == b.SPEC_EINVAL
    assert acc(nsl=None) == b.SPEC_EINVAL
    assert acc(k=65) == b.SPEC_EINVAL
    assert acc(T=-1.0) == b.SPEC_EINVAL
    assert acc(dt=3) == b.SPEC_ENOTSUP
    assert acc(V=524289) == b.SPEC_ENOTSUP
    need = lib.spec_accept_logits_workspace_bytes(4, 15, 151936, 50)
    # tile maxima plus kept ids, probabilities and counts of 4 * 31 rows
    assert need >= 4 * 31 * (2374 * 4 + 50 * 12 + 4)
    assert acc(ws_bytes=need - 1) == b.SPEC_ENOSPC
    assert lib.spec_accept_logits_workspace_bytes(4, 15, 151936, 65) == 0


def test_commit_kv_rejects_bad_arguments(lib):
    def com(**kw):
        a = dict(dt=b.BF16, bs=4, B=32, hkv=8, D=128, P=16, mp=70, np_=300, seq=FAKE, al=FAKE,
                 path=None, tab=FAKE, k=FAKE, v=FAKE, freed=FAKE, err=None)
        a.update(kw)
        return lib.spec_commit_kv(a["dt"], a["bs"], a["B"], a["hkv"], a["D"], a["P"], a["mp"],
                                  a["np_"], a["seq"], a["al"], a["path"], a["tab"], a["k"],
                                  a["v"], a["freed"], a["err"], None)
    assert com(bs=0) == b.SPEC_EINVAL
    assert com(B=0) == b.SPEC_EINVAL
    assert com(B=513) == b.SPEC_EINVAL
    assert com(hkv=0) == b.SPEC_EINVAL
    assert com(seq=None) == b.SPEC_EINVAL
    assert com(freed=None) == b.SPEC_EINVAL
    assert com(k=None) == b.SPEC_EINVAL
    assert com(D=96) == b.SPEC_ENOTSUP
    assert com(P=8) == b.SPEC_ENOTSUP
    assert com(dt=9) == b.SPEC_ENOTSUP


def test_accept_tree_commit_rejects_bad_arguments(lib):
    ws = lib.spec_accept_tree_workspace_bytes(4, 32, 151936)

    def atc(**kw):
        a = dict(bs=4, N=32, V=151936, par=FAKE, tok=FAKE, p=FAKE, u=FAKE, seq=FAKE, al=FAKE,
                 cl=FAKE, bon=FAKE, ot=FAKE, pn=FAKE, nsl=FAKE, dt=b.BF16, hkv=8, D=128, P=16,
                 mp=70, np_=300, tab=FAKE, k=FAKE, v=FAKE, freed=FAKE, ws=FAKE, ws_bytes=ws,
                 err=None)
        a.update(kw)
        return lib.spec_accept_tree_commit(
            a["bs"], a["N"], a["V"], a["par"], a["tok"], a["p"], a["u"], a["seq"], a["al"],
            a["cl"], a["bon"], a["ot"], a["pn"], a["nsl"], a["dt"], a["hkv"], a["D"], a["P"],
            a["mp"], a["np_"], a["tab"], a["k"], a["v"], a["freed"], a["ws"], a["ws_bytes"],
            a["err"], None)
    # the commit's arguments
    assert atc(dt=9) == b.SPEC_ENOTSUP
    assert atc(D=96) == b.SPEC_ENOTSUP
    assert atc(P=8) == b.SPEC_ENOTSUP
    assert atc(hkv=0) == b.SPEC_EINVAL
    assert atc(mp=0) == b.SPEC_EINVAL
    assert atc(tab=None) == b.SPEC_EINVAL
    assert atc(k=None) == b.SPEC_EINVAL
    assert atc(freed=None) == b.SPEC_EINVAL
    # the accept's arguments
    assert atc(N=513) == b.SPEC_EINVAL
    assert atc(bs=0) == b.SPEC_EINVAL
    assert atc(par=None) == b.SPEC_EINVAL
    assert atc(V=600000) == b.SPEC_ENOTSUP
    assert atc(ws_bytes=ws - 1) == b.SPEC_ENOSPC


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built library the entry points raise: there is no other
    implementation behind the names."""
    monkeypatch.setattr(b, "_LIB", None)
    monkeypatch.setattr(b, "lib_path", lambda: str(tmp_path / "libspecattn.so"))
    with pytest.raises(b.SpecError, match="not built"):
        b.load()
    with pytest.raises(b.SpecError, match="not built"):
        va.attn_workspace_bytes(2, 16, 32, 8, 128, 1024)


def test_binding_rejects_bad_buffers_before_any_launch():
    """The binding's checks on the buffers it passes on: the error word must
    be an int32 GPU tensor with at least one element, a workspace must be a GPU
    tensor of at least the planned bytes (counted in bytes, whatever its
    dtype), the page table must have one row per request, and every tensor of
    a call must live on one device. All of them raise before a pointer
    reaches the library."""
    import torch
    with pytest.raises(TypeError):
        b._need_err(torch.zeros(1, dtype=torch.int64))
    with pytest.raises(ValueError):
        b._need_err(torch.zeros(0, dtype=torch.int32))
    with pytest.raises(b.SpecError, match="GPU"):
        b._need_err(torch.zeros(1, dtype=torch.int32))      # a host error word
    assert b._need_err(None) is None
    with pytest.raises(b.SpecError, match="needs a workspace"):
        b._need_ws(None, 64)
    assert b._need_ws(None, 0) == 0
    with pytest.raises(b.SpecError, match="smaller"):
        b._need_ws(torch.empty(15, dtype=torch.float32), 61)  # 60 bytes, not 15
    with pytest.raises(b.SpecError, match="GPU"):
        b._need_ws(torch.empty(16, dtype=torch.float32), 61)  # big enough, but host memory
    with pytest.raises(ValueError, match="page_table"):
        b._need_table(torch.zeros((3, 8), dtype=torch.int32), 4)
    with pytest.raises(TypeError):
        b._need_table(torch.zeros((4, 8), dtype=torch.int64), 4)
    with pytest.raises(b.SpecError, match="GPU"):
        b._need_table(torch.zeros((4, 8), dtype=torch.int32), 4)
    with pytest.raises(b.SpecError, match="different devices"):
        b._same_device(torch.zeros(1), torch.zeros(1, device="meta"))
    out = b._need_out(None, b._accept_outputs(3, 5), "cpu")
    assert out["out_tokens"].shape == (3, 5) and out["bonus"].dtype == torch.int32
    with pytest.raises(ValueError):
        b._need_out(dict(out, bonus=torch.zeros(2, dtype=torch.int32)), b._accept_outputs(3, 5),
                    "cpu")
    # a whole call on host tensors stops at its first check
    q = torch.zeros((2, 4, 2, 64), dtype=torch.float32)
    with pytest.raises(b.SpecError, match="GPU"):
        b.block_attn_call(1, q, torch.zeros((4, 1, 16, 64)), torch.zeros((4, 1, 64, 16)),
                          torch.zeros((2, 2), dtype=torch.int32),
                          torch.zeros(2, dtype=torch.int32), 64)


def test_static_accept_rejects_before_any_launch(lib):
    """spec_accept_static checks like spec_accept, and refuses sizes whose
    workspace would not fit its fixed per-GPU scratch (SPEC_ESCRATCH), all
    on the host."""
    def call(bs=4, K=15, V=151936, greedy=0, p=FAKE, q=FAKE):
        return lib.spec_accept_static(bs, K, V, greedy, p, q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, None, None)
    assert call(bs=0) == b.SPEC_EINVAL
    assert call(K=64) == b.SPEC_EINVAL
    assert call(p=None) == b.SPEC_EINVAL
    assert call(q=None) == b.SPEC_EINVAL
    assert call(V=(1 << 19) + 1) == b.SPEC_ENOTSUP
    big = 1024
    assert lib.spec_accept_workspace_bytes(big, 15, 151936, 0) > b.ACCEPT_STATIC_SCRATCH_BYTES
    assert call(bs=big) == b.SPEC_ESCRATCH
    assert lib.spec_accept_workspace_bytes(256, 15, 151936, 0) <= b.ACCEPT_STATIC_SCRATCH_BYTES
    assert b"scratch" in lib.spec_status_string(b.SPEC_ESCRATCH)
