"""ctypes binding of libspecattn.so (include/specattn.h).

Argument marshalling only: torch tensors are checked for device, dtype, shape
and contiguity, their data pointers and the current HIP stream are handed to
the C ABI, and a negative status raises. Each entry point also has a `*_call`
form that checks once and returns an `enqueue()` closure re-issuing the same
call with the pre-marshalled pointers (for loops that launch the same round
many times without re-checking). Every step of the computation runs in
the library's HIP kernels; there is no other implementation behind these
names, so a missing library or device is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
_LIB = None

SPEC_OK, SPEC_EINVAL, SPEC_ENOTSUP, SPEC_ENOSPC, SPEC_EHIP, SPEC_ESCRATCH = 0, -1, -2, -3, -4, -5
ACCEPT_STATIC_SCRATCH_BYTES = 4 << 20  # SPEC_ACCEPT_STATIC_SCRATCH_BYTES
ERR_SLOT, ERR_CAPACITY, ERR_TOKEN, ERR_ZERO_RESIDUAL, ERR_TREE = 1, 2, 4, 8, 16
BIDIR, CAUSAL, MIXED, TREE = 0, 1, 2, 3
F32, BF16 = 0, 1

_c_int, _c_size, _vp, _f = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float

_SIGS = {
    "spec_version": (_c_int, []),
    "spec_status_string": (ctypes.c_char_p, [_c_int]),
    "spec_prepare_block": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, ctypes.c_int32,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "spec_prepare_tree": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, ctypes.c_int32,
                                   _vp, _vp, _vp, _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _vp]),
    "spec_quadratic_handoff_workspace_bytes": (_c_size, [_c_int] * 3),
    "spec_quadratic_handoff": (_c_int, [_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp,
                                        ctypes.c_int32, _vp, _vp, _vp, _c_size, _vp, _vp]),
    "spec_accept_quadratic_workspace_bytes": (_c_size, [_c_int] * 3),
    "spec_accept_quadratic": (_c_int, [_c_int] * 3 + [_vp] * 5 + [_c_int, _vp, ctypes.c_int32] +
                              [_vp] * 9 + [_c_int] * 6 + [_vp] * 5 + [_c_size, _vp, _vp]),
    "spec_accept_prepare": (_c_int, [_c_int] * 4 + [_vp] * 10 + [_c_int] * 4 +
                            [ctypes.c_int32] + [_vp] * 5 + [_c_size, _vp, _vp]),
    "block_attn_workspace_bytes": (_c_size, [_c_int] * 6),
    "block_attn": (_c_int, [_c_int, _c_int, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                            _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _f, _vp,
                            _vp, _vp, _c_size, _vp, _vp]),
    "block_attn_tree": (_c_int, [_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                 _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _f, _vp,
                                 _vp, _vp, _c_size, _vp, _vp]),
    "spec_draft_argmax": (_c_int, [_c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "spec_accept_workspace_bytes": (_c_size, [_c_int] * 4),
    "spec_accept_tree_workspace_bytes": (_c_size, [_c_int] * 3),
    "spec_accept_tree": (_c_int, [_c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _c_size, _vp, _vp]),
    "spec_accept": (_c_int, [_c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _vp, _vp, _c_size, _vp, _vp]),
    "spec_accept_static": (_c_int, [_c_int] * 4 + [_vp] * 12),
    "spec_commit_kv": (_c_int, [_c_int] * 8 + [_vp] * 9),
    "spec_accept_tree_commit": (_c_int, [_c_int] * 3 + [_vp] * 11 + [_c_int] * 6 +
                                [_vp] * 5 + [_c_size, _vp, _vp]),
    "spec_sampling_filter_workspace_bytes": (_c_size, [_c_int] * 2),
    "spec_sampling_filter": (_c_int, [_c_int, _c_int, _c_int, _vp, _f, _c_int, _f, _vp, _vp, _vp,
                                      _vp, _c_size, _vp]),
    "spec_accept_logits_workspace_bytes": (_c_size, [_c_int] * 4),
    "spec_accept_logits": (_c_int, [_c_int, _c_int, _c_int, _c_int, _f, _c_int, _f, _vp, _vp, _vp,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp, _vp]),
}


class SpecError(RuntimeError):
    pass


def lib_path() -> str:
    return os.path.join(_HERE, "libspecattn.so")


def header_path() -> str:
    return os.path.join(_ROOT, "include", "specattn.h")


def header_functions() -> list:
    """Names of the functions include/specattn.h declares."""
    txt = open(header_path()).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", txt, flags=re.M)))


def load():
    """Load the built library (raises when it is missing). torch is imported
    first: the library's HIP runtime dependency must resolve to the runtime
    torch already loaded (one HIP runtime per process), not load a second
    one."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise SpecError(f"{path} is not built; run __graft_entry__.build() first")
        _torch()
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _check(status: int, what: str):
    if status != SPEC_OK:
        msg = load().spec_status_string(status).decode()
        raise SpecError(f"{what} failed with status {status}: {msg}")


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, shape=None, device=True):
    """Type, dtype, shape and contiguity, then (device=True) that the tensor
    lives on a GPU."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device and not t.is_cuda:
        raise SpecError(f"{name} must live on the GPU")
    return t


def _need_err(err):
    """The device error word: int32 on the GPU with at least one element (or None)."""
    torch = _torch()
    if err is None:
        return None
    _need(err, "err", torch.int32, device=False)
    if err.numel() < 1:
        raise ValueError("err needs at least one int32 element")
    return _need(err, "err")


def _need_ws(ws, need):
    """A workspace on the GPU (contiguous) of at least `need` bytes; returns its
    size in bytes (0 for None)."""
    if ws is None:
        if need > 0:
            raise SpecError(f"the call needs a workspace of {need} bytes")
        return 0
    _need(ws, "ws", device=False)
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise SpecError(f"workspace of {nbytes} bytes is smaller than the {need} the call needs")
    _need(ws, "ws")
    return nbytes


def _need_table(page_table, bs):
    """page_table [bs, max_pages] int32 on the GPU."""
    torch = _torch()
    _need(page_table, "page_table", torch.int32, device=False)
    if page_table.dim() != 2 or page_table.shape[0] != bs:
        raise ValueError(f"page_table must have shape ({bs}, max_pages), got "
                         f"{tuple(page_table.shape)}")
    return _need(page_table, "page_table")


def _need_out(out, specs, dev):
    """Creates (out None) or checks the output tensors of an accept-style call:
    specs maps name -> shape (int32 unless a dtype is given as a third entry)."""
    torch = _torch()
    if out is None:
        out = {}
        for name, spec in specs.items():
            dt = spec[1] if len(spec) > 1 else torch.int32
            out[name] = torch.empty(spec[0], dtype=dt, device=dev)
        return out
    for name, spec in specs.items():
        if name not in out:
            raise KeyError(f"out is missing {name}")
        dt = spec[1] if len(spec) > 1 else torch.int32
        _need(out[name], name, dt, spec[0], device=False)
    for name in specs:
        _need(out[name], name)
    return out


def _same_device(*ts):
    """Every tensor given lives on one GPU, the current one (the library
    launches on the current device and plans for its compute units)."""
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise SpecError(f"tensors live on different devices: {sorted(map(str, devs))}")
    dev = next(iter(devs), None)
    if dev is not None and dev.type == "cuda":
        torch = _torch()
        cur = torch.cuda.current_device()
        if (dev.index if dev.index is not None else cur) != cur:
            raise SpecError(f"tensors live on {dev}, but the current device is cuda:{cur}")


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# --------------------------------------------------------------- workspaces
def attn_workspace_bytes(bs, B, hq, hkv, d, max_kv_len) -> int:
    return int(load().block_attn_workspace_bytes(bs, B, hq, hkv, d, max_kv_len))


def accept_workspace_bytes(bs, K, V, greedy=False) -> int:
    return int(load().spec_accept_workspace_bytes(bs, K, V, int(bool(greedy))))


def workspace(nbytes, device="cuda"):
    """A device workspace of at least nbytes (contents irrelevant to the library)."""
    torch = _torch()
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# -------------------------------------------------------------------- calls
def prepare_block_call(verified_id, seq_lens, page_table, page_size, block, mask_token_id,
                       num_pages, draft_tokens=None, out=None, err=None, stream=None):
    """Checks the arguments of spec_prepare_block once and returns (enqueue, out)."""
    torch = _torch()
    bs = verified_id.shape[0]
    _need(verified_id, "verified_id", torch.int32, (bs,))
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    _need_table(page_table, bs)
    _need_err(err)
    if draft_tokens is not None:
        _need(draft_tokens, "draft_tokens", torch.int32, (bs, block - 1))
    if out is None:
        out = tuple(torch.empty((bs, block), dtype=torch.int32, device=verified_id.device)
                    for _ in range(3))
    for t, nm in zip(out, ("block_ids", "positions", "cache_loc")):
        _need(t, nm, torch.int32, (bs, block))
    _same_device(verified_id, seq_lens, page_table, draft_tokens, *out, err)
    args = (bs, block, page_size, page_table.shape[1], num_pages, mask_token_id, _ptr(verified_id),
            _ptr(seq_lens), _ptr(page_table), _ptr(draft_tokens), _ptr(out[0]), _ptr(out[1]),
            _ptr(out[2]), _ptr(err), _stream(stream))
    fn = load().spec_prepare_block
    keep = (verified_id, seq_lens, page_table, draft_tokens, out, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_prepare_block")

    return enqueue, out


def prepare_block(verified_id, seq_lens, page_table, page_size, block, mask_token_id, num_pages,
                  draft_tokens=None, out=None, err=None, stream=None):
    """Block ids, positions and KV slots of one round (spec_prepare_block)."""
    enqueue, out = prepare_block_call(verified_id, seq_lens, page_table, page_size, block,
                                      mask_token_id, num_pages, draft_tokens, out, err, stream)
    enqueue()
    return out


def prepare_tree_call(verified_id, seq_lens, page_table, page_size, parent, mask_token_id,
                      num_pages, node_tokens=None, out=None, err=None, stream=None):
    """Checks the arguments of spec_prepare_tree once and returns (enqueue,
    out). parent: int32 [N] (one layout for the batch) or [bs, N];
    node_tokens: int32 [bs, N] or None (mask fill); out: block_ids,
    positions, cache_loc [bs, N]."""
    torch = _torch()
    bs = verified_id.shape[0]
    N = parent.shape[-1]
    _need(verified_id, "verified_id", torch.int32, (bs,))
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    _need_table(page_table, bs)
    _need(parent, "parent", torch.int32)
    if tuple(parent.shape) not in ((N,), (bs, N)):
        raise ValueError(f"parent must have shape ({N},) or ({bs}, {N})")
    _need_err(err)
    if node_tokens is not None:
        _need(node_tokens, "node_tokens", torch.int32, (bs, N))
    if out is None:
        out = tuple(torch.empty((bs, N), dtype=torch.int32, device=verified_id.device)
                    for _ in range(3))
    for t, nm in zip(out, ("block_ids", "positions", "cache_loc")):
        _need(t, nm, torch.int32, (bs, N))
    _same_device(verified_id, seq_lens, page_table, parent, node_tokens, *out, err)
    args = (bs, N, page_size, page_table.shape[1], num_pages, mask_token_id, _ptr(verified_id),
            _ptr(seq_lens), _ptr(page_table), _ptr(parent), int(parent.dim() == 2),
            _ptr(node_tokens), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(err),
            _stream(stream))
    fn = load().spec_prepare_tree
    keep = (verified_id, seq_lens, page_table, parent, node_tokens, out, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_prepare_tree")

    return enqueue, out


def prepare_tree(verified_id, seq_lens, page_table, page_size, parent, mask_token_id, num_pages,
                 node_tokens=None, out=None, err=None, stream=None):
    """Block ids, positions (committed length + depth) and KV slots of a tree
    or quadratic block (spec_prepare_tree)."""
    enqueue, out = prepare_tree_call(verified_id, seq_lens, page_table, page_size, parent,
                                     mask_token_id, num_pages, node_tokens, out, err, stream)
    enqueue()
    return out


def block_attn_call(mode, q, k_pool, v_pool, page_table, seq_lens, max_kv_len, n_causal=0,
                    n_causal_per_req=None, sm_scale=0.0, out=None, lse=None, ws=None, err=None,
                    stream=None):
    """Checks the arguments of block_attn once and returns (enqueue, out): each
    enqueue() queues the same call again with the pre-marshalled pointers."""
    torch = _torch()
    bs, B, hq, d = q.shape
    num_pages, hkv, P, d2 = k_pool.shape
    _need(q, "q")
    dt = _dtype_code(q)
    _need(k_pool, "k_pool", q.dtype)
    _need(v_pool, "v_pool", q.dtype, (num_pages, hkv, d, P))
    if d2 != d:
        raise ValueError("k_pool head dim differs from q")
    _need_table(page_table, bs)
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    _need_err(err)
    if n_causal_per_req is not None:
        _need(n_causal_per_req, "n_causal_per_req", torch.int32, (bs,))
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, q.shape)
    if lse is not None:
        _need(lse, "lse", torch.float32, (bs, B, hq))
    need = attn_workspace_bytes(bs, B, hq, hkv, d, max_kv_len)
    if ws is None and need > 0:
        ws = workspace(need, q.device)
    ws_bytes = _need_ws(ws, need)
    _same_device(q, k_pool, v_pool, page_table, seq_lens, n_causal_per_req, out, lse, ws, err)
    args = (mode, n_causal, _ptr(n_causal_per_req), dt, bs, B, hq, hkv, d, P, page_table.shape[1],
            num_pages, max_kv_len, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
            _ptr(seq_lens), sm_scale, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _ptr(err),
            _stream(stream))
    fn = load().block_attn
    keep = (q, k_pool, v_pool, page_table, seq_lens, n_causal_per_req, out, lse, ws, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "block_attn")

    return enqueue, out


def block_attn_tree_call(tree_mask, q, k_pool, v_pool, page_table, seq_lens, max_kv_len,
                         sm_scale=0.0, out=None, lse=None, ws=None, err=None, stream=None):
    """Checks the arguments of block_attn_tree once and returns (enqueue, out).
    tree_mask: int64 tensor of uint64 row bit patterns, W = ceil(B / 64) words
    per row: [B, W] (one tree for the batch) or [bs, B, W] (one tree per
    request); for B <= 64 also [B] or [bs, B]."""
    torch = _torch()
    bs, B, hq, d = q.shape
    num_pages, hkv, P, d2 = k_pool.shape
    _need(q, "q")
    dt = _dtype_code(q)
    _need(k_pool, "k_pool", q.dtype)
    _need(v_pool, "v_pool", q.dtype, (num_pages, hkv, d, P))
    if d2 != d:
        raise ValueError("k_pool head dim differs from q")
    _need_table(page_table, bs)
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    _need_err(err)
    _need(tree_mask, "tree_mask", torch.int64)
    W = (B + 63) // 64
    shapes = {(B, W): False, (bs, B, W): True}
    if W == 1:
        shapes.update({(B,): False, (bs, B): True})
    if tuple(tree_mask.shape) not in shapes:
        raise ValueError(f"tree_mask must have shape ({B}, {W}) or ({bs}, {B}, {W})"
                         + (f", ({B},) or ({bs}, {B})" if W == 1 else ""))
    per_request = shapes[tuple(tree_mask.shape)]
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, q.shape)
    if lse is not None:
        _need(lse, "lse", torch.float32, (bs, B, hq))
    need = attn_workspace_bytes(bs, B, hq, hkv, d, max_kv_len)
    if ws is None and need > 0:
        ws = workspace(need, q.device)
    ws_bytes = _need_ws(ws, need)
    _same_device(tree_mask, q, k_pool, v_pool, page_table, seq_lens, out, lse, ws, err)
    args = (_ptr(tree_mask), int(per_request), dt, bs, B, hq, hkv, d, P, page_table.shape[1],
            num_pages, max_kv_len, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
            _ptr(seq_lens), sm_scale, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _ptr(err),
            _stream(stream))
    fn = load().block_attn_tree
    keep = (tree_mask, q, k_pool, v_pool, page_table, seq_lens, out, lse, ws, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "block_attn_tree")

    return enqueue, out


def block_attn_tree(tree_mask, q, k_pool, v_pool, page_table, seq_lens, max_kv_len, sm_scale=0.0,
                    out=None, lse=None, ws=None, err=None, stream=None):
    """Tree-block attention over the paged cache (block_attn_tree)."""
    enqueue, out = block_attn_tree_call(tree_mask, q, k_pool, v_pool, page_table, seq_lens,
                                        max_kv_len, sm_scale, out, lse, ws, err, stream)
    enqueue()
    return out


def block_attn(mode, q, k_pool, v_pool, page_table, seq_lens, max_kv_len, n_causal=0,
               n_causal_per_req=None, sm_scale=0.0, out=None, lse=None, ws=None, err=None,
               stream=None):
    """Block-query attention over the paged cache (block_attn).

    q [bs, B, Hq, D]; k_pool [pages, Hkv, P, D]; v_pool [pages, Hkv, D, P]."""
    enqueue, out = block_attn_call(mode, q, k_pool, v_pool, page_table, seq_lens, max_kv_len,
                                   n_causal, n_causal_per_req, sm_scale, out, lse, ws, err, stream)
    enqueue()
    return out


def draft_argmax_call(logits, out=None, stream=None):
    """Checks the arguments of spec_draft_argmax once and returns (enqueue, out)."""
    torch = _torch()
    _need(logits, "logits")
    rows, V = logits.shape
    if out is None:
        out = torch.empty(rows, dtype=torch.int32, device=logits.device)
    _need(out, "tokens", torch.int32, (rows,))
    _same_device(logits, out)
    args = (rows, V, _dtype_code(logits), _ptr(logits), _ptr(out), _stream(stream))
    fn = load().spec_draft_argmax
    keep = (logits, out)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_draft_argmax")

    return enqueue, out


def quadratic_handoff_workspace_bytes(bs, k, V) -> int:
    return int(load().spec_quadratic_handoff_workspace_bytes(bs, k, V))


def quadratic_handoff_call(logits, accept_len, k, bonus=None, mask_token_id=0, out=None,
                           ws=None, err=None, stream=None):
    """Checks the arguments of spec_quadratic_handoff once and returns
    (enqueue, out). logits [bs, (k + 1)^2, V] float32 or bfloat16; out:
    next_draft [bs, k] and, when bonus is given, next_block [bs, (k + 1)^2]."""
    torch = _torch()
    bs, n, V = logits.shape
    if n != (k + 1) * (k + 1):
        raise ValueError(f"logits must hold (k + 1)^2 = {(k + 1) ** 2} rows per request")
    _need(logits, "logits")
    dt = _dtype_code(logits)
    _need(accept_len, "accept_len", torch.int32, (bs,))
    if bonus is not None:
        _need(bonus, "bonus", torch.int32, (bs,))
    _need_err(err)
    specs = dict(next_draft=((bs, k),))
    if bonus is not None:
        specs["next_block"] = ((bs, n),)
    out = _need_out(out, specs, logits.device)
    need = quadratic_handoff_workspace_bytes(bs, k, V)
    if ws is None:
        ws = workspace(need, logits.device)
    ws_bytes = _need_ws(ws, need)
    _same_device(logits, accept_len, bonus, ws, err, *out.values())
    args = (bs, k, V, dt, _ptr(logits), _ptr(accept_len), _ptr(bonus), mask_token_id,
            _ptr(out["next_draft"]), _ptr(out.get("next_block")), _ptr(ws), ws_bytes, _ptr(err),
            _stream(stream))
    fn = load().spec_quadratic_handoff
    keep = (logits, accept_len, bonus, out, ws, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_quadratic_handoff")

    return enqueue, out


def quadratic_handoff(logits, accept_len, k, bonus=None, mask_token_id=0, out=None, ws=None,
                      err=None, stream=None):
    """Next round's drafts (and block tokens) from a quadratic block
    (spec_quadratic_handoff)."""
    enqueue, out = quadratic_handoff_call(logits, accept_len, k, bonus, mask_token_id, out, ws,
                                          err, stream)
    enqueue()
    return out


def draft_argmax(logits, out=None, stream=None):
    """Greedy draft tokens: lowest-index argmax of each row of logits [rows, V]."""
    enqueue, out = draft_argmax_call(logits, out, stream)
    enqueue()
    return out


def _accept_outputs(bs, n_tok):
    """Output shapes shared by the accept calls (int32)."""
    return dict(accept_len=((bs,),), commit_len=((bs,),), bonus=((bs,),),
                out_tokens=((bs, n_tok),), new_seq_lens=((bs,),))


def accept_call(p, q, draft, u, seq_lens, greedy=False, out=None, ws=None, err=None, stream=None):
    """Checks the arguments of spec_accept once and returns (enqueue, out)."""
    torch = _torch()
    bs, K1, V = p.shape
    K = K1 - 1
    _need(p, "p", torch.float32)
    _need(draft, "draft", torch.int32, (bs, K))
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    if not greedy:
        _need(q, "q", torch.float32, (bs, K, V))
        _need(u, "u", torch.float32, (bs, K + 1))
    _need_err(err)
    dev = p.device
    out = _need_out(out, _accept_outputs(bs, K + 1), dev)
    need = accept_workspace_bytes(bs, K, V, greedy)
    if ws is None:
        ws = workspace(need, dev)
    ws_bytes = _need_ws(ws, need)
    _same_device(p, None if greedy else q, draft, None if greedy else u, seq_lens, ws, err,
                 *out.values())
    args = (bs, K, V, int(bool(greedy)), _ptr(p), _ptr(q), _ptr(draft), _ptr(u), _ptr(seq_lens),
            _ptr(out["accept_len"]), _ptr(out["commit_len"]), _ptr(out["bonus"]),
            _ptr(out["out_tokens"]), _ptr(out["new_seq_lens"]), _ptr(ws), ws_bytes, _ptr(err),
            _stream(stream))
    fn = load().spec_accept
    keep = (p, q, draft, u, seq_lens, out, ws, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_accept")

    return enqueue, out


def accept_prepare_call(p, q, draft, u, seq_lens, page_table, page_size, block_next,
                        mask_token_id, num_pages, greedy=False, out=None, ws=None, err=None,
                        stream=None):
    """Checks the arguments of spec_accept_prepare once and returns (enqueue,
    out): the outputs of accept_call plus block_ids, positions, cache_loc
    [bs, block_next] of the next round's draft-pass block."""
    torch = _torch()
    bs, K1, V = p.shape
    K = K1 - 1
    _need(p, "p", torch.float32)
    _need(draft, "draft", torch.int32, (bs, K))
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    if not greedy:
        _need(q, "q", torch.float32, (bs, K, V))
        _need(u, "u", torch.float32, (bs, K + 1))
    _need_table(page_table, bs)
    _need_err(err)
    dev = p.device
    out = _need_out(out, dict(_accept_outputs(bs, K + 1), block_ids=((bs, block_next),),
                              positions=((bs, block_next),), cache_loc=((bs, block_next),)),
                    dev)
    need = accept_workspace_bytes(bs, K, V, greedy)
    if ws is None:
        ws = workspace(need, dev)
    ws_bytes = _need_ws(ws, need)
    _same_device(p, None if greedy else q, draft, None if greedy else u, seq_lens, page_table, ws,
                 err, *out.values())
    args = (bs, K, V, int(bool(greedy)), _ptr(p), _ptr(q), _ptr(draft), _ptr(u), _ptr(seq_lens),
            _ptr(out["accept_len"]), _ptr(out["commit_len"]), _ptr(out["bonus"]),
            _ptr(out["out_tokens"]), _ptr(out["new_seq_lens"]), block_next, page_size,
            page_table.shape[1], num_pages, mask_token_id, _ptr(page_table),
            _ptr(out["block_ids"]), _ptr(out["positions"]), _ptr(out["cache_loc"]), _ptr(ws),
            ws_bytes, _ptr(err), _stream(stream))
    fn = load().spec_accept_prepare
    keep = (p, q, draft, u, seq_lens, page_table, out, ws, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_accept_prepare")

    return enqueue, out


def accept_prepare(p, q, draft, u, seq_lens, page_table, page_size, block_next, mask_token_id,
                   num_pages, greedy=False, out=None, ws=None, err=None, stream=None):
    """Speculative accept followed by the next round's draft-pass block in
    one call (spec_accept_prepare)."""
    enqueue, out = accept_prepare_call(p, q, draft, u, seq_lens, page_table, page_size,
                                       block_next, mask_token_id, num_pages, greedy, out, ws, err,
                                       stream)
    enqueue()
    return out


def accept_quadratic_workspace_bytes(bs, k, V) -> int:
    return int(load().spec_accept_quadratic_workspace_bytes(bs, k, V))


def accept_quadratic_call(p, q, draft, u, seq_lens, logits, k_pool, v_pool, page_table,
                          mask_token_id=0, next_block=True, prepare_next=False, out=None,
                          ws=None, err=None, stream=None):
    """Checks the arguments of spec_accept_quadratic once and returns
    (enqueue, out): the outputs of accept_call plus next_draft [bs, k],
    next_block [bs, (k + 1)^2] (unless next_block is False), with
    prepare_next the next round's positions and cache_loc [bs, (k + 1)^2],
    and freed [bs, (k + 1)^2]; k_pool / v_pool are updated in place."""
    torch = _torch()
    bs, K1, V = p.shape
    k = K1 - 1
    n = (k + 1) * (k + 1)
    _need(p, "p", torch.float32)
    _need(q, "q", torch.float32, (bs, k, V))
    _need(draft, "draft", torch.int32, (bs, k))
    _need(u, "u", torch.float32, (bs, k + 1))
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    _need(logits, "logits", shape=(bs, n, V))
    ldt = _dtype_code(logits)
    num_pages, hkv, P, d = k_pool.shape
    _need(k_pool, "k_pool")
    kdt = _dtype_code(k_pool)
    _need(v_pool, "v_pool", k_pool.dtype, (num_pages, hkv, d, P))
    _need_table(page_table, bs)
    _need_err(err)
    specs = dict(_accept_outputs(bs, k + 1), next_draft=((bs, k),), freed=((bs, n),))
    if next_block:
        specs["next_block"] = ((bs, n),)
    if prepare_next:
        specs["positions"] = ((bs, n),)
        specs["cache_loc"] = ((bs, n),)
    out = _need_out(out, specs, p.device)
    need = accept_quadratic_workspace_bytes(bs, k, V)
    if ws is None:
        ws = workspace(need, p.device)
    ws_bytes = _need_ws(ws, need)
    _same_device(p, q, draft, u, seq_lens, logits, k_pool, v_pool, page_table, ws, err,
                 *out.values())
    args = (bs, k, V, _ptr(p), _ptr(q), _ptr(draft), _ptr(u), _ptr(seq_lens), ldt, _ptr(logits),
            mask_token_id, _ptr(out["accept_len"]), _ptr(out["commit_len"]), _ptr(out["bonus"]),
            _ptr(out["out_tokens"]), _ptr(out["new_seq_lens"]), _ptr(out["next_draft"]),
            _ptr(out.get("next_block")), _ptr(out.get("positions")), _ptr(out.get("cache_loc")),
            kdt, hkv, d, P, page_table.shape[1], num_pages,
            _ptr(page_table), _ptr(k_pool), _ptr(v_pool), _ptr(out["freed"]), _ptr(ws), ws_bytes,
            _ptr(err), _stream(stream))
    fn = load().spec_accept_quadratic
    keep = (p, q, draft, u, seq_lens, logits, k_pool, v_pool, page_table, out, ws, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_accept_quadratic")

    return enqueue, out


def accept_quadratic(p, q, draft, u, seq_lens, logits, k_pool, v_pool, page_table,
                     mask_token_id=0, next_block=True, prepare_next=False, out=None, ws=None,
                     err=None, stream=None):
    """A quadratic round's accept, hand-off and spine commit in one call
    (spec_accept_quadratic); with prepare_next also the next round's block
    positions and slots."""
    enqueue, out = accept_quadratic_call(p, q, draft, u, seq_lens, logits, k_pool, v_pool,
                                         page_table, mask_token_id, next_block, prepare_next,
                                         out, ws, err, stream)
    enqueue()
    return out


def accept(p, q, draft, u, seq_lens, greedy=False, out=None, ws=None, err=None, stream=None):
    """Speculative accept / bonus (spec_accept). Returns a dict of int32 tensors:
    accept_len, commit_len, bonus, out_tokens [bs, K+1], new_seq_lens."""
    enqueue, out = accept_call(p, q, draft, u, seq_lens, greedy, out, ws, err, stream)
    enqueue()
    return out


def accept_static_call(p, q, draft, u, seq_lens, greedy=False, out=None, err=None,
                       stream=None):
    """Checks the arguments of spec_accept_static once and returns (enqueue,
    out): the accept of accept_call with its workspace in the library's fixed
    per-GPU array (no workspace tensor; calls on one GPU must be ordered)."""
    torch = _torch()
    bs, K1, V = p.shape
    K = K1 - 1
    _need(p, "p", torch.float32)
    _need(draft, "draft", torch.int32, (bs, K))
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    if not greedy:
        _need(q, "q", torch.float32, (bs, K, V))
        _need(u, "u", torch.float32, (bs, K + 1))
    _need_err(err)
    dev = p.device
    out = _need_out(out, _accept_outputs(bs, K + 1), dev)
    if accept_workspace_bytes(bs, K, V, greedy) > ACCEPT_STATIC_SCRATCH_BYTES:
        raise SpecError(f"spec_accept_static: bs {bs}, K {K}, V {V} need more than the "
                        f"{ACCEPT_STATIC_SCRATCH_BYTES} bytes of fixed scratch")
    _same_device(p, None if greedy else q, draft, None if greedy else u, seq_lens, err,
                 *out.values())
    args = (bs, K, V, int(bool(greedy)), _ptr(p), _ptr(q), _ptr(draft), _ptr(u), _ptr(seq_lens),
            _ptr(out["accept_len"]), _ptr(out["commit_len"]), _ptr(out["bonus"]),
            _ptr(out["out_tokens"]), _ptr(out["new_seq_lens"]), _ptr(err), _stream(stream))
    fn = load().spec_accept_static
    keep = (p, q, draft, u, seq_lens, out, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_accept_static")

    return enqueue, out


def accept_static(p, q, draft, u, seq_lens, greedy=False, out=None, err=None, stream=None):
    """Speculative accept / bonus without a workspace (spec_accept_static):
    the outputs of accept()."""
    enqueue, out = accept_static_call(p, q, draft, u, seq_lens, greedy, out, err, stream)
    enqueue()
    return out


def accept_tree_workspace_bytes(bs, N, V) -> int:
    return int(load().spec_accept_tree_workspace_bytes(bs, N, V))


def accept_tree_call(parent, token, p, u, seq_lens, out=None, ws=None, err=None, stream=None):
    """Checks the arguments of spec_accept_tree once and returns (enqueue, out).
    parent, token [bs, N] int32; p [bs, N, V] float32; u [bs, N] float32."""
    torch = _torch()
    bs, N, V = p.shape
    _need(p, "p", torch.float32)
    _need(parent, "parent", torch.int32, (bs, N))
    _need(token, "token", torch.int32, (bs, N))
    _need(u, "u", torch.float32, (bs, N))
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    _need_err(err)
    dev = p.device
    out = _need_out(out, dict(_accept_outputs(bs, N), path_nodes=((bs, N),)), dev)
    need = accept_tree_workspace_bytes(bs, N, V)
    if ws is None:
        ws = workspace(need, dev)
    ws_bytes = _need_ws(ws, need)
    _same_device(parent, token, p, u, seq_lens, ws, err, *out.values())
    args = (bs, N, V, _ptr(parent), _ptr(token), _ptr(p), _ptr(u), _ptr(seq_lens),
            _ptr(out["accept_len"]), _ptr(out["commit_len"]), _ptr(out["bonus"]),
            _ptr(out["out_tokens"]), _ptr(out["path_nodes"]), _ptr(out["new_seq_lens"]),
            _ptr(ws), ws_bytes, _ptr(err), _stream(stream))
    fn = load().spec_accept_tree
    keep = (parent, token, p, u, seq_lens, out, ws, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_accept_tree")

    return enqueue, out


def accept_tree_commit_call(parent, token, p, u, seq_lens, k_pool, v_pool, page_table, out=None,
                            ws=None, err=None, stream=None):
    """Checks the arguments of spec_accept_tree_commit once and returns
    (enqueue, out): the tree accept of accept_tree_call plus the commit of its
    path (k_pool / v_pool updated in place); out also holds freed [bs, N]."""
    torch = _torch()
    bs, N, V = p.shape
    _need(p, "p", torch.float32)
    _need(parent, "parent", torch.int32, (bs, N))
    _need(token, "token", torch.int32, (bs, N))
    _need(u, "u", torch.float32, (bs, N))
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    num_pages, hkv, P, d = k_pool.shape
    _need(k_pool, "k_pool")
    dt = _dtype_code(k_pool)
    _need(v_pool, "v_pool", k_pool.dtype, (num_pages, hkv, d, P))
    _need_table(page_table, bs)
    _need_err(err)
    dev = p.device
    out = _need_out(out, dict(_accept_outputs(bs, N), path_nodes=((bs, N),),
                              freed=((bs, N),)), dev)
    need = accept_tree_workspace_bytes(bs, N, V)
    if ws is None:
        ws = workspace(need, dev)
    ws_bytes = _need_ws(ws, need)
    _same_device(parent, token, p, u, seq_lens, k_pool, v_pool, page_table, ws, err,
                 *out.values())
    args = (bs, N, V, _ptr(parent), _ptr(token), _ptr(p), _ptr(u), _ptr(seq_lens),
            _ptr(out["accept_len"]), _ptr(out["commit_len"]), _ptr(out["bonus"]),
            _ptr(out["out_tokens"]), _ptr(out["path_nodes"]), _ptr(out["new_seq_lens"]),
            dt, hkv, d, P, page_table.shape[1], num_pages, _ptr(page_table), _ptr(k_pool),
            _ptr(v_pool), _ptr(out["freed"]), _ptr(ws), ws_bytes, _ptr(err), _stream(stream))
    fn = load().spec_accept_tree_commit
    keep = (parent, token, p, u, seq_lens, k_pool, v_pool, page_table, out, ws, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_accept_tree_commit")

    return enqueue, out


def accept_tree_commit(parent, token, p, u, seq_lens, k_pool, v_pool, page_table, out=None,
                       ws=None, err=None, stream=None):
    """Tree accept and commit in one call (spec_accept_tree_commit): the
    outputs of accept_tree plus freed [bs, N]; the pools are updated in place."""
    enqueue, out = accept_tree_commit_call(parent, token, p, u, seq_lens, k_pool, v_pool,
                                           page_table, out, ws, err, stream)
    enqueue()
    return out


def accept_tree(parent, token, p, u, seq_lens, out=None, ws=None, err=None, stream=None):
    """Tree accept (spec_accept_tree). Returns a dict of int32 tensors:
    accept_len, commit_len, bonus, out_tokens [bs, N], path_nodes [bs, N],
    new_seq_lens."""
    enqueue, out = accept_tree_call(parent, token, p, u, seq_lens, out, ws, err, stream)
    enqueue()
    return out


# ------------------------------------------------------ sampling parameters
def sampling_filter_workspace_bytes(rows, V) -> int:
    return int(load().spec_sampling_filter_workspace_bytes(rows, V))


def sampling_filter_call(logits, temperature, top_k, top_p, out=None, ws=None, stream=None):
    """Checks the arguments of spec_sampling_filter once and returns (enqueue,
    out). logits [rows, V] float32 or bfloat16; out: kept_ids [rows, top_k]
    int32, kept_probs [rows, top_k] float64, n_kept [rows] int32."""
    torch = _torch()
    rows, V = logits.shape
    _need(logits, "logits")
    dt = _dtype_code(logits)
    dev = logits.device
    out = _need_out(out, dict(kept_ids=((rows, top_k),),
                              kept_probs=((rows, top_k), torch.float64),
                              n_kept=((rows,),)), dev)
    need = sampling_filter_workspace_bytes(rows, V)
    if ws is None:
        ws = workspace(need, dev)
    ws_bytes = _need_ws(ws, need)
    _same_device(logits, ws, *out.values())
    args = (rows, V, dt, _ptr(logits), float(temperature), int(top_k), float(top_p),
            _ptr(out["kept_ids"]), _ptr(out["kept_probs"]), _ptr(out["n_kept"]), _ptr(ws),
            ws_bytes, _stream(stream))
    fn = load().spec_sampling_filter
    keep = (logits, out, ws)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_sampling_filter")

    return enqueue, out


def sampling_filter(logits, temperature, top_k, top_p, out=None, ws=None, stream=None):
    """Temperature / top-k / top-p processing of logits rows
    (spec_sampling_filter). Returns kept_ids, kept_probs, n_kept."""
    enqueue, out = sampling_filter_call(logits, temperature, top_k, top_p, out, ws, stream)
    enqueue()
    return out


def accept_logits_workspace_bytes(bs, K, V, top_k) -> int:
    return int(load().spec_accept_logits_workspace_bytes(bs, K, V, top_k))


def accept_logits_call(target_logits, draft_logits, draft, u, seq_lens, temperature, top_k,
                       top_p, out=None, ws=None, err=None, stream=None):
    """Checks the arguments of spec_accept_logits once and returns (enqueue,
    out). target_logits [bs, K+1, V], draft_logits [bs, K, V] (float32 or
    bfloat16, the same dtype), draft [bs, K] int32, u [bs, K+1] float32."""
    torch = _torch()
    bs, K1, V = target_logits.shape
    K = K1 - 1
    _need(target_logits, "target_logits")
    dt = _dtype_code(target_logits)
    _need(draft_logits, "draft_logits", target_logits.dtype, (bs, K, V))
    _need(draft, "draft", torch.int32, (bs, K))
    _need(u, "u", torch.float32, (bs, K + 1))
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    _need_err(err)
    dev = target_logits.device
    out = _need_out(out, _accept_outputs(bs, K + 1), dev)
    need = accept_logits_workspace_bytes(bs, K, V, top_k)
    if ws is None:
        ws = workspace(need, dev)
    ws_bytes = _need_ws(ws, need)
    _same_device(target_logits, draft_logits, draft, u, seq_lens, ws, err, *out.values())
    args = (bs, K, V, dt, float(temperature), int(top_k), float(top_p), _ptr(target_logits),
            _ptr(draft_logits), _ptr(draft), _ptr(u), _ptr(seq_lens), _ptr(out["accept_len"]),
            _ptr(out["commit_len"]), _ptr(out["bonus"]), _ptr(out["out_tokens"]),
            _ptr(out["new_seq_lens"]), _ptr(ws), ws_bytes, _ptr(err), _stream(stream))
    fn = load().spec_accept_logits
    keep = (target_logits, draft_logits, draft, u, seq_lens, out, ws, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_accept_logits")

    return enqueue, out


def accept_logits(target_logits, draft_logits, draft, u, seq_lens, temperature, top_k, top_p,
                  out=None, ws=None, err=None, stream=None):
    """Speculative accept on logits under sampling parameters
    (spec_accept_logits). Returns the same dict as accept()."""
    enqueue, out = accept_logits_call(target_logits, draft_logits, draft, u, seq_lens,
                                      temperature, top_k, top_p, out, ws, err, stream)
    enqueue()
    return out


# ------------------------------------------------------- committed prefix
def commit_kv_call(k_pool, v_pool, page_table, seq_lens, accept_len, block, path_nodes=None,
                   freed=None, err=None, stream=None):
    """Checks the arguments of spec_commit_kv once and returns (enqueue,
    freed): k_pool / v_pool are updated in place; freed [bs, block] int32
    receives the released slots. path_nodes [bs, block] int32 (the accepted
    node ids of a tree verify) or None (a linear verify)."""
    torch = _torch()
    num_pages, hkv, P, d = k_pool.shape
    _need(k_pool, "k_pool")
    dt = _dtype_code(k_pool)
    _need(v_pool, "v_pool", k_pool.dtype, (num_pages, hkv, d, P))
    bs = seq_lens.shape[0]
    _need(seq_lens, "seq_lens", torch.int32, (bs,))
    _need(accept_len, "accept_len", torch.int32, (bs,))
    _need_table(page_table, bs)
    _need_err(err)
    if path_nodes is not None:
        _need(path_nodes, "path_nodes", torch.int32, (bs, block))
    if freed is None:
        freed = torch.empty((bs, block), dtype=torch.int32, device=k_pool.device)
    _need(freed, "freed", torch.int32, (bs, block))
    _same_device(k_pool, v_pool, page_table, seq_lens, accept_len, path_nodes, freed, err)
    args = (dt, bs, block, hkv, d, P, page_table.shape[1], num_pages, _ptr(seq_lens),
            _ptr(accept_len), _ptr(path_nodes), _ptr(page_table), _ptr(k_pool), _ptr(v_pool),
            _ptr(freed), _ptr(err), _stream(stream))
    fn = load().spec_commit_kv
    keep = (k_pool, v_pool, page_table, seq_lens, accept_len, path_nodes, freed, err)

    def enqueue():
        _ = keep
        st = fn(*args)
        if st != SPEC_OK:
            _check(st, "spec_commit_kv")

    return enqueue, freed


def commit_kv(k_pool, v_pool, page_table, seq_lens, accept_len, block, path_nodes=None,
              freed=None, err=None, stream=None):
    """Committed prefix after an accept (spec_commit_kv): moves the accepted
    tree path's K/V in place and returns the released slots [bs, block]."""
    enqueue, freed = commit_kv_call(k_pool, v_pool, page_table, seq_lens, accept_len, block,
                                    path_nodes, freed, err, stream)
    enqueue()
    return freed
