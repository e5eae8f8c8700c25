"""ctypes binding over libd2f.so (argument marshalling only).

Every function here forwards to the C entry point of the same name declared in
include/d2f.h.  Torch tensors supply device memory and the current HIP stream;
all arithmetic runs in the library's HIP kernels.  There is no fallback: if
the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# D2F_LIB selects another build of the library (the host-sanitized one).
LIB_PATH = os.environ.get("D2F_LIB") or os.path.join(_PKG, "libd2f.so")

D2F_OK = 0
STATUS_NAMES = {0: "D2F_OK", 1: "D2F_ERR_INVALID_ARG", 2: "D2F_ERR_CAPACITY",
                3: "D2F_ERR_ORDER", 4: "D2F_ERR_WORKSPACE", 5: "D2F_ERR_HIP",
                6: "D2F_ERR_UNSUPPORTED"}
D2F_F32, D2F_BF16 = 0, 1
MASKED, COMMITTED = 0, 1
CONSERVATIVE, AGGRESSIVE = 0, 1

EXPORTS = ("d2f_block_attn_workspace_size", "d2f_block_attn", "d2f_kv_commit",
           "d2f_confidence_commit_workspace_size", "d2f_confidence_commit",
           "d2f_confidence_commit_ex", "d2f_prophet_threshold",
           "d2f_block_attn_paged", "d2f_kv_commit_paged", "d2f_decode_advance_paged",
           "d2f_block_attn_range_workspace_size", "d2f_block_attn_range", "d2f_attn_combine",
           "d2f_window_init", "d2f_window_after_commit", "d2f_decode_advance",
           "d2f_status_string", "d2f_last_error", "d2f_version",
           "d2f_confidence_commit_noalloc")
MAX_WINDOW = 64  # D2F_MAX_WINDOW
MEASURES = {"maxprob": 0, "margin": 1, "neg_entropy": 2, "logit_gap": 3}  # d2f_conf_measure_t


class D2FError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_heads_q", ctypes.c_int32),
                ("n_heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_win_blocks", ctypes.c_int32),
                ("cache_capacity", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float)]


class WindowParams(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("max_win_blocks", ctypes.c_int32),
                ("total_blocks", ctypes.c_int32), ("tau_add", ctypes.c_float),
                ("tau_act", ctypes.c_float)]


class WindowState(ctypes.Structure):
    _fields_ = [("first", ctypes.c_int32), ("n_win", ctypes.c_int32),
                ("started", ctypes.c_int32), ("persisted", ctypes.c_int32),
                ("committed", ctypes.c_int32 * MAX_WINDOW),
                ("phase", ctypes.c_uint8 * MAX_WINDOW)]


_lib = None
_vp, _i32, _i64, _f32, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                              ctypes.c_size_t)
_pi32 = ctypes.POINTER(ctypes.c_int32)


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libd2f.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(f"{p} is missing: build it with "
                                "`python -m block_causal_attention_d2f_amd.build`")
    lib = ctypes.CDLL(p)
    pdesc = ctypes.POINTER(AttnDesc)
    sig = {
        "d2f_block_attn_workspace_size": (_i32, [pdesc, _pi32, _pi32, ctypes.POINTER(_sz)]),
        "d2f_block_attn": (_i32, [pdesc, _vp, _vp, _vp, _vp, _vp, _pi32, _pi32, _vp, _vp, _vp,
                                  _sz, _vp]),
        "d2f_kv_commit": (_i32, [pdesc, _i32, _vp, _vp, _i64, _vp, _vp, _i64, _i32, _i32, _pi32,
                                 _vp, _vp]),
        "d2f_confidence_commit_workspace_size": (_i32, [_i32, _i32, ctypes.POINTER(_sz)]),
        "d2f_confidence_commit": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _i32, _f32, _i32,
                                         _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
        "d2f_confidence_commit_ex": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _i32, _i32,
                                            _f32, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _vp,
                                            _vp, _sz, _vp]),
        "d2f_prophet_threshold": (_f32, [_f32]),
        "d2f_block_attn_paged": (_i32, [pdesc, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _pi32, _pi32,
                                        _vp, _vp, _vp, _sz, _vp]),
        "d2f_kv_commit_paged": (_i32, [pdesc, _vp, _i32, _vp, _i32, _pi32, _vp, _vp]),
        "d2f_block_attn_range_workspace_size": (_i32, [pdesc, _pi32, _pi32, _pi32,
                                                       ctypes.POINTER(_sz)]),
        "d2f_block_attn_range": (_i32, [pdesc, _vp, _vp, _vp, _pi32, _pi32, _pi32, _vp, _vp,
                                        _vp, _sz, _vp]),
        "d2f_attn_combine": (_i32, [pdesc, _vp, _vp, _vp, _vp, _vp, _vp, _pi32, _vp]),
        "d2f_decode_advance_paged": (_i32, [pdesc, _vp, _i32, _vp, _pi32,
                                            ctypes.POINTER(WindowParams),
                                            ctypes.POINTER(WindowState), _pi32, _vp, _vp, _vp,
                                            _vp, _vp, _vp, _i32, _pi32, _pi32, _vp]),
        "d2f_window_init": (_i32, [ctypes.POINTER(WindowParams), ctypes.POINTER(WindowState)]),
        "d2f_window_after_commit": (_i32, [ctypes.POINTER(WindowParams),
                                           ctypes.POINTER(WindowState), _pi32, _pi32, _pi32]),
        "d2f_decode_advance": (_i32, [pdesc, _i32, _vp, _vp, _i64, _vp, _vp, _i64,
                                      ctypes.POINTER(WindowParams), ctypes.POINTER(WindowState),
                                      _pi32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _pi32, _pi32,
                                      _vp]),
        "d2f_confidence_commit_noalloc": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _i32,
                                                 _f32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
        "d2f_status_string": (ctypes.c_char_p, [_i32]),
        "d2f_last_error": (ctypes.c_char_p, []),
        "d2f_version": (_i32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    if path is None:
        _lib = lib
    return lib


def _check(st: int):
    if st != D2F_OK:
        lib = load()
        raise D2FError(st, lib.d2f_last_error().decode(errors="replace"))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _i32_array(xs: Sequence[int]):
    return (ctypes.c_int32 * max(1, len(xs)))(*[int(x) for x in xs])


def make_desc(batch, n_heads_q, n_heads_kv, head_dim, block_size, max_win_blocks,
              cache_capacity, dtype, softmax_scale=0.0) -> AttnDesc:
    dt = {torch.float32: D2F_F32, torch.bfloat16: D2F_BF16}.get(dtype, dtype)
    return AttnDesc(int(batch), int(n_heads_q), int(n_heads_kv), int(head_dim), int(block_size),
                    int(max_win_blocks), int(cache_capacity), int(dt), float(softmax_scale))


def _desc_from(q, k_cache, block_size, softmax_scale) -> AttnDesc:
    nb, hq, wmax, d = q.shape
    hkv, cap = k_cache.shape[1], k_cache.shape[2]
    if wmax % block_size:
        raise ValueError("window rows of q must be a multiple of block_size")
    return make_desc(nb, hq, hkv, d, block_size, wmax // block_size, cap, q.dtype, softmax_scale)


def d2f_block_attn_workspace_size(desc: AttnDesc, prefix_len, n_win_blocks) -> int:
    out = ctypes.c_size_t(0)
    _check(load().d2f_block_attn_workspace_size(ctypes.byref(desc), _i32_array(prefix_len),
                                                _i32_array(n_win_blocks), ctypes.byref(out)))
    return int(out.value)


def _contig(name, t, dtype=None, device=None):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def d2f_block_attn(q, k_cache, v_cache, k_win, v_win, prefix_len, n_win_blocks, block_size,
                   out=None, lse=None, want_lse=True, softmax_scale=0.0, workspace=None,
                   stream=None):
    """Block-causal attention of the window over the frozen cache (one layer).

    q [nb][Hq][Wmax][D]; k_cache, v_cache [nb][Hkv][cap][D]; k_win, v_win
    [nb][Hkv][Wmax][D]; prefix_len, n_win_blocks: host sequences of ints.
    Returns (out, lse); lse is None unless want_lse.
    """
    desc = _desc_from(q, k_cache, block_size, softmax_scale)
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("k_win", k_win),
                 ("v_win", v_win)):
        _contig(n, t, q.dtype, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    pl, nw = _i32_array(prefix_len), _i32_array(n_win_blocks)

    def call(ws):
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        return load().d2f_block_attn(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(k_win), _ptr(v_win), pl, nw, _ptr(out), _ptr(lse),
                                     _ptr(ws), nbytes, _stream(stream))
    _call_with_workspace(call, workspace, lambda: d2f_block_attn_workspace_size(
        desc, prefix_len, n_win_blocks), q.device)
    return out, lse


def _call_with_workspace(call, workspace, size, device):
    """Run call(workspace); only if the library reports the workspace too
    small (which it checks before launching anything), size it and run again
    -- so the work plan is made once per call in the common case."""
    st = call(workspace)
    if st == 4:  # D2F_ERR_WORKSPACE
        st = call(torch.empty(max(size(), 256), dtype=torch.uint8, device=device))
    _check(st)


def d2f_block_attn_range(q, k_cache, v_cache, key_lo, key_hi, n_win_blocks, block_size,
                         out=None, lse=None, softmax_scale=0.0, workspace=None, stream=None):
    """Window queries over cache keys [key_lo[b], key_hi[b]) only (see d2f.h).
    Returns (out, lse)."""
    nb, hq, wmax, d = q.shape
    hkv, cap = k_cache.shape[1], k_cache.shape[2]
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _contig(n, t, q.dtype, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    desc = make_desc(nb, hq, hkv, d, block_size, wmax // block_size, cap, q.dtype, softmax_scale)
    lo, hi, nw = _i32_array(key_lo), _i32_array(key_hi), _i32_array(n_win_blocks)

    def call(ws):
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        return load().d2f_block_attn_range(ctypes.byref(desc), _ptr(q), _ptr(k_cache),
                                           _ptr(v_cache), lo, hi, nw, _ptr(out), _ptr(lse),
                                           _ptr(ws), nbytes, _stream(stream))

    def size():
        n = ctypes.c_size_t(0)
        _check(load().d2f_block_attn_range_workspace_size(ctypes.byref(desc), lo, hi, nw,
                                                          ctypes.byref(n)))
        return int(n.value)
    _call_with_workspace(call, workspace, size, q.device)
    return out, lse


def d2f_attn_combine(out_a, lse_a, out_b, lse_b, n_win_blocks, block_size, out=None, lse=None,
                     stream=None):
    """Log-space join of two attention results over disjoint keys (see d2f.h).
    Returns (out, lse); out / lse may be out_a / lse_a."""
    nb, hq, wmax, d = out_a.shape
    for n, t in (("out_a", out_a), ("out_b", out_b)):
        _contig(n, t, out_a.dtype, out_a.device)
    for n, t in (("lse_a", lse_a), ("lse_b", lse_b)):
        _contig(n, t, torch.float32, out_a.device)
    if out is None:
        out = torch.empty_like(out_a)
    if lse is None:
        lse = torch.empty_like(lse_a)
    desc = make_desc(nb, hq, hq, d, block_size, wmax // block_size, 1, out_a.dtype)
    _check(load().d2f_attn_combine(ctypes.byref(desc), _ptr(out_a), _ptr(lse_a), _ptr(out_b),
                                   _ptr(lse_b), _ptr(out), _ptr(lse), _i32_array(n_win_blocks),
                                   _stream(stream)))
    return out, lse


def d2f_kv_commit(k_cache, v_cache, k_win, v_win, prefix_len: list, request: int,
                  block_size: int, block: int = 0, prefix_len_dev=None, stream=None):
    """Append window block `block` (must be 0, the oldest) of `request` to the
    cache.  Accepts one layer ([nb][Hkv][cap][D]) or a stack of layers
    ([L][nb][Hkv][cap][D]).  prefix_len (a Python list) is updated in place."""
    layered = k_cache.dim() == 5
    kc0 = k_cache[0] if layered else k_cache
    kw0 = k_win[0] if layered else k_win
    n_layers = k_cache.shape[0] if layered else 1
    nb, hkv, cap, d = kc0.shape
    wmax = kw0.shape[2]
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_win", k_win), ("v_win", v_win)):
        _contig(n, t, k_cache.dtype, k_cache.device)
    desc = make_desc(nb, hkv, hkv, d, block_size, wmax // block_size, cap, k_cache.dtype)
    pl = _i32_array(prefix_len)
    _check(load().d2f_kv_commit(ctypes.byref(desc), n_layers, _ptr(k_cache), _ptr(v_cache),
                                kc0.numel(), _ptr(k_win), _ptr(v_win), kw0.numel(), int(request),
                                int(block), pl, _ptr(prefix_len_dev), _stream(stream)))
    prefix_len[request] = int(pl[request])
    return prefix_len


def d2f_block_attn_paged(q, k_pages, v_pages, page_table, win_pages, prefix_len, n_win_blocks,
                         out=None, lse=None, want_lse=True, softmax_scale=0.0, workspace=None,
                         stream=None):
    """Block-causal attention over a paged cache (one layer; see d2f.h).

    q [nb][Hq][Wmax][D] bf16; k_pages, v_pages [n_pages][Hkv][B][D] bf16 (one
    page = one block); page_table int32 [nb][table_stride] and win_pages int32
    [nb][Wmax / B] on the device; prefix_len (multiples of B), n_win_blocks:
    host sequences.  Returns (out, lse)."""
    nb, hq, wmax, d = q.shape
    n_pages, hkv, bsz, d2 = k_pages.shape
    if d2 != d or wmax % bsz:
        raise ValueError("page and query shapes disagree")
    for n, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages)):
        _contig(n, t, q.dtype, q.device)
    _contig("page_table", page_table, torch.int32, q.device)
    _contig("win_pages", win_pages, torch.int32, q.device)
    table_stride = page_table.shape[1] if page_table.dim() == 2 else 0
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    cap = table_stride * bsz + wmax
    desc = make_desc(nb, hq, hkv, d, bsz, wmax // bsz, cap, q.dtype, softmax_scale)
    pl, nw = _i32_array(prefix_len), _i32_array(n_win_blocks)

    def call(ws):
        nbytes = 0 if ws is None else ws.numel() * ws.element_size()
        return load().d2f_block_attn_paged(
            ctypes.byref(desc), _ptr(q), _ptr(k_pages), _ptr(v_pages), n_pages, _ptr(page_table),
            table_stride, _ptr(win_pages), pl, nw, _ptr(out), _ptr(lse), _ptr(ws), nbytes,
            _stream(stream))
    _call_with_workspace(call, workspace, lambda: d2f_block_attn_workspace_size(
        desc, prefix_len, n_win_blocks), q.device)
    return out, lse


def d2f_kv_commit_paged(page_table, win_pages, prefix_len: list, request: int, block_size: int,
                        n_heads_kv: int = 1, head_dim: int = 128, prefix_len_dev=None,
                        stream=None):
    """Persist request's oldest window block by moving its page into the page
    table (no copy).  prefix_len (a Python list) is updated in place."""
    nb, table_stride = page_table.shape
    mw = win_pages.shape[1]
    _contig("page_table", page_table, torch.int32, page_table.device)
    _contig("win_pages", win_pages, torch.int32, page_table.device)
    desc = make_desc(nb, n_heads_kv, n_heads_kv, head_dim, block_size, mw,
                     table_stride * block_size, torch.bfloat16)
    pl = _i32_array(prefix_len)
    _check(load().d2f_kv_commit_paged(ctypes.byref(desc), _ptr(page_table), table_stride,
                                      _ptr(win_pages), int(request), pl, _ptr(prefix_len_dev),
                                      _stream(stream)))
    prefix_len[request] = int(pl[request])
    return prefix_len


def d2f_confidence_commit_workspace_size(n_rows: int, vocab: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load().d2f_confidence_commit_workspace_size(int(n_rows), int(vocab),
                                                       ctypes.byref(out)))
    return int(out.value)


def d2f_confidence_commit(logits, mask_state, tokens, block_phase, block_size: int, tau: float,
                          k_aggr: int = 1, mask_token_id: int = 0, conf_out=None,
                          argmax_out=None, n_committed=None, block_complete=None,
                          workspace=None, stream=None, want_conf=True, measure="maxprob",
                          early_gap=None, early_group_blocks: int = 0):
    """One commit pass.  logits [rows][V] fp32 (row stride may exceed V);
    mask_state uint8 [rows] and tokens int32 [rows] are updated in place.
    ``measure``: "maxprob" (d2f_confidence_commit), "margin", "neg_entropy" or
    "logit_gap" (d2f_confidence_commit_ex); ``early_gap``: Prophet's early
    commit thresholds, one per group of ``early_group_blocks`` blocks (a
    float, a sequence or a device float32 tensor), or None.
    Returns dict(n_committed, block_complete, conf, argmax)."""
    rows, vocab = logits.shape
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    if measure not in MEASURES:
        raise ValueError(f"unknown measure {measure!r}")
    dev = logits.device
    _contig("mask_state", mask_state, torch.uint8, dev)
    _contig("tokens", tokens, torch.int32, dev)
    _contig("block_phase", block_phase, torch.uint8, dev)
    n_blocks = rows // block_size if block_size > 0 else 0
    if n_committed is None:
        n_committed = torch.empty(n_blocks, dtype=torch.int32, device=dev)
    if block_complete is None:
        block_complete = torch.empty(n_blocks, dtype=torch.uint8, device=dev)
    if want_conf and conf_out is None:
        conf_out = torch.full((rows,), float("nan"), dtype=torch.float32, device=dev)
    if want_conf and argmax_out is None:
        argmax_out = torch.full((rows,), -1, dtype=torch.int32, device=dev)
    need = d2f_confidence_commit_workspace_size(rows, vocab)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    gb = min(early_group_blocks, n_blocks) if early_group_blocks > 0 else max(n_blocks, 1)
    n_groups = max(1, (n_blocks + gb - 1) // gb)
    if early_gap is not None and not isinstance(early_gap, torch.Tensor):
        vals = [float(early_gap)] * n_groups if isinstance(early_gap, (int, float)) \
            else [float(v) for v in early_gap]
        early_gap = torch.tensor(vals, dtype=torch.float32, device=dev)
    if early_gap is not None:
        _contig("early_gap", early_gap, torch.float32, dev)
        if early_gap.numel() < n_groups:   # the kernels read one threshold per group
            raise ValueError(f"early_gap holds {early_gap.numel()} thresholds for "
                             f"{n_groups} groups")
    args_tail = (_ptr(conf_out), _ptr(argmax_out), _ptr(n_committed), _ptr(block_complete),
                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if measure == "maxprob" and early_gap is None:
        _check(load().d2f_confidence_commit(
            _ptr(logits), logits.stride(0), rows, vocab, _ptr(mask_state), _ptr(tokens),
            _ptr(block_phase), int(block_size), ctypes.c_float(tau), int(k_aggr),
            int(mask_token_id), *args_tail))
    else:
        _check(load().d2f_confidence_commit_ex(
            _ptr(logits), logits.stride(0), rows, vocab, _ptr(mask_state), _ptr(tokens),
            _ptr(block_phase), int(block_size), MEASURES[measure], ctypes.c_float(tau),
            int(k_aggr), int(mask_token_id), _ptr(early_gap), int(early_group_blocks),
            *args_tail))
    return dict(n_committed=n_committed, block_complete=block_complete, conf=conf_out,
                argmax=argmax_out)


NOALLOC_SCRATCH_BYTES = 8 << 20  # D2F_NOALLOC_SCRATCH_BYTES


def d2f_confidence_commit_noalloc(logits, mask_state, tokens, block_phase, block_size: int,
                                  tau: float, k_aggr: int = 1, mask_token_id: int = 0,
                                  conf_out=None, argmax_out=None, n_committed=None,
                                  block_complete=None, stream=None):
    """The commit pass of d2f_confidence_commit without a workspace: the
    library's per-device scratch array holds the partials (see d2f.h).  With
    every output buffer passed in, this call allocates nothing.
    Returns dict(n_committed, block_complete, conf, argmax)."""
    rows, vocab = logits.shape
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    dev = logits.device
    _contig("mask_state", mask_state, torch.uint8, dev)
    _contig("tokens", tokens, torch.int32, dev)
    _contig("block_phase", block_phase, torch.uint8, dev)
    n_blocks = rows // block_size if block_size > 0 else 0
    if n_committed is None:
        n_committed = torch.empty(n_blocks, dtype=torch.int32, device=dev)
    if block_complete is None:
        block_complete = torch.empty(n_blocks, dtype=torch.uint8, device=dev)
    _check(load().d2f_confidence_commit_noalloc(
        _ptr(logits), logits.stride(0), rows, vocab, _ptr(mask_state), _ptr(tokens),
        _ptr(block_phase), int(block_size), ctypes.c_float(tau), int(k_aggr),
        int(mask_token_id), _ptr(conf_out), _ptr(argmax_out), _ptr(n_committed),
        _ptr(block_complete), _stream(stream)))
    return dict(n_committed=n_committed, block_complete=block_complete, conf=conf_out,
                argmax=argmax_out)


def prophet_threshold(progress: float) -> float:
    return float(load().d2f_prophet_threshold(ctypes.c_float(progress)))


def version() -> int:
    return int(load().d2f_version())


class Window:
    """The library's active-window scheduler (host only; see d2f.h)."""

    def __init__(self, block_size: int, max_win_blocks: int, total_blocks: int,
                 tau_add: float, tau_act: float):
        self.params = WindowParams(int(block_size), int(max_win_blocks), int(total_blocks),
                                   float(tau_add), float(tau_act))
        self.state = WindowState()
        _check(load().d2f_window_init(ctypes.byref(self.params), ctypes.byref(self.state)))

    @property
    def first(self) -> int:
        return self.state.first

    @property
    def n_win(self) -> int:
        return self.state.n_win

    @property
    def started(self) -> int:
        return self.state.started

    @property
    def persisted(self) -> int:
        return self.state.persisted

    @property
    def done(self) -> bool:
        return self.state.persisted == self.params.total_blocks

    @property
    def committed(self) -> list:
        return [self.state.committed[k] for k in range(self.state.n_win)]

    @property
    def phase(self) -> list:
        return [self.state.phase[k] for k in range(self.state.n_win)]

    def after_commit(self, n_committed: Sequence[int]):
        """Apply one commit pass; returns (blocks persisted, blocks appended)."""
        p, a = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(load().d2f_window_after_commit(ctypes.byref(self.params), ctypes.byref(self.state),
                                              _i32_array(n_committed), ctypes.byref(p),
                                              ctypes.byref(a)))
        return p.value, a.value


def d2f_decode_advance(k_cache, v_cache, k_win, v_win, windows: Sequence[Window],
                       prefix_len: list, n_committed, mask_state, tokens, block_phase,
                       out_tokens, mask_token_id: int, prefix_len_dev=None, stream=None):
    """The step's bookkeeping after the commit pass (see d2f.h): schedule every
    request's window, append persisted blocks' K/V, slide the slot rows.

    Caches / windows as for d2f_kv_commit (one layer or a [L] stack);
    mask_state uint8 / tokens int32 [batch * Wmax]; block_phase uint8 and
    n_committed int32 [batch * max_win_blocks]; out_tokens int32
    [batch][total_blocks * block_size].  `windows` (one Window per request,
    same parameters) and `prefix_len` are updated in place.  Returns
    (persisted, appended) per request."""
    layered = k_cache.dim() == 5
    kc0 = k_cache[0] if layered else k_cache
    kw0 = k_win[0] if layered else k_win
    n_layers = k_cache.shape[0] if layered else 1
    nb, hkv, cap, d = kc0.shape
    if len(windows) != nb or len(prefix_len) != nb:
        raise ValueError("one window and one prefix length per request")
    params = windows[0].params if nb else None
    for w in windows:
        if (w.params.block_size, w.params.max_win_blocks, w.params.total_blocks,
                w.params.tau_add, w.params.tau_act) != \
                (params.block_size, params.max_win_blocks, params.total_blocks, params.tau_add,
                 params.tau_act):
            raise ValueError("every window must have the same parameters")
    dev = k_cache.device
    for n, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_win", k_win), ("v_win", v_win)):
        _contig(n, t, k_cache.dtype, dev)
    _contig("mask_state", mask_state, torch.uint8, dev)
    _contig("tokens", tokens, torch.int32, dev)
    _contig("block_phase", block_phase, torch.uint8, dev)
    _contig("n_committed", n_committed, torch.int32, dev)
    _contig("out_tokens", out_tokens, torch.int32, dev)
    block_size = params.block_size if nb else 1
    wmax = kw0.shape[2]
    desc = make_desc(nb, hkv, hkv, d, block_size, wmax // block_size, cap, k_cache.dtype)
    if nb and (mask_state.numel() != nb * wmax or tokens.numel() != nb * wmax or
               block_phase.numel() != nb * params.max_win_blocks or
               n_committed.numel() != nb * params.max_win_blocks or
               out_tokens.numel() != nb * params.total_blocks * block_size):
        raise ValueError("slot buffers do not match batch, window and total_blocks")
    states = (WindowState * max(1, nb))()
    for i, w in enumerate(windows):
        states[i] = w.state
    pl = _i32_array(prefix_len)
    pers = (ctypes.c_int32 * max(1, nb))()
    app = (ctypes.c_int32 * max(1, nb))()
    _check(load().d2f_decode_advance(
        ctypes.byref(desc), n_layers, _ptr(k_cache), _ptr(v_cache), kc0.numel(), _ptr(k_win),
        _ptr(v_win), kw0.numel(), ctypes.byref(params) if nb else None, states, pl,
        _ptr(prefix_len_dev), _ptr(n_committed), _ptr(mask_state), _ptr(tokens),
        _ptr(block_phase), _ptr(out_tokens), int(mask_token_id), pers, app, _stream(stream)))
    for i, w in enumerate(windows):
        w.state = states[i]
        prefix_len[i] = int(pl[i])
    return [pers[i] for i in range(nb)], [app[i] for i in range(nb)]


def d2f_decode_advance_paged(page_table, win_pages, new_pages, windows: Sequence[Window],
                             prefix_len: list, n_committed, mask_state, tokens, block_phase,
                             out_tokens, mask_token_id: int, n_heads_kv: int = 1,
                             head_dim: int = 128, prefix_len_dev=None, stream=None):
    """d2f_decode_advance for a paged cache: persisted blocks' pages join
    page_table (no copy); new_pages (host ints, one per request) are taken by
    appended blocks.  windows and prefix_len are updated in place.  Returns
    (persisted, appended) per request."""
    nb, table_stride = page_table.shape
    mw = win_pages.shape[1]
    if len(windows) != nb or len(prefix_len) != nb or len(new_pages) != nb:
        raise ValueError("one window, prefix length and new page per request")
    params = windows[0].params
    dev = page_table.device
    _contig("page_table", page_table, torch.int32, dev)
    _contig("win_pages", win_pages, torch.int32, dev)
    _contig("mask_state", mask_state, torch.uint8, dev)
    _contig("tokens", tokens, torch.int32, dev)
    _contig("block_phase", block_phase, torch.uint8, dev)
    _contig("n_committed", n_committed, torch.int32, dev)
    _contig("out_tokens", out_tokens, torch.int32, dev)
    B = params.block_size
    if (params.max_win_blocks != mw or mask_state.numel() != nb * mw * B or
            out_tokens.numel() != nb * params.total_blocks * B):
        raise ValueError("slot buffers do not match batch, window and total_blocks")
    desc = make_desc(nb, n_heads_kv, n_heads_kv, head_dim, B, mw, table_stride * B,
                     torch.bfloat16)
    states = (WindowState * nb)()
    for i, w in enumerate(windows):
        states[i] = w.state
    pl = _i32_array(prefix_len)
    pers = (ctypes.c_int32 * nb)()
    app = (ctypes.c_int32 * nb)()
    _check(load().d2f_decode_advance_paged(
        ctypes.byref(desc), _ptr(page_table), table_stride, _ptr(win_pages),
        _i32_array(new_pages), ctypes.byref(params), states, pl, _ptr(prefix_len_dev),
        _ptr(n_committed), _ptr(mask_state), _ptr(tokens), _ptr(block_phase), _ptr(out_tokens),
        int(mask_token_id), pers, app, _stream(stream)))
    for i, w in enumerate(windows):
        w.state = states[i]
        prefix_len[i] = int(pl[i])
    return [pers[i] for i in range(nb)], [app[i] for i in range(nb)]

