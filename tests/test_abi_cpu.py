"""C-ABI checks that need no GPU: the library loads, exports every function
include/d2f.h declares, and rejects bad arguments with the documented status
before anything is launched.  Device pointers here are fake, never touched:
every call below returns from host-side validation."""
import ctypes
import os
import re

import pytest

import block_causal_attention_d2f_amd as d2f
from block_causal_attention_d2f_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "d2f.h")

OK, INVALID, CAPACITY, ORDER, WORKSPACE, HIP, UNSUPPORTED = range(7)
FAKE = ctypes.c_void_p(1 << 20)  # 16-byte aligned, never dereferenced on the host


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libd2f.so not built")
    return d2f.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(d2f_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("d2f_block_attn", "d2f_kv_commit", "d2f_confidence_commit"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.d2f_version() == 100


def test_status_strings(lib):
    for s in range(7):
        assert lib.d2f_status_string(s)
    assert lib.d2f_status_string(99) == b"unknown status"


def desc(**kw):
    base = dict(batch=1, n_heads_q=4, n_heads_kv=2, head_dim=128, block_size=16,
                max_win_blocks=3, cache_capacity=100, dtype=B.D2F_BF16, softmax_scale=0.0)
    base.update(kw)
    return B.make_desc(**base)


def attn(lib, d, prefix, nwin, ws=None, ws_bytes=0, q=FAKE, out=FAKE):
    return lib.d2f_block_attn(ctypes.byref(d) if d is not None else None, q, FAKE, FAKE, FAKE,
                              FAKE, B._i32_array(prefix), B._i32_array(nwin), out, None, ws,
                              ws_bytes, None)


def ws_size(lib, d, prefix, nwin):
    out = ctypes.c_size_t(123)
    st = lib.d2f_block_attn_workspace_size(ctypes.byref(d), B._i32_array(prefix),
                                           B._i32_array(nwin), ctypes.byref(out))
    return st, out.value


def test_attention_argument_errors(lib):
    assert lib.d2f_block_attn(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, None, 0,
                              None) == INVALID
    assert attn(lib, desc(n_heads_q=3), [10], [1]) == INVALID          # group mismatch
    assert attn(lib, desc(), [10], [-1]) == INVALID                    # negative window
    assert attn(lib, desc(), [10], [0]) == OK                          # idle request: no work
    assert attn(lib, desc(), [10], [4]) == INVALID                     # > max_win_blocks
    assert attn(lib, desc(), [-1], [1]) == INVALID
    assert attn(lib, desc(), [60], [3]) == CAPACITY                    # 60 + 48 > 100
    assert attn(lib, desc(head_dim=32), [10], [1]) == UNSUPPORTED      # bf16 needs D in {64,128}
    assert attn(lib, desc(dtype=7), [10], [1]) == INVALID
    assert attn(lib, desc(), [10], [1], q=None) == INVALID
    assert attn(lib, desc(), [10], [1], q=ctypes.c_void_p((1 << 20) + 8)) == INVALID  # misaligned
    assert b"aligned" in lib.d2f_last_error()
    assert attn(lib, desc(batch=0), [], []) == OK                      # nothing to do
    assert attn(lib, desc(block_size=0), [1], [1]) == INVALID


def test_workspace_sizing_and_errors(lib):
    # A long prefix is split into key ranges, which needs workspace.
    d = desc(n_heads_q=32, n_heads_kv=32, cache_capacity=40000, max_win_blocks=4)
    st, need = ws_size(lib, d, [32768], [4])
    assert st == OK and need > 0
    assert need % (64 * (128 + 2) * 4) == 0
    assert attn(lib, d, [32768], [4]) == WORKSPACE
    # The size covers the contiguous and the paged call; both plans split
    # this prefix, so a workspace of one split unit's partials is too small.
    assert attn(lib, d, [32768], [4], ws=FAKE, ws_bytes=64 * (128 + 2) * 4) == WORKSPACE
    assert attn(lib, d, [32768], [4], ws=ctypes.c_void_p((1 << 20) + 16), ws_bytes=need) == WORKSPACE
    # A short key list is not split.
    st, need = ws_size(lib, desc(), [0], [1])
    assert st == OK and need == 0
    st, _ = ws_size(lib, desc(), [90], [1])
    assert st == CAPACITY


def kv(lib, d, prefix, request=0, block=0, layers=1, stride=0):
    pl = B._i32_array(prefix)
    st = lib.d2f_kv_commit(ctypes.byref(d), layers, FAKE, FAKE, stride, FAKE, FAKE, stride,
                           request, block, pl, None, None)
    return st, list(pl)[:len(prefix)]


def test_kv_commit_errors(lib):
    d = desc(batch=2, cache_capacity=64)
    assert kv(lib, d, [10, 10], block=1) == (ORDER, [10, 10])
    assert kv(lib, d, [10, 50], request=1) == (CAPACITY, [10, 50])   # 50 + 16 > 64
    assert kv(lib, d, [10, 10], request=2)[0] == INVALID
    assert kv(lib, d, [10, 10], layers=0)[0] == INVALID
    assert kv(lib, d, [10, 10], layers=2, stride=5)[0] == INVALID   # stride below one layer
    assert b"strides" in lib.d2f_last_error()


def commit(lib, rows, vocab, bsz, k_aggr=1, ws=FAKE, ws_bytes=1 << 30, ld=None, tau=0.9):
    return lib.d2f_confidence_commit(FAKE, vocab if ld is None else ld, rows, vocab, FAKE, FAKE,
                                     FAKE, bsz, ctypes.c_float(tau), k_aggr, 0, None, None, FAKE,
                                     FAKE, ws, ws_bytes, None)


def test_confidence_commit_errors(lib):
    assert commit(lib, 30, 100, 16) == INVALID          # rows not a multiple of B
    assert commit(lib, 32, 100, 16, k_aggr=-1) == INVALID
    assert commit(lib, 32, 100, 16, ld=50) == INVALID   # ld < vocab
    assert commit(lib, 32, 0, 16) == INVALID
    assert commit(lib, 2048, 100, 2048) == UNSUPPORTED  # block larger than one workgroup holds
    assert commit(lib, 32, 100, 16, tau=float("nan")) == INVALID
    out = ctypes.c_size_t(0)
    assert lib.d2f_confidence_commit_workspace_size(32, 126464, ctypes.byref(out)) == OK
    # 16 chunks of 8192 logits, 16 B each, then the early commit's two words per row
    assert out.value == 32 * 16 * 16 + 2 * 32 * 4
    assert commit(lib, 32, 126464, 16, ws_bytes=out.value - 1) == WORKSPACE
    assert commit(lib, 32, 126464, 16, ws=None) == WORKSPACE
    assert commit(lib, 0, 126464, 16) == OK             # nothing to do


def advance(lib, d, params, states, prefix, layers=1, stride=0, null_tokens=False):
    n = max(1, len(states))
    arr = (B.WindowState * n)(*states)
    pl = (ctypes.c_int32 * n)(*prefix)
    pers = (ctypes.c_int32 * n)()
    app = (ctypes.c_int32 * n)()
    st = lib.d2f_decode_advance(ctypes.byref(d), layers, FAKE, FAKE, stride, FAKE, FAKE, stride,
                                ctypes.byref(params) if params is not None else None, arr, pl,
                                None, FAKE, FAKE, None if null_tokens else FAKE, FAKE, FAKE, 7,
                                pers, app, None)
    return st, [arr[i].n_win for i in range(len(states))], list(pl)[:len(prefix)]


def test_decode_advance_errors(lib):
    """Argument errors return before the one device transfer; the host state
    stays as it was."""
    d = desc(batch=2, max_win_blocks=3, block_size=16, cache_capacity=200)
    good = B.WindowParams(16, 3, 4, 0.25, 0.75)
    s = B.WindowState()
    assert lib.d2f_window_init(ctypes.byref(good), ctypes.byref(s)) == OK
    # params disagree with the desc on block size / window blocks
    assert advance(lib, d, B.WindowParams(8, 3, 4, 0.25, 0.75), [s, s], [0, 0])[0] == INVALID
    assert advance(lib, d, B.WindowParams(16, 2, 4, 0.25, 0.75), [s, s], [0, 0])[0] == INVALID
    assert b"differ" in lib.d2f_last_error()
    assert advance(lib, d, None, [s, s], [0, 0])[0] == INVALID
    assert advance(lib, d, good, [s, s], [0, 0], null_tokens=True)[0] == INVALID
    assert advance(lib, d, good, [s, s], [0, 0], layers=0)[0] == INVALID
    assert advance(lib, d, good, [s, s], [0, 0], layers=2, stride=5)[0] == INVALID
    assert advance(lib, d, good, [s, s], [-1, 0])[0] == INVALID
    bad = B.WindowState()
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(s), ctypes.sizeof(s))
    bad.started = 3                     # first + n_win != started
    assert advance(lib, d, good, [s, bad], [0, 0]) == (INVALID, [1, 1], [0, 0])
    assert b"inconsistent" in lib.d2f_last_error()
    # an empty batch is a no-op
    assert advance(lib, desc(batch=0, max_win_blocks=3), good, [], [])[0] == OK


def commit_ex(lib, measure, early=None, group=0, rows=32, vocab=100, bsz=16):
    return lib.d2f_confidence_commit_ex(FAKE, vocab, rows, vocab, FAKE, FAKE, FAKE, bsz, measure,
                                        ctypes.c_float(0.9), 1, 0, early, group, None, None, FAKE,
                                        FAKE, FAKE, 1 << 30, None)


def test_confidence_commit_ex_errors(lib):
    assert commit_ex(lib, 4) == INVALID                              # unknown measure
    assert commit_ex(lib, -1) == INVALID
    assert commit_ex(lib, 2, early=FAKE) == INVALID                  # entropy keeps no gap
    assert b"gap" in lib.d2f_last_error()
    assert commit_ex(lib, 3, early=FAKE, group=-1) == INVALID
    assert commit_ex(lib, 1, rows=30) == INVALID                     # rows not a multiple of B
    assert commit_ex(lib, 3, rows=0) == OK                           # nothing to do


def test_prophet_threshold_steps(lib):
    f = lib.d2f_prophet_threshold
    got = [f(ctypes.c_float(p)) for p in (-1.0, 0.0, 0.3, 0.34, 0.66, 0.67, 1.0, 2.0)]
    assert got == [7.5, 7.5, 7.5, 5.0, 5.0, 2.5, 2.5, 2.5]


def paged(lib, d, prefix, nwin, table_stride=8, n_pages=16, pt=FAKE, wp=FAKE):
    n = max(1, len(prefix))
    return lib.d2f_block_attn_paged(ctypes.byref(d), FAKE, FAKE, FAKE, n_pages, pt, table_stride,
                                    wp, (ctypes.c_int32 * n)(*prefix), (ctypes.c_int32 * n)(*nwin),
                                    FAKE, None, FAKE, 1 << 30, None)


def test_paged_attention_errors(lib):
    assert paged(lib, desc(dtype=B.D2F_F32), [16], [1]) == UNSUPPORTED     # bf16 only
    assert paged(lib, desc(block_size=12), [24], [1]) == UNSUPPORTED       # not a power of two
    assert paged(lib, desc(block_size=4), [8], [1]) == UNSUPPORTED         # below 8
    assert paged(lib, desc(), [24], [1]) == INVALID                        # not whole blocks
    assert b"whole number of blocks" in lib.d2f_last_error()
    assert paged(lib, desc(), [160], [1], table_stride=8) == CAPACITY      # 10 blocks > 8 slots
    assert paged(lib, desc(), [16], [4]) == INVALID                        # > max_win_blocks
    assert paged(lib, desc(), [16], [1], pt=None) == INVALID               # table missing
    assert paged(lib, desc(), [16], [1], n_pages=0) == INVALID
    assert paged(lib, desc(batch=0), [], []) == OK


def test_paged_persist_errors(lib):
    d = desc(batch=2)
    pl = (ctypes.c_int32 * 2)(16, 24)
    assert lib.d2f_kv_commit_paged(ctypes.byref(d), FAKE, 4, FAKE, 1, pl, None, None) == INVALID
    assert lib.d2f_kv_commit_paged(ctypes.byref(d), FAKE, 1, FAKE, 0, pl, None, None) == CAPACITY
    assert lib.d2f_kv_commit_paged(ctypes.byref(d), FAKE, 4, FAKE, 2, pl, None, None) == INVALID
    assert list(pl) == [16, 24]
