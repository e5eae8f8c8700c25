"""fp64 oracle: block-causal attention of the active window over a frozen cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages say so:

* [D2F-wiki] section "블록 단위 인과 어텐션" (block-wise causal attention): the
  output sequence is cut into blocks of a fixed size; inside a block every
  token attends to every other token of that block (both directions), and
  between blocks a block attends only to blocks before it.  Because finished
  blocks' K/V no longer change, they are kept in an ordinary KV cache.
* [D2F-wiki] section "인터블록 병렬 디코딩" and [D2F-review] section "쉽게
  이해하기": later blocks are predicted while earlier ones are still only
  partly denoised.  Reading taken here: a window block attends to every
  earlier window block, whatever its state, and to the whole cache.
* The cache holds the prompt and the completed blocks and is visible to every
  window token ([D2F-wiki] "블록 단위 인과 어텐션"; the window sits after the
  cache).  Block boundaries inside the window are counted from the window's
  first token, so the cache length need not be a multiple of the block size.

Softmax scale: 1/sqrt(head_dim) unless given (the pages are silent; this is
the usual scaled dot-product attention).  Grouped query heads: query head h
reads KV head h // (n_heads_q // n_heads_kv).  LSE is the natural-log
normaliser m + ln(sum exp(s - m)).
"""
import numpy as np

from .common import as_f64


def visible(prefix_len: int, win_rows: int, block_size: int) -> np.ndarray:
    """Boolean [win_rows, prefix_len + win_rows]: may window row i see key j?

    Keys are the cache (j < prefix_len) followed by the window.  A cached key
    is always visible; window key j is visible to window row i when its block
    index (j - prefix_len) // block_size is not after row i's block
    i // block_size.
    """
    P, W, B = int(prefix_len), int(win_rows), int(block_size)
    i = np.arange(W)[:, None]
    j = np.arange(P + W)[None, :]
    in_cache = j < P
    key_block = (j - P) // B
    row_block = i // B
    return in_cache | (key_block <= row_block)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray, scale: float):
    """Masked softmax attention of rows q [W, D] over keys k, v [N, D].

    Returns (out [W, D], lse [W]) in float64.  Every row must see >= 1 key.
    """
    s = scale * (q @ k.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    out = (e @ v) / l[:, None]
    return out, m + np.log(l)


def block_attn(q, k_cache, v_cache, k_win, v_win, prefix_len, n_win_blocks, block_size,
               scale=None, pairs=None):
    """Window attention for a batch.

    q        [nb][Hq][Wmax][D]     k_win, v_win [nb][Hkv][Wmax][D]
    k_cache, v_cache [nb][Hkv][cap][D]
    prefix_len[b], n_win_blocks[b]: host lists.

    Returns (out [nb][Hq][Wmax][D], lse [nb][Hq][Wmax]) as float64; rows at or
    past n_win_blocks[b] * block_size are NaN (they are not part of the step).
    ``pairs`` optionally restricts the work to a list of (b, h); the other
    heads are left NaN.
    """
    q = as_f64(q)
    nb, hq, wmax, d = q.shape
    hkv = k_cache.shape[1]
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.full((nb, hq, wmax, d), np.nan)
    lse = np.full((nb, hq, wmax), np.nan)
    if pairs is None:
        pairs = [(b, h) for b in range(nb) for h in range(hq)]
    cache_f64 = {}
    for b, h in pairs:
        g = h // group
        P = int(prefix_len[b])
        W = int(n_win_blocks[b]) * int(block_size)
        if W == 0:
            continue  # an idle request has no window rows, hence no outputs
        key = (b, g)
        if key not in cache_f64:
            kk = np.concatenate([as_f64(k_cache[b, g, :P]), as_f64(k_win[b, g, :W])], axis=0)
            vv = np.concatenate([as_f64(v_cache[b, g, :P]), as_f64(v_win[b, g, :W])], axis=0)
            cache_f64 = {key: (kk, vv)}  # keep one KV head resident at a time
        kk, vv = cache_f64[key]
        o, l = attend(q[b, h, :W], kk, vv, visible(P, W, block_size), scale)
        out[b, h, :W] = o
        lse[b, h, :W] = l
    return out, lse


def gather_pages(pages, table_row, n_blocks):
    """The rows of the first n_blocks pages listed in table_row, in order:
    pages [n_pages][Hkv][B][D] -> [Hkv][n_blocks * B][D] (float64)."""
    pages = as_f64(pages)
    hkv, B, d = pages.shape[1:]
    if n_blocks == 0:
        return np.zeros((hkv, 0, d))
    ids = [int(i) for i in np.asarray(table_row)[:n_blocks]]
    return np.concatenate([pages[i] for i in ids], axis=1)


def block_attn_paged(q, k_pages, v_pages, page_table, win_pages, prefix_len, n_win_blocks,
                     block_size, scale=None, pairs=None):
    """Window attention over a paged cache: request b's cache is the pages
    page_table[b][0 .. P/B) and its window block k is page win_pages[b][k]
    ([D2F-wiki] section "운영 관점", KV cache management: completed blocks kept
    in a paged cache).  The keys are gathered into the contiguous layout and
    block_attn applies the definition; rows past the window are NaN."""
    q = as_f64(q)
    nb, hq, wmax, d = q.shape
    B = int(block_size)
    kp, vp = as_f64(k_pages), as_f64(v_pages)
    hkv = kp.shape[1]
    cap = max([int(p) for p in prefix_len] + [0]) + wmax
    kc = np.zeros((nb, hkv, max(cap, 1), d))
    vc = np.zeros_like(kc)
    kw = np.zeros((nb, hkv, wmax, d))
    vw = np.zeros_like(kw)
    pt, wp = np.asarray(page_table), np.asarray(win_pages)
    for b in range(nb):
        P, n = int(prefix_len[b]), int(n_win_blocks[b])
        assert P % B == 0
        kc[b, :, :P] = gather_pages(kp, pt[b] if P else [], P // B)
        vc[b, :, :P] = gather_pages(vp, pt[b] if P else [], P // B)
        kw[b, :, :n * B] = gather_pages(kp, wp[b] if n else [], n)
        vw[b, :, :n * B] = gather_pages(vp, wp[b] if n else [], n)
    return block_attn(q, kc, vc, kw, vw, prefix_len, n_win_blocks, B, scale=scale, pairs=pairs)


def attn_range(q, k_cache, v_cache, key_lo, key_hi, n_win_blocks, block_size, scale=None):
    """The window's query rows attend to cache keys [key_lo[b], key_hi[b])
    only, all of them visible ([dLLM-survey] section "FlashBlock: 블록 외부
    어텐션 캐싱": the part of the attention outside a block).  Returns (out,
    lse) as block_attn does; rows past the window, and requests with an empty
    range, are NaN."""
    q = as_f64(q)
    nb, hq, wmax, d = q.shape
    kc, vc = as_f64(k_cache), as_f64(v_cache)
    group = hq // kc.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.full((nb, hq, wmax, d), np.nan)
    lse = np.full((nb, hq, wmax), np.nan)
    for b in range(nb):
        lo, hi, W = int(key_lo[b]), int(key_hi[b]), int(n_win_blocks[b]) * int(block_size)
        if hi <= lo or W == 0:
            continue
        for h in range(hq):
            kk, vv = kc[b, h // group, lo:hi], vc[b, h // group, lo:hi]
            o, l = attend(q[b, h, :W], kk, vv, np.ones((W, hi - lo), bool), scale)
            out[b, h, :W] = o
            lse[b, h, :W] = l
    return out, lse


def combine(out_a, lse_a, out_b, lse_b):
    """Joint softmax attention of two disjoint key sets from the two parts:
    L = log(e^L_a + e^L_b), O = O_a e^(L_a - L) + O_b e^(L_b - L) (the log-space
    composition of [dLLM-survey] "FlashBlock"); a part with L = -inf has no keys
    and weight 0."""
    oa, ob = as_f64(out_a), as_f64(out_b)
    la, lb = as_f64(lse_a), as_f64(lse_b)
    with np.errstate(invalid="ignore"):
        L = np.logaddexp(la, lb)
        wa = np.where(np.isneginf(la), 0.0, np.exp(la - L))
        wb = np.where(np.isneginf(lb), 0.0, np.exp(lb - L))
    out = np.where(np.isneginf(la)[..., None], 0.0, oa) * wa[..., None] + \
        np.where(np.isneginf(lb)[..., None], 0.0, ob) * wb[..., None]
    return out, L
