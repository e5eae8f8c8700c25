"""Oracle for the KV append (a plain slice copy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[D2F-wiki] section "블록 단위 인과 어텐션": a completed block's K/V never change,
so they go into an ordinary KV cache.  Section "KV 캐시 관리 방식" (KV cache
management): the completion of a block is the signal to make its cache
entries permanent.  Reading taken: only the oldest window block is appended,
so the cache stays one contiguous prefix; its K/V rows are copied unchanged
to cache slots [P, P + B) and the prefix length grows by B.
"""
import numpy as np


def kv_commit(k_cache, v_cache, k_win, v_win, prefix_len, request, block_size):
    """Return (k_cache', v_cache', prefix_len') after appending window block 0
    of ``request`` (arrays [nb][Hkv][cap][D] and [nb][Hkv][Wmax][D])."""
    k2 = np.asarray(k_cache).copy()
    v2 = np.asarray(v_cache).copy()
    p = list(int(x) for x in prefix_len)
    b, B = int(request), int(block_size)
    P = p[b]
    if P + B > k2.shape[2]:
        raise ValueError("cache capacity exceeded")
    k2[b, :, P:P + B] = np.asarray(k_win)[b, :, 0:B]
    v2[b, :, P:P + B] = np.asarray(v_win)[b, :, 0:B]
    p[b] = P + B
    return k2, v2, p


def drop_oldest_block(x, request, block_size):
    """Window array with request's block 0 removed and the rest moved up one
    block (the state of the window after its oldest block left it)."""
    y = np.asarray(x).copy()
    b, B = int(request), int(block_size)
    y[b, :, :-B] = np.asarray(x)[b, :, B:]
    y[b, :, -B:] = np.nan
    return y


def kv_commit_paged(page_table, win_pages, prefix_len, request, block_size):
    """Paged persist ([D2F-wiki] section "운영 관점", KV cache management: block
    completion is the signal that makes its entries permanent): the page of
    request's oldest window block becomes cache page P / B; the window's page
    list moves up by one and its last entry becomes -1; P grows by B.
    Returns (page_table', win_pages', prefix_len')."""
    pt = np.asarray(page_table).copy()
    wp = np.asarray(win_pages).copy()
    p = [int(x) for x in prefix_len]
    b, B = int(request), int(block_size)
    P = p[b]
    if P % B or P // B >= pt.shape[1]:
        raise ValueError("prefix not whole blocks, or page table full")
    pt[b, P // B] = wp[b, 0]
    wp[b, :-1] = np.asarray(win_pages)[b, 1:]
    wp[b, -1] = -1
    p[b] = P + B
    return pt, wp, p
