"""Pins of the paged-cache oracle: the gather written against the contiguous
layout it must reproduce (random page permutations give bit-identical fp64
results), and the paged persist (a table update) against the contiguous
append plus the exact-reuse property."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import kv_cache as OK


def scatter(shape, x, seed):
    """Put a contiguous cache/window into randomly numbered pages."""
    g = np.random.default_rng(seed)
    B, nb = shape.block_size, shape.batch
    kc, vc = np.asarray(x["k_cache"], np.float64), np.asarray(x["v_cache"], np.float64)
    kw, vw = np.asarray(x["k_win"], np.float64), np.asarray(x["v_win"], np.float64)
    hkv, d = kc.shape[1], kc.shape[3]
    need = sum(p // B for p in shape.prefix_len) + sum(shape.n_win_blocks)
    n_pages = need + 5
    perm = list(g.permutation(n_pages))
    kp = np.full((n_pages, hkv, B, d), np.nan)
    vp = np.full_like(kp, np.nan)
    ts = max(p // B for p in shape.prefix_len) + 2
    pt = np.full((nb, ts), -1, np.int32)
    wp = np.full((nb, shape.max_win_blocks), -1, np.int32)
    for b in range(nb):
        for i in range(shape.prefix_len[b] // B):
            pg = perm.pop()
            pt[b, i] = pg
            kp[pg], vp[pg] = kc[b, :, i * B:(i + 1) * B], vc[b, :, i * B:(i + 1) * B]
        for k in range(shape.n_win_blocks[b]):
            pg = perm.pop()
            wp[b, k] = pg
            kp[pg], vp[pg] = kw[b, :, k * B:(k + 1) * B], vw[b, :, k * B:(k + 1) * B]
    return kp, vp, pt, wp


@pytest.mark.parametrize("case", [
    (1, 4, 2, 16, 8, [48], [3]),
    (3, 6, 3, 8, 16, [32, 0, 64], [2, 1, 3]),
    (2, 2, 2, 8, 8, [16, 8], [0, 2]),        # an idle request
])
def test_paged_gather_equals_contiguous(case):
    nb, hq, hkv, d, B, prefix, nwin = case
    sh = W.make_shape(nb, hq, hkv, d, B, prefix, nwin, dtype="f32", max_win_blocks=max(nwin))
    x = W.attn_inputs(sh, seed=3)
    kp, vp, pt, wp = scatter(sh, x, seed=4)
    o1, l1 = OA.block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], prefix,
                           nwin, B)
    o2, l2 = OA.block_attn_paged(x["q"], kp, vp, pt, wp, prefix, nwin, B)
    assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(l1, l2, equal_nan=True)


def test_paged_persist_is_the_contiguous_append():
    sh = W.make_shape(2, 4, 2, 8, 8, [16, 8], [3, 2], dtype="f32", extra_capacity=16)
    x = W.attn_inputs(sh, seed=5)
    kp, vp, pt, wp = scatter(sh, x, seed=6)
    first = wp[1, 0]
    pt2, wp2, p2 = OK.kv_commit_paged(pt, wp, sh.prefix_len, 1, 8)
    assert p2 == [16, 16] and pt2[1, 1] == first and list(wp2[1]) == [wp[1, 1], wp[1, 2], -1]
    assert np.array_equal(pt2[0], pt[0]) and np.array_equal(wp2[0], wp[0])
    # the same step on the contiguous layout
    k2, v2, pc = OK.kv_commit(x["k_cache"], x["v_cache"], x["k_win"], x["v_win"],
                              sh.prefix_len, 1, 8)
    assert pc == p2
    kw2 = OK.drop_oldest_block(x["k_win"], 1, 8)
    vw2 = OK.drop_oldest_block(x["v_win"], 1, 8)
    nwin2 = [3, 1]
    o1, l1 = OA.block_attn(x["q"], k2, v2, kw2, vw2, pc, nwin2, 8)
    o2, l2 = OA.block_attn_paged(x["q"], kp, vp, pt2, wp2, p2, nwin2, 8)
    assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(l1, l2, equal_nan=True)
    # exact reuse: request 1's surviving block (old window rows 8..15, queried
    # with the same q rows) sees the same keys in the same order
    o0, l0 = OA.block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"],
                           sh.prefix_len, sh.n_win_blocks, 8)
    q2 = np.asarray(x["q"]).astype(np.float64)
    q2[1, :, 0:8] = q2[1, :, 8:16]
    o3, l3 = OA.block_attn_paged(q2, kp, vp, pt2, wp2, p2, nwin2, 8)
    assert np.array_equal(o0[1, :, 8:16], o3[1, :, 0:8])
    assert np.array_equal(l0[1, :, 8:16], l3[1, :, 0:8])


def test_paged_persist_errors():
    pt = np.zeros((1, 2), np.int32)
    wp = np.zeros((1, 2), np.int32)
    with pytest.raises(ValueError):
        OK.kv_commit_paged(pt, wp, [12], 0, 8)    # not whole blocks
    with pytest.raises(ValueError):
        OK.kv_commit_paged(pt, wp, [16], 0, 8)    # table full
