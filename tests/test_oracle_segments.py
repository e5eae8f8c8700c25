"""Pins of the segment oracle: attention over a cache key range joined with
the window-only attention reproduces the full block-causal attention
(log-space composition is exact), for any cut of the cache; the join is
associative and a part with no keys is its identity.  Also the accuracy
study of reusing a stale outside part (an approximation in D2F)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as OA


def parts(sh, x, cuts):
    """Full attention of sh assembled from cache ranges between the cuts and
    the window-only part."""
    nb = sh.batch
    zero = [0] * nb
    acc_o, acc_l = OA.block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], zero,
                                 sh.n_win_blocks, sh.block_size)
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        lo_b = [min(lo, p) for p in sh.prefix_len]
        hi_b = [min(hi, p) for p in sh.prefix_len]
        o, l = OA.attn_range(x["q"], x["k_cache"], x["v_cache"], lo_b, hi_b, sh.n_win_blocks,
                             sh.block_size)
        empty = np.array([h <= l_ for l_, h in zip(lo_b, hi_b)])
        o[empty], l[empty] = 0.0, -np.inf   # an empty part: no keys
        acc_o, acc_l = OA.combine(acc_o, acc_l, o, l)
    return acc_o, acc_l


@pytest.mark.parametrize("case", [
    (1, 2, 2, 16, 8, [40], [3], [0, 40]),
    (2, 4, 2, 8, 4, [37, 12], [2, 3], [0, 5, 20, 37]),   # uneven cuts, GQA
    (1, 2, 1, 8, 16, [0], [2], [0, 0]),                  # empty cache
])
def test_composition_is_exact(case):
    nb, hq, hkv, d, B, prefix, nwin, cuts = case
    sh = W.make_shape(nb, hq, hkv, d, B, prefix, nwin, dtype="f32")
    x = W.attn_inputs(sh, seed=2)
    full_o, full_l = OA.block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"],
                                   prefix, nwin, B)
    o, l = parts(sh, x, cuts)
    for b in range(nb):
        Wb = nwin[b] * B
        np.testing.assert_allclose(o[b, :, :Wb], full_o[b, :, :Wb], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l[b, :, :Wb], full_l[b, :, :Wb], rtol=0, atol=1e-12)


def test_join_identity_and_associativity():
    g = np.random.default_rng(1)
    o = [g.normal(size=(1, 2, 5, 4)) for _ in range(3)]
    l = [g.normal(size=(1, 2, 5)) for _ in range(3)]
    a1 = OA.combine(*OA.combine(o[0], l[0], o[1], l[1]), o[2], l[2])
    a2 = OA.combine(o[0], l[0], *OA.combine(o[1], l[1], o[2], l[2]))
    np.testing.assert_allclose(a1[0], a2[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a1[1], a2[1], rtol=0, atol=1e-14)
    e_o, e_l = np.full_like(o[0], np.nan), np.full_like(l[0], -np.inf)
    i1 = OA.combine(o[0], l[0], e_o, e_l)
    assert np.array_equal(i1[0], o[0]) and np.array_equal(i1[1], l[0])


def test_range_against_brute_force():
    sh = W.make_shape(1, 2, 1, 8, 4, [30], [2], dtype="f32")
    x = W.attn_inputs(sh, seed=4)
    o, l = OA.attn_range(x["q"], x["k_cache"], x["v_cache"], [7], [19], [2], 4)
    q = np.asarray(x["q"], np.float64)
    k = np.asarray(x["k_cache"], np.float64)[0, 0, 7:19]
    v = np.asarray(x["v_cache"], np.float64)[0, 0, 7:19]
    for h in range(2):
        for i in range(8):
            s = [float(np.dot(q[0, h, i], kk)) / np.sqrt(8) for kk in k]
            m = max(s)
            w = [np.exp(t - m) for t in s]
            assert abs(l[0, h, i] - (m + np.log(sum(w)))) < 1e-13
            want = sum(wi * vv for wi, vv in zip(w, v)) / sum(w)
            np.testing.assert_allclose(o[0, h, i], want, rtol=0, atol=1e-13)


def reuse_error(eps, seed=0):
    """Error of the outside part computed with the queries of an earlier
    step (the window's queries drift by eps * N(0, 1) per entry) against the
    exact attention with the current queries (LLaDA-like heads, 512-key cache)."""
    sh = W.make_shape(1, 4, 4, 64, 16, [512], [2], dtype="f32")
    x = W.attn_inputs(sh, seed=seed)
    q_old = np.asarray(x["q"], np.float64)
    q_new = q_old + eps * np.random.default_rng(seed + 1).normal(size=q_old.shape)
    exact_o, _ = OA.block_attn(q_new, x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], [512],
                               [2], 16)
    out_o, out_l = OA.attn_range(q_old, x["k_cache"], x["v_cache"], [0], [512], [2], 16)
    win_o, win_l = OA.block_attn(q_new, x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], [0],
                                 [2], 16)
    o, _ = OA.combine(out_o, out_l, win_o, win_l)
    err = np.abs(o[0, :, :32] - exact_o[0, :, :32])
    return float(err.max()), float(err.mean())


def test_stale_outside_part_accuracy():
    """Reuse is exact for unchanged queries and its error grows with the drift
    of the queries: the numbers quoted in the design notes."""
    rows = [(eps,) + reuse_error(eps) for eps in (0.0, 0.01, 0.05, 0.1, 0.3, 1.0)]
    for eps, mx, mean in rows:
        print(f"drift {eps:5.2f}: max {mx:.3e} mean {mean:.3e}")
    assert rows[0][1] < 1e-13
    maxes = [r[1] for r in rows]
    assert all(a < b for a, b in zip(maxes, maxes[1:]))
