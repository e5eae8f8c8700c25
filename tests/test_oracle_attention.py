"""Pins for the fp64 attention oracle (CPU only).

Each test checks the oracle against something other than its own formula:
hand-written masks from the block-causal rule, a scalar brute force written
in the whole-sequence view, torch's scaled_dot_product_attention on the two
special cases the pages name (block size 1 = causal attention; one block
covering the window = full bidirectional attention), closed forms, and the
exact-reuse invariant of completed blocks.
"""
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import kv_cache as OK

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(sh, x, scale=None, pairs=None):
    return OA.block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"],
                         sh.prefix_len, sh.n_win_blocks, sh.block_size, scale=scale, pairs=pairs)


def _f64(shape_dims, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape_dims, generator=g, dtype=torch.float64)


def _inputs64(sh, seed=0):
    nb, hq, hkv, d, w, cap = (sh.batch, sh.n_heads_q, sh.n_heads_kv, sh.head_dim, sh.w_max,
                              sh.cache_capacity)
    return dict(q=_f64((nb, hq, w, d), seed + 1), k_cache=_f64((nb, hkv, cap, d), seed + 2),
                v_cache=_f64((nb, hkv, cap, d), seed + 3), k_win=_f64((nb, hkv, w, d), seed + 4),
                v_win=_f64((nb, hkv, w, d), seed + 5))


def _golden_masks():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "block_causal_masks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("case"):
                _, p, b, nw = line.split()
                cur = (int(p), int(b), int(nw), [])
                cases.append(cur)
            else:
                cur[3].append([c == "1" for c in line])
    return [(p, b, nw, np.array(rows)) for p, b, nw, rows in cases]


@pytest.mark.parametrize("case", _golden_masks(), ids=lambda c: f"P{c[0]}B{c[1]}nw{c[2]}")
def test_mask_matches_hand_written_fixture(case):
    P, B, nw, expect = case
    # Recover the mask from attention outputs: with q = 0 every visible score
    # is equal, and with V = identity over keys row i's output is 1/count on
    # exactly its visible keys.
    n = P + nw * B
    sh = W.make_shape(1, 1, 1, n, B, [P], [nw], dtype="f32")
    eye = np.eye(n)
    x = dict(q=np.zeros((1, 1, nw * B, n)), k_cache=np.ones((1, 1, sh.cache_capacity, n)),
             v_cache=np.zeros((1, 1, sh.cache_capacity, n)), k_win=np.ones((1, 1, nw * B, n)),
             v_win=eye[None, None, P:])
    x["v_cache"][0, 0, :P] = eye[:P]
    out, lse = _run(sh, x)
    got = out[0, 0] > 0
    assert got.shape == expect.shape
    assert (got == expect).all()
    counts = expect.sum(axis=1)
    np.testing.assert_allclose(out[0, 0][expect], np.repeat(1.0 / counts, counts), rtol=1e-15)
    np.testing.assert_allclose(lse[0, 0], np.log(counts), rtol=1e-15)


def _brute_force(q, kc, vc, kw, vw, P, nw, B, scale, group):
    """Scalar loops in the whole-sequence view: the cached keys belong to
    blocks that precede the window, window position i belongs to block i//B,
    and a query sees a key whenever the key's block is not later than its
    own."""
    Wn = nw * B
    hq, d = q.shape[0], q.shape[2]
    out = np.full((hq, Wn, d), np.nan)
    lse = np.full((hq, Wn), np.nan)
    seq_block = [-1] * P + [i // B for i in range(Wn)]
    for h in range(hq):
        g = h // group
        keys = [kc[g, j] for j in range(P)] + [kw[g, i] for i in range(Wn)]
        vals = [vc[g, j] for j in range(P)] + [vw[g, i] for i in range(Wn)]
        for i in range(Wn):
            qb = i // B
            sc = []
            for j in range(P + Wn):
                if seq_block[j] <= qb:
                    sc.append((j, scale * sum(q[h, i, t] * keys[j][t] for t in range(d))))
            mx = max(s for _, s in sc)
            den = sum(math.exp(s - mx) for _, s in sc)
            for t in range(d):
                out[h, i, t] = sum(math.exp(s - mx) * vals[j][t] for j, s in sc) / den
            lse[h, i] = mx + math.log(den)
    return out, lse


@pytest.mark.parametrize("P,B,nw,hq,hkv,d", [(0, 1, 3, 1, 1, 3), (5, 2, 3, 2, 1, 4),
                                            (3, 3, 2, 2, 2, 8), (4, 2, 1, 4, 2, 2),
                                            (1, 1, 1, 1, 1, 5)])
def test_brute_force_scalar_loops(P, B, nw, hq, hkv, d):
    sh = W.make_shape(1, hq, hkv, d, B, [P], [nw], dtype="f32", extra_capacity=2)
    x = _inputs64(sh, seed=P * 100 + B * 10 + nw)
    scale = 0.37
    out, lse = _run(sh, x, scale=scale)
    n = {k: v.numpy() for k, v in x.items()}
    bo, bl = _brute_force(n["q"][0], n["k_cache"][0], n["v_cache"][0], n["k_win"][0],
                          n["v_win"][0], P, nw, B, scale, hq // hkv)
    np.testing.assert_allclose(out[0], bo, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0], bl, rtol=0, atol=1e-13)


def test_block_size_one_is_causal_attention():
    # B = 1 leaves one token per block: a window token sees the cache and the
    # window tokens up to and including itself, i.e. causal attention.
    P, nw, d, h = 7, 9, 16, 3
    sh = W.make_shape(1, h, h, d, 1, [P], [nw], dtype="f32")
    x = _inputs64(sh, seed=11)
    out, lse = _run(sh, x)
    # Full-sequence causal SDPA over P + nw tokens; the cache positions get
    # arbitrary queries and only the last nw rows are compared.
    qfull = torch.cat([_f64((1, h, P, d), 99), x["q"]], dim=2)
    kfull = torch.cat([x["k_cache"][:, :, :P], x["k_win"]], dim=2)
    vfull = torch.cat([x["v_cache"][:, :, :P], x["v_win"]], dim=2)
    ref = torch.nn.functional.scaled_dot_product_attention(qfull, kfull, vfull, is_causal=True)
    np.testing.assert_allclose(out[0], ref[0, :, P:].numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("P", [0, 13])
def test_one_block_is_bidirectional_attention(P):
    d, h, B = 8, 2, 12
    sh = W.make_shape(1, h, h, d, B, [P], [1], dtype="f32")
    x = _inputs64(sh, seed=21 + P)
    out, _ = _run(sh, x)
    kfull = torch.cat([x["k_cache"][:, :, :P], x["k_win"]], dim=2)
    vfull = torch.cat([x["v_cache"][:, :, :P], x["v_win"]], dim=2)
    ref = torch.nn.functional.scaled_dot_product_attention(x["q"], kfull, vfull)
    np.testing.assert_allclose(out[0], ref[0].numpy(), rtol=0, atol=1e-12)


def test_lse_matches_scipy_logsumexp():
    from scipy.special import logsumexp
    P, B, nw, d = 6, 4, 3, 8
    sh = W.make_shape(1, 1, 1, d, B, [P], [nw], dtype="f32")
    x = _inputs64(sh, seed=5)
    _, lse = _run(sh, x, scale=1.0)
    q = x["q"][0, 0].numpy()
    keys = np.concatenate([x["k_cache"][0, 0, :P].numpy(), x["k_win"][0, 0].numpy()])
    for i in range(nw * B):
        n_vis = P + (i // B + 1) * B  # keys visible to row i are a prefix of the key list
        ref = logsumexp(keys[:n_vis] @ q[i])
        assert abs(lse[0, 0, i] - ref) < 1e-12


def test_constant_values_and_score_shift():
    P, B, nw, d, h = 9, 4, 3, 8, 2
    sh = W.make_shape(1, h, h, d, B, [P], [nw], dtype="f32")
    x = _inputs64(sh, seed=8)
    c = np.linspace(-1.0, 2.0, d)
    xc = dict(x)
    xc["v_cache"] = torch.tensor(np.broadcast_to(c, x["v_cache"].shape).copy())
    xc["v_win"] = torch.tensor(np.broadcast_to(c, x["v_win"].shape).copy())
    out, _ = _run(sh, xc)
    np.testing.assert_allclose(out[0], np.broadcast_to(c, out[0].shape), rtol=0, atol=1e-14)
    # Adding the same vector u to every key moves all scores of row i by the
    # same amount scale * q_i.u; the softmax, hence the output, is unchanged
    # and the LSE moves by exactly that amount.
    u = _f64((d,), 77)
    xs = dict(x)
    xs["k_cache"] = x["k_cache"] + u
    xs["k_win"] = x["k_win"] + u
    o1, l1 = _run(sh, x)
    o2, l2 = _run(sh, xs)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    shift = (x["q"].numpy() @ u.numpy()) / math.sqrt(d)
    np.testing.assert_allclose(l2 - l1, shift, rtol=0, atol=1e-12)


def test_single_visible_key_returns_its_value():
    # No cache, B = 1: window row 0 sees only window key 0.
    sh = W.make_shape(1, 1, 1, 6, 1, [0], [4], dtype="f32")
    x = _inputs64(sh, seed=3)
    out, _ = _run(sh, x)
    np.testing.assert_array_equal(out[0, 0, 0], x["v_win"][0, 0, 0].numpy())


def test_gqa_head_grouping():
    # KV head g holds the constant value g + 1 in every V row; query head h
    # must return the constant of KV head h // (Hq / Hkv).
    hq, hkv = 6, 2
    sh = W.make_shape(1, hq, hkv, 4, 2, [3], [2], dtype="f32")
    x = _inputs64(sh, seed=4)
    for g in range(hkv):
        x["v_cache"][0, g] = g + 1.0
        x["v_win"][0, g] = g + 1.0
    out, _ = _run(sh, x)
    for h in range(hq):
        np.testing.assert_allclose(out[0, h], h // (hq // hkv) + 1.0, rtol=0, atol=1e-14)


def test_later_blocks_do_not_affect_earlier_rows():
    P, B, nw, d, h = 10, 4, 4, 8, 2
    sh = W.make_shape(1, h, h, d, B, [P], [nw], dtype="f32")
    x = _inputs64(sh, seed=9)
    o1, l1 = _run(sh, x)
    for k in range(nw - 1):
        y = {n: t.clone() for n, t in x.items()}
        lo = (k + 1) * B
        for n in ("q", "k_win", "v_win"):
            y[n][:, :, lo:] = _f64(tuple(y[n][:, :, lo:].shape), 1000 + k)
        o2, l2 = _run(sh, y)
        np.testing.assert_array_equal(o2[:, :, :lo], o1[:, :, :lo])
        np.testing.assert_array_equal(l2[:, :, :lo], l1[:, :, :lo])
        assert not np.array_equal(o2[:, :, lo:], o1[:, :, lo:])


@pytest.mark.parametrize("P", [0, 7, 16])
def test_cached_block_equals_recomputed_block(P):
    # The exactness claim: a completed block's K/V moved from the window into
    # the cache give the same outputs for the rows that stay in the window.
    B, nw, d, hq, hkv = 4, 3, 8, 4, 2
    sh = W.make_shape(1, hq, hkv, d, B, [P], [nw], dtype="f32", extra_capacity=B)
    x = {k: v.numpy() for k, v in _inputs64(sh, seed=P).items()}
    o1, l1 = _run(sh, x)
    kc, vc, p2 = OK.kv_commit(x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], [P], 0, B)
    y = dict(q=OK.drop_oldest_block(x["q"], 0, B), k_cache=kc, v_cache=vc,
             k_win=OK.drop_oldest_block(x["k_win"], 0, B),
             v_win=OK.drop_oldest_block(x["v_win"], 0, B))
    sh2 = W.make_shape(1, hq, hkv, d, B, p2, [nw - 1], dtype="f32", max_win_blocks=nw,
                       cache_capacity=sh.cache_capacity)
    o2, l2 = _run(sh2, y)
    np.testing.assert_array_equal(o2[:, :, :(nw - 1) * B], o1[:, :, B:])
    np.testing.assert_array_equal(l2[:, :, :(nw - 1) * B], l1[:, :, B:])


def test_rows_past_window_are_nan_and_pairs_subset():
    sh = W.make_shape(2, 2, 1, 4, 2, [3, 1], [1, 3], dtype="f32")
    x = _inputs64(sh, seed=2)
    out, lse = _run(sh, x)
    assert np.isnan(out[0, :, 2:]).all() and not np.isnan(out[0, :, :2]).any()
    assert not np.isnan(out[1]).any()
    o2, _ = _run(sh, x, pairs=[(1, 1)])
    np.testing.assert_array_equal(o2[1, 1], out[1, 1])
    assert np.isnan(o2[0]).all() and np.isnan(o2[1, 0]).all()


def test_idle_requests_have_no_rows_and_leave_the_others_alone():
    # Requests 1 (no cache, no window) and 2 (cache only) are idle: they have
    # no window rows, so no outputs; each active request's rows equal those of
    # the same request attended on its own.
    prefix, nwin, B = [5, 0, 7, 3], [2, 0, 0, 1], 2
    sh = W.make_shape(4, 4, 2, 8, B, prefix, nwin, dtype="f32", max_win_blocks=2)
    x = _inputs64(sh, seed=11)
    out, lse = _run(sh, x)
    assert np.isnan(out[1]).all() and np.isnan(out[2]).all()
    assert np.isnan(lse[1]).all() and np.isnan(lse[2]).all()
    for b in (0, 3):
        one = W.make_shape(1, 4, 2, 8, B, [prefix[b]], [nwin[b]], dtype="f32", max_win_blocks=2,
                           cache_capacity=sh.cache_capacity)
        y = {k: v[b:b + 1] for k, v in x.items()}
        o1, l1 = _run(one, y)
        rows = nwin[b] * B
        np.testing.assert_array_equal(out[b, :, :rows], o1[0, :, :rows])
        np.testing.assert_array_equal(lse[b, :, :rows], l1[0, :, :rows])
