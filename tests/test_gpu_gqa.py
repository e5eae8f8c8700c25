"""GPU parity of the grouped-query attention kernel (attn_gqa.hip) against the
fp64 oracle, through the C ABI.

The library sends a bf16 call there when the query heads share KV heads and
the call has at least 40 query rows per compute unit (10240 rows on the
256-CU MI355X).  The random draws keep at least 64 rows per compute unit;
the edge cases go down to 42 (48-row units, keys split between the wave
groups), and a second set of draws spans 30-64 rows per compute unit, on both
sides of the routing threshold, with the paged layout checked bit for bit.  The draws vary batch, KV
heads, group size, head_dim, block size and window, with prefixes that mix
tile-boundary lengths (0, 1, 63, 64, 65) and uniform ones; unread cache
slots and window rows are NaN and padding rows must stay untouched."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import compare_attn, oracle_attn, poisoned_inputs, run_attn, say, to_pages

pytestmark = pytest.mark.gpu

MIN_ROWS = 64 * 256  # lower bound of the random draws' query rows
ROUTE_ROWS = 40 * 256  # query rows that route a grouped-query bf16 call to the kernel


def _rows(sh):
    return sum(sh.n_heads_q * sh.win_rows(b) for b in range(sh.batch))


def _draw(k):
    rng = np.random.default_rng(9000 + k)
    while True:
        nb = int(rng.integers(1, 7))
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([2, 3, 4, 7, 8]))
        d = int(rng.choice([64, 128]))
        bsz = int(rng.choice([8, 16, 32, 64]))
        mw = int(rng.integers(1, 5))
        nwin = [int(rng.integers(1, mw + 1)) for _ in range(nb)]
        nwin[0] = mw
        edge = [0, 1, 63, 64, 65, 127, 128]
        prefix = [int(rng.choice(edge)) if rng.random() < 0.4 else int(rng.integers(0, 2600))
                  for _ in range(nb)]
        sh = W.make_shape(nb, hkv * g, hkv, d, bsz, prefix, nwin, dtype="bf16",
                          max_win_blocks=mw, extra_capacity=int(rng.integers(0, 9)))
        if _rows(sh) >= MIN_ROWS:
            return sh


def _pairs(sh, k, n=10):
    rng = np.random.default_rng(77 + k)
    pairs = {(b, int(rng.integers(0, sh.n_heads_q))) for b in range(sh.batch)}
    while len(pairs) < min(n, sh.batch * sh.n_heads_q):
        pairs.add((int(rng.integers(0, sh.batch)), int(rng.integers(0, sh.n_heads_q))))
    return sorted(pairs)


@pytest.mark.parametrize("k", range(10))
def test_random_gqa_shapes(k):
    sh = _draw(k)
    say(f"--- gqa draw {k}: {sh} rows {_rows(sh)}")
    x = poisoned_inputs(sh, seed=k)
    out, lse = run_attn(sh, x, out_fill=7.0)
    pairs = _pairs(sh, k)
    ref_o, ref_l = oracle_attn(sh, x, pairs=pairs)
    compare_attn(sh, out, lse, ref_o, ref_l, pairs=pairs, label=f"gqa-draw{k}")
    o = out.float().cpu().numpy()
    lo = lse.cpu().numpy()
    for b in range(sh.batch):
        assert (o[b, :, sh.win_rows(b):] == 7.0).all()
        assert (lo[b, :, sh.win_rows(b):] == 7.0).all()


def _draw_near_threshold(k):
    """Whole-block prefixes (so the paged layout applies), 30-64 query rows per
    compute unit: both sides of the grouped-query routing threshold, and the
    units of at most 8 blocks whose wave groups split each tile's keys."""
    rng = np.random.default_rng(12000 + k)
    while True:
        nb = int(rng.integers(2, 13))
        hkv = int(rng.choice([2, 4, 8]))
        g = int(rng.choice([2, 4, 7, 8]))
        d = int(rng.choice([64, 128]))
        bsz = int(rng.choice([8, 16, 32]))
        mw = int(rng.integers(1, 5))
        nwin = [int(rng.integers(0, mw + 1)) for _ in range(nb)]
        nwin[0] = mw
        prefix = [int(rng.integers(0, 2600)) // bsz * bsz for _ in range(nb)]
        sh = W.make_shape(nb, hkv * g, hkv, d, bsz, prefix, nwin, dtype="bf16",
                          max_win_blocks=mw, extra_capacity=int(rng.integers(0, 9)))
        if 30 * 256 <= _rows(sh) < MIN_ROWS:
            return sh


@pytest.mark.parametrize("k", range(8))
def test_random_gqa_near_threshold(k):
    import block_causal_attention_d2f_amd as d2f
    sh = _draw_near_threshold(k)
    say(f"--- gqa near-threshold draw {k}: {sh} rows {_rows(sh)}")
    x = poisoned_inputs(sh, seed=500 + k)
    out, lse = run_attn(sh, x, out_fill=7.0)
    rng = np.random.default_rng(600 + k)
    active = [b for b in range(sh.batch) if sh.win_rows(b) > 0]
    pairs = sorted({(int(rng.choice(active)), int(rng.integers(0, sh.n_heads_q)))
                    for _ in range(8)})
    ref_o, ref_l = oracle_attn(sh, x, pairs=pairs)
    compare_attn(sh, out, lse, ref_o, ref_l, pairs=pairs, label=f"gqa-near{k}")
    o = out.float().cpu().numpy()
    lo = lse.cpu().numpy()
    for b in range(sh.batch):
        assert (o[b, :, sh.win_rows(b):] == 7.0).all()
        assert (lo[b, :, sh.win_rows(b):] == 7.0).all()
    kp, vp, pt, wp = to_pages(sh, x, seed=k)
    o2 = torch.full_like(x["q"], 7.0)
    l2 = torch.full(x["q"].shape[:3], 7.0, device="cuda")
    d2f.d2f_block_attn_paged(x["q"], kp, vp, pt, wp, sh.prefix_len, sh.n_win_blocks,
                             out=o2, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), out.view(torch.int16)), "paged outputs differ"
    assert torch.equal(l2, lse), "paged lse differs"


@pytest.mark.parametrize("case", [
    # (nb, Hq, Hkv, D, B, prefix, nwin)
    (8, 16, 8, 128, 64, [0, 1, 63, 64, 65, 500, 2047, 3000], [4] * 8),  # group 2
    (11, 12, 4, 64, 64, [129 * i for i in range(11)], [4] * 11),       # group 3, head_dim 64
    (16, 64, 8, 128, 8, [7 * i * i for i in range(16)], [4] * 16),      # B = 8: 4 blocks per tile
    (2, 128, 8, 128, 48, [0, 777], [3, 3]),                              # group 16, B = 48
    (8, 28, 4, 128, 32, [2048, 2047, 1, 64, 65, 0, 1500, 2048], [3] * 8), # Dream shape, B = 32
    (8, 28, 4, 128, 16, [2048, 2047, 1, 64, 65, 0, 1500, 2048], [3] * 8), # B = 16: 48-row units
    (8, 28, 4, 64, 16, [16, 0, 700, 2048, 33, 64, 1, 999], [3] * 8),      # the same, head_dim 64
])
def test_gqa_edge_shapes(case):
    nb, hq, hkv, d, b, prefix, nwin = case
    sh = W.make_shape(nb, hq, hkv, d, b, prefix, nwin, dtype="bf16", extra_capacity=5)
    assert _rows(sh) >= ROUTE_ROWS
    say(f"--- gqa edge {case}: rows {_rows(sh)}")
    x = poisoned_inputs(sh, seed=nb + hq)
    out, lse = run_attn(sh, x, out_fill=7.0)
    pairs = _pairs(sh, nb + hq, n=12)
    ref_o, ref_l = oracle_attn(sh, x, pairs=pairs)
    compare_attn(sh, out, lse, ref_o, ref_l, pairs=pairs, label=f"gqa-edge-G{hq // hkv}-B{b}")


@pytest.mark.parametrize("nwin", [[4, 4, 3, 2, 4, 4], [2, 2, 1, 1, 2, 2]])
def test_gqa_deterministic_and_causal(nwin):
    """Two runs bit-identical; re-drawing the last window block (its q, K and
    V) leaves the rows of the earlier blocks bit-identical.  The second draw
    has 80-row units (80 rows per CU): each tile's keys are split between
    the two wave groups and joined at the end."""
    sh = W.make_shape(6, 32, 4, 128, 64, [2048, 65, 0, 1000, 1, 64], nwin, dtype="bf16")
    assert _rows(sh) >= MIN_ROWS
    x = poisoned_inputs(sh, seed=5)
    o1, l1 = run_attn(sh, x, out_fill=7.0)
    o2, l2 = run_attn(sh, x, out_fill=7.0)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    B = sh.block_size
    y = {k: v.clone() for k, v in x.items()}
    for b in range(sh.batch):
        lo = (sh.n_win_blocks[b] - 1) * B
        for n in ("q", "k_win", "v_win"):
            t = y[n][b, :, lo:lo + B]
            y[n][b, :, lo:lo + B] = torch.randn(t.shape, device="cuda").to(t.dtype)
    o3, l3 = run_attn(sh, y, out_fill=7.0)
    for b in range(sh.batch):
        keep = (sh.n_win_blocks[b] - 1) * B
        assert torch.equal(o1[b, :, :keep].view(torch.int16), o3[b, :, :keep].view(torch.int16))
        assert torch.equal(l1[b, :, :keep], l3[b, :, :keep])
    pairs = [(0, 0), (1, 31), (2, 9), (3, 17), (4, 5), (5, 30)]
    ref_o, ref_l = oracle_attn(sh, y, pairs=pairs)
    compare_attn(sh, o3, l3, ref_o, ref_l, pairs=pairs, label="gqa-redrawn")


@pytest.mark.parametrize("bsz,nb", [(64, 6), (32, 8)])
def test_gqa_key_range(bsz, nb):
    """The window's queries over a cache key range (the outside-block part)
    on a grouped-query shape: against the oracle's range attention (block 32:
    96-row units, keys split between the wave groups)."""
    import block_causal_attention_d2f_amd as d2f
    from oracle import attention as OA
    prefix = [2048, 1500, 700, 64, 3000, 129, 2100, 999][:nb]
    sh = W.make_shape(nb, 28, 4, 128, bsz, prefix, [4 if bsz == 64 else 3] * nb, dtype="bf16")
    assert _rows(sh) >= MIN_ROWS
    x = poisoned_inputs(sh, seed=6)
    lo = [100, 0, 63, 1, 2500, 0, 2099, 500][:nb]
    hi = [2048, 1437, 700, 64, 3000, 129, 2100, 999][:nb]
    out = torch.full_like(x["q"], 7.0)
    lse = torch.full(x["q"].shape[:3], 7.0, device="cuda")
    d2f.d2f_block_attn_range(x["q"], x["k_cache"], x["v_cache"], lo, hi, sh.n_win_blocks,
                             sh.block_size, out=out, lse=lse)
    torch.cuda.synchronize()
    ref_o, ref_l = OA.attn_range(x["q"], x["k_cache"], x["v_cache"], lo, hi, sh.n_win_blocks,
                                 sh.block_size)
    compare_attn(sh, out, lse, ref_o, ref_l, label="gqa-range")
