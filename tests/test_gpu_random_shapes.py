"""Seeded random shapes, for breadth beyond the hand-picked edge cases:
d2f_block_attn (through the C ABI) against the fp64 oracle over batch, head
counts, GQA group, head_dim, block size, ragged and empty prefixes (including
the tile-boundary lengths 63/64/65/127/128), idle requests and spare cache
capacity; d2f_block_attn_paged against d2f_block_attn, bit for bit, on
whole-block prefixes of the same draws; and attention in segments (cache key
ranges at random cut points joined to the window-only part) against the
oracle's full attention."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import compare_attn, oracle_attn, poisoned_inputs, run_attn, say, to_pages

pytestmark = pytest.mark.gpu

EDGE_PREFIX = [0, 1, 63, 64, 65, 127, 128, 511]
N_DRAWS = 12


def draw(seed, dtype, paged=False):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([64, 128] if dtype == "bf16" else [32, 64, 128]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 3, 4, 7, 8]))
    bsz = int(rng.choice([8, 16, 32, 64] if paged else [1, 2, 5, 8, 16, 32, 48, 64]))
    nb = int(rng.integers(1, 5))
    max_win = int(min(rng.integers(1, 5), max(1, 256 // bsz)))  # windows of at most 256 rows
    prefix = [int(rng.choice(EDGE_PREFIX)) if rng.random() < 0.5 else int(rng.integers(0, 3000))
              for _ in range(nb)]
    if paged:
        prefix = [p // bsz * bsz for p in prefix]
    nwin = [int(rng.integers(0, max_win + 1)) for _ in range(nb)]
    if max(nwin) == 0:
        nwin[int(rng.integers(0, nb))] = max_win
    return W.make_shape(nb, hkv * g, hkv, d, bsz, prefix, nwin, dtype=dtype,
                        max_win_blocks=max_win, extra_capacity=int(rng.integers(0, 9)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", range(N_DRAWS))
def test_random_shape_against_oracle(dtype, k):
    seed = 7000 + 100 * k + (0 if dtype == "f32" else 50)
    sh = draw(seed, dtype)
    say(f"--- random attention case seed={seed}: {sh}")
    x = poisoned_inputs(sh, seed=seed)
    out, lse = run_attn(sh, x, out_fill=7.0)
    ref_o, ref_l = oracle_attn(sh, x)
    compare_attn(sh, out, lse, ref_o, ref_l, label=f"random-{dtype}-{seed}")
    o = out.float().cpu().numpy()
    lv = lse.cpu().numpy()
    for b in range(sh.batch):
        assert (o[b, :, sh.win_rows(b):] == 7.0).all(), "padding rows were written"
        assert (lv[b, :, sh.win_rows(b):] == 7.0).all(), "padding LSE entries were written"


@pytest.mark.parametrize("k", range(N_DRAWS // 2))
def test_random_paged_equals_contiguous(k):
    import block_causal_attention_d2f_amd as d2f
    seed = 9000 + 100 * k
    sh = draw(seed, "bf16", paged=True)
    say(f"--- random paged case seed={seed}: {sh}")
    x = poisoned_inputs(sh, seed=seed)
    kp, vp, pt, wp = to_pages(sh, x, seed=seed)
    o1 = torch.full_like(x["q"], 7.0)
    l1 = torch.full(x["q"].shape[:3], 7.0, device="cuda")
    o2, l2 = o1.clone(), l1.clone()
    d2f.d2f_block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"],
                       sh.prefix_len, sh.n_win_blocks, sh.block_size, out=o1, lse=l1)
    d2f.d2f_block_attn_paged(x["q"], kp, vp, pt, wp, sh.prefix_len, sh.n_win_blocks,
                             out=o2, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "outputs differ"
    assert torch.equal(l1, l2), "lse differs"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("k", range(4))
def test_random_segments_compose_to_full_attention(dtype, k):
    """The window-only part joined with 1..3 cache key ranges that tile
    [0, P) at random cut points (empty ranges included, their parts start at
    LSE = -inf) equals full block-causal attention, against the oracle."""
    import block_causal_attention_d2f_amd as d2f
    seed = 11000 + 100 * k + (0 if dtype == "f32" else 50)
    sh = draw(seed, dtype)
    rng = np.random.default_rng(seed + 1)
    n_ranges = int(rng.integers(1, 4))
    cuts = [[0] + sorted(int(c) for c in rng.integers(0, p + 1, n_ranges - 1)) + [p]
            for p in sh.prefix_len]
    say(f"--- random segments case seed={seed}: {sh}, cuts {cuts}")
    x = poisoned_inputs(sh, seed=seed)
    B, nwin = sh.block_size, sh.n_win_blocks
    o, l = d2f.d2f_block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"],
                              [0] * sh.batch, nwin, B)
    for j in range(n_ranges):
        lo = [c[j] for c in cuts]
        hi = [c[j + 1] for c in cuts]
        po = torch.zeros_like(x["q"])
        pl = torch.full(x["q"].shape[:3], float("-inf"), device="cuda")
        d2f.d2f_block_attn_range(x["q"], x["k_cache"], x["v_cache"], lo, hi, nwin, B, out=po,
                                 lse=pl)
        o, l = d2f.d2f_attn_combine(o, l, po, pl, nwin, B, out=o, lse=l)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_attn(sh, x)
    compare_attn(sh, o, l, ref_o, ref_l, label=f"segments-{dtype}-{seed}")


def test_more_requests_than_one_launch():
    """70 requests, past the 64 a launch carries: full attention, the paged
    call and the segment join are each planned as two launches; all against
    the oracle (paged: bit for bit against contiguous)."""
    import block_causal_attention_d2f_amd as d2f
    rng = np.random.default_rng(424242)
    nb, B = 70, 8
    prefix = [int(p) // B * B for p in rng.integers(0, 300, nb)]
    nwin = [int(n) for n in rng.integers(0, 3, nb)]
    nwin[0] = 2
    sh = W.make_shape(nb, 4, 2, 64, B, prefix, nwin, dtype="bf16", max_win_blocks=2)
    say(f"--- 70-request case: {sh}")
    x = poisoned_inputs(sh, seed=4242)
    out, lse = run_attn(sh, x, out_fill=7.0)
    ref_o, ref_l = oracle_attn(sh, x)
    compare_attn(sh, out, lse, ref_o, ref_l, label="70-requests")
    kp, vp, pt, wp = to_pages(sh, x, seed=4242)
    o2 = torch.full_like(x["q"], 7.0)
    l2 = torch.full(x["q"].shape[:3], 7.0, device="cuda")
    d2f.d2f_block_attn_paged(x["q"], kp, vp, pt, wp, prefix, nwin, out=o2, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)
    wo, wl = d2f.d2f_block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"],
                                [0] * nb, nwin, B)
    co = torch.zeros_like(x["q"])
    cl = torch.full(x["q"].shape[:3], float("-inf"), device="cuda")
    d2f.d2f_block_attn_range(x["q"], x["k_cache"], x["v_cache"], [0] * nb, prefix, nwin, B,
                             out=co, lse=cl)
    jo, jl = d2f.d2f_attn_combine(wo, wl, co, cl, nwin, B)
    torch.cuda.synchronize()
    compare_attn(sh, jo, jl, ref_o, ref_l, label="70-requests-segments")
