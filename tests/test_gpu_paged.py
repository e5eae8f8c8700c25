"""GPU checks of the paged cache: d2f_block_attn_paged gives the same bits as
d2f_block_attn on the same keys laid out in randomly numbered pages, matches
the paged oracle, and d2f_kv_commit_paged persists a block by a table update
after which attention equals the contiguous path's after d2f_kv_commit."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import kv_cache as OK
from parity import compare_attn, poisoned_inputs, say, to_pages

pytestmark = pytest.mark.gpu


CASES = [
    # nb, hq, hkv, d, B, prefix, nwin
    (1, 32, 32, 128, 16, [512], [2]),           # the LLaDA-shaped step (32-row units)
    (2, 8, 2, 64, 16, [128, 16], [2, 3]),       # GQA 4, head_dim 64
    (3, 4, 1, 128, 8, [1000 // 8 * 8, 64, 0], [4, 1, 2]),   # B = 8, empty prefix, key splits
    (1, 8, 8, 128, 32, [4096], [3]),            # B = 32, a long prefix split across units
    (2, 28, 4, 128, 64, [2048, 1024], [3, 2]),  # Dream-like GQA 7, B = 64
    (3, 4, 2, 128, 16, [48, 96, 32], [2, 0, 1]),  # an idle request
    # Grouped-query shapes with >= 40 query rows per CU (the grouped-query
    # kernel's paged loader): Dream-like B = 64, B = 16 (48-row units with
    # keys split between the wave groups), B = 32 with ragged prefixes,
    # head_dim 64 with 16-row pages, 8-row pages.
    (8, 28, 4, 128, 64, [2048, 1984, 64, 0, 1024, 2048, 512, 1920], [3] * 8),
    (8, 28, 4, 128, 16, [2048, 1984, 64, 0, 1024, 2048, 512, 1920], [3] * 8),
    (6, 32, 4, 128, 32, [2048, 32, 0, 4096, 1024, 96], [3] * 6),
    (10, 28, 4, 64, 16, [16 * i * i for i in range(10)], [4] * 10),
    (16, 64, 8, 128, 8, [8 * i for i in range(16)], [4] * 16),
    # 142 key tiles in a unit: the page entries of tiles 64.. and 128.. are
    # fetched while earlier tiles are in flight.
    (4, 64, 8, 128, 16, [9008, 16, 4096, 8192], [4] * 4),
]


@pytest.mark.parametrize("case", CASES)
def test_paged_equals_contiguous_bit_for_bit(case):
    import block_causal_attention_d2f_amd as d2f
    nb, hq, hkv, d, B, prefix, nwin = case
    sh = W.make_shape(nb, hq, hkv, d, B, prefix, nwin, dtype="bf16",
                      max_win_blocks=max(nwin) if max(nwin) else 1)
    say(f"--- paged case {case}")
    x = poisoned_inputs(sh, seed=sum(prefix) + B)
    kp, vp, pt, wp = to_pages(sh, x, seed=B)
    o1 = torch.full_like(x["q"], 7.0)
    l1 = torch.full(x["q"].shape[:3], 7.0, device="cuda")
    o2, l2 = o1.clone(), l1.clone()
    d2f.d2f_block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], prefix, nwin,
                       B, out=o1, lse=l1)
    d2f.d2f_block_attn_paged(x["q"], kp, vp, pt, wp, prefix, nwin, out=o2, lse=l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "outputs differ"
    assert torch.equal(l1, l2), "lse differs"
    pairs = [(b, h) for b in range(nb) for h in range(min(hq, 4))]
    ro, rl = OA.block_attn_paged(x["q"].cpu(), kp.cpu(), vp.cpu(), pt.cpu(), wp.cpu(), prefix,
                                 nwin, B, pairs=pairs)
    if sum(nwin):
        compare_attn(sh, o2, l2, ro, rl, pairs=pairs, label=f"paged-B{B}-d{d}")


def test_paged_persist_then_attend():
    """Persist blocks of two requests in turn: the tables follow the oracle
    and attention equals the contiguous path after the same appends."""
    import block_causal_attention_d2f_amd as d2f
    B = 16
    sh = W.make_shape(2, 8, 4, 128, B, [64, 32], [3, 2], dtype="bf16", extra_capacity=64)
    x = W.attn_inputs(sh, device="cuda", seed=9)
    kp, vp, pt, wp = to_pages(sh, x, seed=10, spare=4)
    prefix_p, prefix_c = list(sh.prefix_len), list(sh.prefix_len)
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    kw, vw = x["k_win"].clone(), x["v_win"].clone()
    nwin = list(sh.n_win_blocks)
    pdev = torch.tensor(prefix_p, dtype=torch.int32, device="cuda")
    ot_pt, ot_wp, ot_p = pt.cpu().numpy(), wp.cpu().numpy(), list(prefix_p)
    for req in (0, 1, 0):
        d2f.d2f_kv_commit_paged(pt, wp, prefix_p, req, B, n_heads_kv=4, prefix_len_dev=pdev)
        ot_pt, ot_wp, ot_p = OK.kv_commit_paged(ot_pt, ot_wp, ot_p, req, B)
        d2f.d2f_kv_commit(kc, vc, kw, vw, prefix_c, req, B)
        kw[req, :, :-B] = kw[req, :, B:].clone()
        vw[req, :, :-B] = vw[req, :, B:].clone()
        nwin[req] -= 1
        torch.cuda.synchronize()
        assert prefix_p == prefix_c == ot_p and pdev.cpu().tolist() == prefix_p
        assert np.array_equal(pt.cpu().numpy(), ot_pt) and np.array_equal(wp.cpu().numpy(), ot_wp)
        o1, l1 = d2f.d2f_block_attn(x["q"], kc, vc, kw, vw, prefix_c, nwin, B)
        o2, l2 = d2f.d2f_block_attn_paged(x["q"], kp, vp, pt, wp, prefix_p, nwin)
        torch.cuda.synchronize()
        for b in range(2):
            r = nwin[b] * B
            assert torch.equal(o1[b, :, :r].view(torch.int16), o2[b, :, :r].view(torch.int16))
            assert torch.equal(l1[b, :, :r], l2[b, :, :r])
    say("[paged] persist + attend ok")
