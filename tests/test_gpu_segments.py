"""GPU checks of attention in segments: d2f_block_attn_range (window queries
over a cache key range) and d2f_attn_combine (log-space join) against the
oracle, and the exact composition -- cache range + window-only, joined --
against the full d2f_block_attn."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from parity import ATOL_F32, LSE_F32, MAX_BF16, MEAN_BF16, LSE_BF16, poisoned_inputs, say

pytestmark = pytest.mark.gpu


def _cmp(sh, got_o, got_l, ref_o, ref_l, label):
    errs, lerrs = [], []
    for b in range(sh.batch):
        Wb = sh.win_rows(b)
        if Wb == 0 or np.isnan(ref_l[b, :, :Wb]).all():
            continue
        errs.append(np.abs(got_o[b, :, :Wb].float().cpu().numpy() - ref_o[b, :, :Wb]).ravel())
        lerrs.append(np.abs(got_l[b, :, :Wb].cpu().numpy() - ref_l[b, :, :Wb]).ravel())
    e, le = np.concatenate(errs), np.concatenate(lerrs)
    say(f"[segments {label}] max={e.max():.3e} mean={e.mean():.3e} lse={le.max():.3e}")
    if sh.dtype == "f32":
        assert e.max() <= ATOL_F32 and le.max() <= LSE_F32
    else:
        assert e.max() <= MAX_BF16 and e.mean() <= MEAN_BF16 and le.max() <= LSE_BF16


CASES = [
    # nb, hq, hkv, d, B, prefix, nwin, dtype, key_lo, key_hi
    (1, 32, 32, 128, 16, [512], [2], "bf16", [0], [512]),
    (2, 8, 2, 128, 16, [3000, 700], [3, 1], "bf16", [37, 0], [2999, 700]),   # offsets, splits
    (3, 4, 4, 64, 32, [100, 64, 90], [2, 1, 2], "bf16", [5, 0, 90], [99, 64, 90]),  # empty range
    (2, 4, 2, 64, 16, [200, 70], [2, 3], "f32", [1, 63], [200, 64]),
    (1, 2, 2, 32, 8, [129], [3], "f32", [64], [129]),
]


@pytest.mark.parametrize("case", CASES)
def test_range_against_oracle(case):
    import block_causal_attention_d2f_amd as d2f
    nb, hq, hkv, d, B, prefix, nwin, dt, lo, hi = case
    sh = W.make_shape(nb, hq, hkv, d, B, prefix, nwin, dtype=dt)
    x = poisoned_inputs(sh, seed=sum(prefix))
    out = torch.full_like(x["q"], 7.0)
    lse = torch.full(x["q"].shape[:3], 7.0, device="cuda")
    d2f.d2f_block_attn_range(x["q"], x["k_cache"], x["v_cache"], lo, hi, nwin, B, out=out,
                             lse=lse)
    torch.cuda.synchronize()
    ro, rl = OA.attn_range(x["q"].cpu(), x["k_cache"].cpu(), x["v_cache"].cpu(), lo, hi, nwin, B)
    _cmp(sh, out, lse, ro, rl, f"range-{dt}-d{d}")
    for b in range(nb):   # idle requests and rows past the window untouched
        first = 0 if hi[b] <= lo[b] else sh.win_rows(b)
        assert (out[b, :, first:].float() == 7.0).all() and (lse[b, :, first:] == 7.0).all()


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 32)])
def test_composition_equals_full_attention(dt, d):
    """Cache range [0, P) and the window-only part, joined on the GPU, give
    the full block-causal attention (and the join matches the oracle's)."""
    import block_causal_attention_d2f_amd as d2f
    sh = W.make_shape(2, 4, 2, d, 16, [1000, 64], [3, 2], dtype=dt)
    x = W.attn_inputs(sh, device="cuda", seed=8)
    full_o, full_l = d2f.d2f_block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"],
                                        x["v_win"], sh.prefix_len, sh.n_win_blocks, 16)
    out_o, out_l = d2f.d2f_block_attn_range(x["q"], x["k_cache"], x["v_cache"], [0, 0],
                                            sh.prefix_len, sh.n_win_blocks, 16)
    win_o, win_l = d2f.d2f_block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"],
                                      [0, 0], sh.n_win_blocks, 16)
    o, l = d2f.d2f_attn_combine(out_o, out_l, win_o, win_l, sh.n_win_blocks, 16)
    torch.cuda.synchronize()
    ro, rl = OA.combine(out_o.cpu().double().numpy(), out_l.cpu().double().numpy(),
                        win_o.cpu().double().numpy(), win_l.cpu().double().numpy())
    for b in range(2):
        Wb = sh.win_rows(b)
        # the join against the oracle's join of the same parts
        tol = 2e-6 if dt == "f32" else 8e-3  # one output rounding in bf16
        assert np.abs(o[b, :, :Wb].float().cpu().numpy() - ro[b, :, :Wb]).max() <= tol
        assert np.abs(l[b, :, :Wb].cpu().numpy() - rl[b, :, :Wb]).max() <= 1e-5
    exact_o, exact_l = OA.block_attn(x["q"].cpu(), x["k_cache"].cpu(), x["v_cache"].cpu(),
                                     x["k_win"].cpu(), x["v_win"].cpu(), sh.prefix_len,
                                     sh.n_win_blocks, 16)
    _cmp(sh, o, l, exact_o, exact_l, f"composed-{dt}-d{d}")
    _cmp(sh, full_o, full_l, exact_o, exact_l, f"full-{dt}-d{d}")
    # in place: out / lse may alias the first part
    d2f.d2f_attn_combine(out_o, out_l, win_o, win_l, sh.n_win_blocks, 16, out=out_o, lse=out_l)
    torch.cuda.synchronize()
    for b in range(2):   # rows past each window are left as they were
        Wb = sh.win_rows(b)
        assert torch.equal(out_o[b, :, :Wb], o[b, :, :Wb]) and torch.equal(out_l[b, :, :Wb],
                                                                           l[b, :, :Wb])
