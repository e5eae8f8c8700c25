"""GPU checks of d2f_kv_commit: byte-exact append, prefix bookkeeping, and
the exact-reuse claim (attention after appending a completed block equals
attention with that block still in the window) on the 32K-prefix workload."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import kv_cache as OK
from parity import compare_attn, oracle_attn, run_attn, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,d,layers", [("bf16", 128, 1), ("bf16", 128, 3), ("f32", 32, 2),
                                            ("bf16", 6, 2)])
def test_append_is_byte_exact(dtype, d, layers):
    import block_causal_attention_d2f_amd as d2f
    sh = W.make_shape(3, 4, 2, d, 16, [40, 0, 17], [2, 1, 3], dtype=dtype, extra_capacity=32)
    xs = [W.attn_inputs(sh, layer=l, device="cuda", seed=5) for l in range(layers)]
    kc = torch.stack([x["k_cache"] for x in xs])
    vc = torch.stack([x["v_cache"] for x in xs])
    kw = torch.stack([x["k_win"] for x in xs])
    vw = torch.stack([x["v_win"] for x in xs])
    kc0, vc0 = kc.clone(), vc.clone()
    prefix = list(sh.prefix_len)
    pdev = torch.tensor(prefix, dtype=torch.int32, device="cuda")
    arg = (kc, vc, kw, vw) if layers > 1 else (kc[0], vc[0], kw[0], vw[0])
    for req in (2, 0, 2):
        p0 = prefix[req]
        d2f.d2f_kv_commit(*arg, prefix, req, sh.block_size, prefix_len_dev=pdev)
        torch.cuda.synchronize()
        assert prefix[req] == p0 + sh.block_size
        assert pdev.cpu().tolist() == prefix
        for l in range(layers):
            assert torch.equal(kc[l, req, :, p0:p0 + 16].view(torch.uint8),
                               kw[l, req, :, 0:16].view(torch.uint8))
            assert torch.equal(vc[l, req, :, p0:p0 + 16].view(torch.uint8),
                               vw[l, req, :, 0:16].view(torch.uint8))
        kc0[:, req, :, p0:p0 + 16] = kw[:, req, :, 0:16]
        vc0[:, req, :, p0:p0 + 16] = vw[:, req, :, 0:16]
    # nothing else changed
    assert torch.equal(kc.view(torch.uint8), kc0.view(torch.uint8))
    assert torch.equal(vc.view(torch.uint8), vc0.view(torch.uint8))


def test_order_and_capacity_errors():
    import block_causal_attention_d2f_amd as d2f
    sh = W.make_shape(1, 2, 2, 64, 16, [16], [2], dtype="bf16")
    x = W.attn_inputs(sh, device="cuda")
    prefix = [16]
    with pytest.raises(d2f.D2FError) as e:
        d2f.d2f_kv_commit(x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], prefix, 0, 16,
                          block=1)
    assert e.value.status == 3 and prefix == [16]
    d2f.d2f_kv_commit(x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], prefix, 0, 16)
    d2f.d2f_kv_commit(x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], prefix, 0, 16)
    assert prefix == [48]
    with pytest.raises(d2f.D2FError) as e:   # capacity 48 is now full
        d2f.d2f_kv_commit(x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], prefix, 0, 16)
    assert e.value.status == 2


def _shift_in_fresh_block(shape, x, it, seed=0):
    """Window after its oldest block left: blocks 1.. move up one block, a
    fresh block (drawn with tid + 100 * it) takes the last slot."""
    B = shape.block_size
    for n in ("q", "k_win", "v_win"):
        t = x[n]
        t[:, :, :-B] = t[:, :, B:].clone()
        t[:, :, -B:] = W.fresh_block(shape, n, it, device="cuda", seed=seed)


# Scaled closeness of two bf16 attention outputs: mean |a - b| over mean |b|.
# The kernel's own error is a few 1e-3 of the output's size: the
# probabilities enter the PV product rounded to bf16 (relative error <= 2^-9
# each) and the output is rounded to bf16 once more; an fp64 simulation of
# exactly these roundings on this workload's shape gives 2.3e-3.  Dropping
# or replacing the 16 keys of one appended block among 32K changes a
# 32K-prefix output by about 2.0e-2 of its size (same simulation), so a bound
# of 6e-3 tells the two apart, where the absolute bf16 tolerance (2e-2
# against outputs of about 7e-3) cannot.  The measured values are printed.
REL_MEAN = 6e-3


def _rel_mean(a, b):
    return float((a - b).abs().mean() / b.abs().mean())


def test_llada_p32k_sequential_appends_reuse_exactness():
    """64 blocks appended in sequence to the 32K-prefix cache.  After every
    append: the cache's new rows equal the window block byte for byte; the
    window slides by one block and the surviving rows' outputs are compared
    with those computed before the append (exact reuse); one query head,
    rotating through all 32, is checked against the oracle on the grown
    cache."""
    import block_causal_attention_d2f_amd as d2f
    c = W.config("llada_p32k")
    sh = c["shape"]
    B = sh.block_size
    x = W.attn_inputs(sh, device="cuda")
    prefix = list(sh.prefix_len)
    pdev = torch.tensor(prefix, dtype=torch.int32, device="cuda")
    out_prev, lse_prev = run_attn(sh, x)
    worst_drift = worst_rel = worst_oracle = 0.0
    for it in range(c["n_kv_commits"]):
        p0 = prefix[0]
        k_blk = x["k_win"][0, :, :B].clone()
        v_blk = x["v_win"][0, :, :B].clone()
        d2f.d2f_kv_commit(x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], prefix, 0, B,
                          prefix_len_dev=pdev)
        torch.cuda.synchronize()
        assert prefix[0] == p0 + B, it
        assert torch.equal(x["k_cache"][0, :, p0:p0 + B].view(torch.uint8),
                           k_blk.view(torch.uint8)), it
        assert torch.equal(x["v_cache"][0, :, p0:p0 + B].view(torch.uint8),
                           v_blk.view(torch.uint8)), it
        _shift_in_fresh_block(sh, x, it)
        sh.prefix_len = list(prefix)
        out, lse = run_attn(sh, x)
        # Surviving rows (old blocks 1..3 are now blocks 0..2): same outputs.
        a = out[:, :, :-B].float()
        b = out_prev[:, :, B:].float()
        diff = (a - b).abs()
        rel = _rel_mean(a, b)
        worst_drift = max(worst_drift, float(diff.max()))
        worst_rel = max(worst_rel, rel)
        assert float(diff.max()) <= 2e-2 and float(diff.mean()) <= 2e-3, (it, float(diff.max()))
        assert rel <= REL_MEAN, (it, rel)
        assert float((lse[:, :, :-B] - lse_prev[:, :, B:]).abs().max()) <= 1e-3
        # The oracle on the grown cache, one head per append (all 32 twice).
        h = it % sh.n_heads_q
        pairs = [(0, h)]
        ro, rl = oracle_attn(sh, x, pairs=pairs)
        compare_attn(sh, out, lse, ro, rl, pairs=pairs, label=f"llada_p32k-append{it}-h{h}")
        W_rows = sh.win_rows(0)
        g = out[0, h, :W_rows].float().cpu().double()
        r = torch.as_tensor(ro[0, h, :W_rows])
        rel_o = float((g - r).abs().mean() / r.abs().mean())
        worst_oracle = max(worst_oracle, rel_o)
        assert rel_o <= REL_MEAN, (it, h, rel_o)
        out_prev, lse_prev = out, lse
    assert prefix == [32768 + 64 * B] and pdev.cpu().tolist() == prefix
    say(f"[llada_p32k appends] 64 appends ok, worst surviving-row drift {worst_drift:.3e} "
        f"(mean/mean {worst_rel:.2e}), worst oracle mean/mean {worst_oracle:.2e}")


def test_reuse_oracle_vs_gpu_small():
    """Kept-in-window vs appended-to-cache on a small shape, both on the GPU
    and in the oracle (the oracle's two results are bit-identical)."""
    import block_causal_attention_d2f_amd as d2f
    sh = W.make_shape(1, 4, 4, 128, 16, [300], [3], dtype="bf16", extra_capacity=16)
    x = W.attn_inputs(sh, device="cuda", seed=2)
    o1, l1 = run_attn(sh, x)
    r1, _ = oracle_attn(sh, x)
    prefix = list(sh.prefix_len)
    d2f.d2f_kv_commit(x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], prefix, 0, 16)
    y = {k: v.clone() for k, v in x.items()}
    for n in ("q", "k_win", "v_win"):
        y[n] = torch.as_tensor(np.nan_to_num(OK.drop_oldest_block(y[n].float().cpu().numpy(), 0, 16)),
                               device="cuda").to(x[n].dtype)
    sh2 = W.make_shape(1, 4, 4, 128, 16, prefix, [2], dtype="bf16", max_win_blocks=3,
                       cache_capacity=sh.cache_capacity)
    o2, l2 = run_attn(sh2, y)
    r2, _ = oracle_attn(sh2, y)
    assert np.array_equal(r2[:, :, :32], r1[:, :, 16:])
    d = (o2[:, :, :32].float() - o1[:, :, 16:].float()).abs()
    assert float(d.max()) <= 2e-2
