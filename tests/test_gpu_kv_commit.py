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


def test_llada_p32k_sequential_appends_reuse_exactness():
    """64 blocks appended in sequence to the 32K-prefix cache.  After every
    append the window slides by one block; the surviving rows' outputs are
    compared with those computed before the append (exact reuse), and sampled
    heads are checked against the oracle on the grown cache."""
    import block_causal_attention_d2f_amd as d2f
    c = W.config("llada_p32k")
    sh = c["shape"]
    B = sh.block_size
    x = W.attn_inputs(sh, device="cuda")
    prefix = list(sh.prefix_len)
    pdev = torch.tensor(prefix, dtype=torch.int32, device="cuda")
    out_prev, lse_prev = run_attn(sh, x)
    worst = 0.0
    for it in range(c["n_kv_commits"]):
        d2f.d2f_kv_commit(x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], prefix, 0, B,
                          prefix_len_dev=pdev)
        _shift_in_fresh_block(sh, x, it)
        sh.prefix_len = list(prefix)
        out, lse = run_attn(sh, x)
        # Surviving rows (old blocks 1..3 are now blocks 0..2): same outputs.
        a = out[:, :, :-B].float()
        b = out_prev[:, :, B:].float()
        diff = (a - b).abs()
        worst = max(worst, float(diff.max()))
        assert float(diff.max()) <= 2e-2 and float(diff.mean()) <= 2e-3, (it, float(diff.max()))
        assert float((lse[:, :, :-B] - lse_prev[:, :, B:]).abs().max()) <= 1e-3
        if it in (0, 31, 63) or it % 8 == 3:
            h = (7 * it) % sh.n_heads_q
            pairs = [(0, h)]
            ro, rl = oracle_attn(sh, x, pairs=pairs)
            compare_attn(sh, out, lse, ro, rl, pairs=pairs, label=f"llada_p32k-append{it}-h{h}")
        out_prev, lse_prev = out, lse
    assert prefix == [32768 + 64 * B] and pdev.cpu().tolist() == prefix
    say(f"[llada_p32k appends] 64 appends ok, worst surviving-row drift {worst:.3e}")


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
