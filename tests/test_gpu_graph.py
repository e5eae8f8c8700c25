"""The three calls captured into a HIP graph give, on every replay, the same
bits as the eager calls (the benchmark times the step this way)."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import block_causal_attention_d2f_amd as d2f
    c = W.config("llada_p512")
    sh = c["shape"]
    x = W.attn_inputs(sh, device="cuda", seed=4)
    ci = W.config_commit_inputs(c, device="cuda", seed=4)
    out = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
    desc = d2f.make_desc(sh.batch, sh.n_heads_q, sh.n_heads_kv, sh.head_dim, sh.block_size,
                         sh.max_win_blocks, sh.cache_capacity, x["q"].dtype)
    ws_a = torch.empty(max(256, d2f.d2f_block_attn_workspace_size(desc, sh.prefix_len,
                                                                 sh.n_win_blocks)),
                       dtype=torch.uint8, device="cuda")
    rows = W.total_rows(sh)
    ws_c = torch.empty(d2f.d2f_confidence_commit_workspace_size(rows, c["vocab"]),
                       dtype=torch.uint8, device="cuda")
    ms, tok = ci.mask_state.clone(), ci.tokens.clone()
    nc = torch.empty(rows // sh.block_size, dtype=torch.int32, device="cuda")
    bc = torch.empty(rows // sh.block_size, dtype=torch.uint8, device="cuda")
    conf = torch.empty(rows, dtype=torch.float32, device="cuda")
    am = torch.empty(rows, dtype=torch.int32, device="cuda")
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    # A second attention call with a long prefix: its keys are split across
    # workgroups and merged by a second kernel inside the graph.
    sh2 = W.make_shape(1, 8, 8, 128, 16, [8192], [2], dtype="bf16")
    x2 = W.attn_inputs(sh2, device="cuda", seed=5)
    out2 = torch.empty_like(x2["q"])
    lse2 = torch.empty(x2["q"].shape[:3], dtype=torch.float32, device="cuda")
    desc2 = d2f.make_desc(sh2.batch, sh2.n_heads_q, sh2.n_heads_kv, sh2.head_dim, sh2.block_size,
                          sh2.max_win_blocks, sh2.cache_capacity, x2["q"].dtype)
    need2 = d2f.d2f_block_attn_workspace_size(desc2, sh2.prefix_len, sh2.n_win_blocks)
    assert need2 > 0
    ws_a2 = torch.empty(need2, dtype=torch.uint8, device="cuda")

    def step():
        d2f.d2f_block_attn(x["q"], kc, vc, x["k_win"], x["v_win"], sh.prefix_len,
                           sh.n_win_blocks, sh.block_size, out=out, lse=lse, workspace=ws_a)
        d2f.d2f_confidence_commit(ci.logits, ms, tok, ci.block_phase, sh.block_size, 0.9, 1,
                                  ci.mask_token_id, conf_out=conf, argmax_out=am, n_committed=nc,
                                  block_complete=bc, workspace=ws_c)
        d2f.d2f_kv_commit(kc, vc, x["k_win"], x["v_win"], list(sh.prefix_len), 0, sh.block_size)
        d2f.d2f_block_attn(x2["q"], x2["k_cache"], x2["v_cache"], x2["k_win"], x2["v_win"],
                           sh2.prefix_len, sh2.n_win_blocks, sh2.block_size, out=out2, lse=lse2,
                           workspace=ws_a2)

    def snapshot():
        return [t.clone() for t in (out, lse, ms, tok, nc, bc, conf, am, kc, vc, out2, lse2)]

    def reset():
        ms.copy_(ci.mask_state)
        tok.copy_(ci.tokens)
        for t in (out, lse, conf, out2, lse2):
            t.fill_(0.0)

    reset()
    step()
    torch.cuda.synchronize()
    eager = snapshot()
    g = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(eager, got):
            assert torch.equal(a, b), f"replay {i} differs from the eager step"
        # unrelated eager work between replays
        y = torch.randn(1 << 20, device="cuda").sum()
        assert torch.isfinite(y)


def test_graph_replays_of_the_other_calls():
    """Paged attention and the paged persist, the commit pass under another
    measure with Prophet's early commit, and attention in segments with the
    join: captured together, every replay equals the eager calls.
    (d2f_decode_advance synchronises the stream to read the commit counts, so
    it is not captured.)"""
    import block_causal_attention_d2f_amd as d2f
    from test_gpu_paged import to_pages
    B = 16
    sh = W.make_shape(2, 8, 4, 128, B, [256, 96], [3, 2], dtype="bf16", extra_capacity=64)
    x = W.attn_inputs(sh, device="cuda", seed=21)
    kp, vp, pt0, wp0 = to_pages(sh, x, seed=22, spare=2)
    pt, wp = pt0.clone(), wp0.clone()
    o_p = torch.empty_like(x["q"])
    l_p = torch.empty(x["q"].shape[:3], device="cuda")
    o_r, l_r = torch.empty_like(o_p), torch.empty_like(l_p)
    o_w, l_w = torch.empty_like(o_p), torch.empty_like(l_p)
    o_c, l_c = torch.empty_like(o_p), torch.empty_like(l_p)
    ws = torch.empty(16 << 20, dtype=torch.uint8, device="cuda")
    phases = [W.AGGRESSIVE, W.AGGRESSIVE, W.CONSERVATIVE, W.AGGRESSIVE, W.CONSERVATIVE]
    ci = W.commit_inputs(5 * B, 20000, B, phases, 3.0, True, committed_frac=0.2, device="cuda",
                         seed=23)
    ms, tok = ci.mask_state.clone(), ci.tokens.clone()
    nc = torch.empty(5, dtype=torch.int32, device="cuda")
    bc = torch.empty(5, dtype=torch.uint8, device="cuda")
    conf = torch.empty(5 * B, device="cuda")
    am = torch.empty(5 * B, dtype=torch.int32, device="cuda")
    wsc = torch.empty(d2f.d2f_confidence_commit_workspace_size(5 * B, 20000), dtype=torch.uint8,
                      device="cuda")
    early = torch.tensor([0.5, 9.0], device="cuda")
    pdev = torch.zeros(2, dtype=torch.int32, device="cuda")

    def step():
        d2f.d2f_block_attn_paged(x["q"], kp, vp, pt, wp, sh.prefix_len, sh.n_win_blocks, out=o_p,
                                 lse=l_p, workspace=ws)
        d2f.d2f_kv_commit_paged(pt, wp, list(sh.prefix_len), 1, B, n_heads_kv=4,
                                prefix_len_dev=pdev)
        d2f.d2f_confidence_commit(ci.logits, ms, tok, ci.block_phase, B, 0.8, 1, ci.mask_token_id,
                                  conf_out=conf, argmax_out=am, n_committed=nc, block_complete=bc,
                                  workspace=wsc, measure="margin", early_gap=early,
                                  early_group_blocks=3)
        d2f.d2f_block_attn_range(x["q"], x["k_cache"], x["v_cache"], [0, 0], sh.prefix_len,
                                 sh.n_win_blocks, B, out=o_r, lse=l_r, workspace=ws)
        d2f.d2f_block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"], [0, 0],
                           sh.n_win_blocks, B, out=o_w, lse=l_w, workspace=ws)
        d2f.d2f_attn_combine(o_r, l_r, o_w, l_w, sh.n_win_blocks, B, out=o_c, lse=l_c)

    def reset():
        pt.copy_(pt0)
        wp.copy_(wp0)
        ms.copy_(ci.mask_state)
        tok.copy_(ci.tokens)
        for t in (o_p, l_p, o_r, l_r, o_w, l_w, o_c, l_c, conf):
            t.fill_(0.0)
        pdev.zero_()

    def snapshot():
        return [t.clone() for t in (o_p, l_p, pt, wp, pdev, ms, tok, nc, bc, conf, am, o_c, l_c)]

    reset()
    step()
    torch.cuda.synchronize()
    eager = snapshot()
    g = torch.cuda.CUDAGraph()
    reset()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, snapshot()):
            assert torch.equal(a, b), f"replay {i} differs from the eager calls"
        y = torch.randn(1 << 20, device="cuda").sum()
        assert torch.isfinite(y)
