"""The three calls captured into a HIP graph give, on every replay, the same
bits as the eager calls (the benchmark times the step this way)."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import block_causal_attention_d2f_amd as d2f
    c = W.config("cfg2")
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

    def step():
        d2f.d2f_block_attn(x["q"], kc, vc, x["k_win"], x["v_win"], sh.prefix_len,
                           sh.n_win_blocks, sh.block_size, out=out, lse=lse, workspace=ws_a)
        d2f.d2f_confidence_commit(ci.logits, ms, tok, ci.block_phase, sh.block_size, 0.9, 1,
                                  ci.mask_token_id, conf_out=conf, argmax_out=am, n_committed=nc,
                                  block_complete=bc, workspace=ws_c)
        d2f.d2f_kv_commit(kc, vc, x["k_win"], x["v_win"], list(sh.prefix_len), 0, sh.block_size)

    def snapshot():
        return [t.clone() for t in (out, lse, ms, tok, nc, bc, conf, am, kc, vc)]

    def reset():
        ms.copy_(ci.mask_state)
        tok.copy_(ci.tokens)
        for t in (out, lse, conf):
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
