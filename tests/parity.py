"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
and compare with the fp64 oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

import workloads as W
from oracle import attention as OA
from oracle import commit as OC

# Tolerances, from the statement of the target:
#   fp32 inputs:             max |gpu - oracle| <= 1e-5
#   bf16 inputs, fp32 accum: max <= 2e-2 and mean <= 2e-3
ATOL_F32 = 1e-5
MAX_BF16 = 2e-2
MEAN_BF16 = 2e-3
# LSE: fp32 path as above; the bf16 path's scores are exact bf16 products
# summed in fp32, so the normaliser is held to a tight 1e-3.
LSE_F32 = 1e-5
LSE_BF16 = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_attn(shape, x, out_fill=None, softmax_scale=0.0):
    import block_causal_attention_d2f_amd as d2f
    out = lse = None
    if out_fill is not None:
        out = torch.full_like(x["q"], out_fill)
        lse = torch.full(x["q"].shape[:3], out_fill, dtype=torch.float32, device=x["q"].device)
    out, lse = d2f.d2f_block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"],
                                  shape.prefix_len, shape.n_win_blocks, shape.block_size,
                                  out=out, lse=lse, softmax_scale=softmax_scale)
    torch.cuda.synchronize()
    return out, lse


def oracle_attn(shape, x, pairs=None, scale=None):
    return OA.block_attn(x["q"], x["k_cache"], x["v_cache"], x["k_win"], x["v_win"],
                         shape.prefix_len, shape.n_win_blocks, shape.block_size, scale=scale,
                         pairs=pairs)


def valid_rows_mask(shape):
    m = np.zeros((shape.batch, shape.n_heads_q, shape.w_max), bool)
    for b in range(shape.batch):
        m[b, :, :shape.win_rows(b)] = True
    return m


def compare_attn(shape, out, lse, ref_out, ref_lse, pairs=None, label=""):
    """Element-wise comparison over the valid rows of the compared (b, h)."""
    sel = valid_rows_mask(shape)
    if pairs is not None:
        keep = np.zeros_like(sel)
        for b, h in pairs:
            keep[b, h] = sel[b, h]
        sel = keep
    got = out.detach().float().cpu().double().numpy()[sel]
    want = ref_out[sel]
    assert np.isfinite(got).all(), f"{label}: non-finite outputs"
    err = np.abs(got - want)
    gl = lse.detach().cpu().double().numpy()[sel]
    lerr = np.abs(gl - ref_lse[sel])
    stats = dict(max=float(err.max()), mean=float(err.mean()), lse_max=float(lerr.max()),
                 n=int(err.size))
    say(f"[attn {label}] dtype={shape.dtype} max={stats['max']:.3e} mean={stats['mean']:.3e} "
        f"lse_max={stats['lse_max']:.3e} n={stats['n']}")
    if shape.dtype == "f32":
        assert stats["max"] <= ATOL_F32, stats
        assert stats["lse_max"] <= LSE_F32, stats
    else:
        assert stats["max"] <= MAX_BF16, stats
        assert stats["mean"] <= MEAN_BF16, stats
        assert stats["lse_max"] <= LSE_BF16, stats
    return stats


def run_commit(ci, tau, k_aggr, device="cuda", measure="maxprob", early_gap=None,
               early_group_blocks=0):
    import block_causal_attention_d2f_amd as d2f
    ms = ci.mask_state.to(device).clone()
    tok = ci.tokens.to(device).clone()
    res = d2f.d2f_confidence_commit(ci.logits, ms, tok, ci.block_phase.to(device), ci.block_size,
                                    tau, k_aggr, ci.mask_token_id, measure=measure,
                                    early_gap=early_gap, early_group_blocks=early_group_blocks)
    torch.cuda.synchronize()
    return dict(mask_state=ms.cpu().numpy(), tokens=tok.cpu().numpy().astype(np.int64),
                n_committed=res["n_committed"].cpu().numpy(),
                block_complete=res["block_complete"].cpu().numpy(),
                conf=res["conf"].cpu().double().numpy(),
                argmax=res["argmax"].cpu().numpy().astype(np.int64))


def compare_commit(ci, got, tau, k_aggr, blocks=None, label="", measure="maxprob",
                   early_gap=None, early_group_blocks=0):
    """Bit-exact comparison of argmax and every decision, except rows whose
    fp64 confidence lies within the measure's band (1e-6 for probabilities)
    of tau, aggressive blocks whose k-th / (k+1)-th confidences are that
    close, and early-commit groups whose smallest gap is that close to the
    threshold (all counted and reported).  ``blocks`` restricts the oracle
    to a subset of blocks (not with the early commit)."""
    B = ci.block_size
    n_blocks = ci.mask_state.shape[0] // B
    assert blocks is None or early_gap is None
    blocks = list(range(n_blocks)) if blocks is None else list(blocks)
    rows = np.concatenate([np.arange(k * B, (k + 1) * B) for k in blocks])
    rows_t = torch.as_tensor(rows, device=ci.logits.device)
    ref = OC.confidence_commit(ci.logits.index_select(0, rows_t), ci.mask_state.cpu()[rows],
                               ci.tokens.cpu()[rows], ci.block_phase.cpu()[blocks], B, tau, k_aggr,
                               ci.mask_token_id, measure=measure, early_gap=early_gap,
                               early_group_blocks=early_group_blocks)
    near_row = ref["near_tau"].copy()
    near_blk = ref["near_topk"].copy()
    gb = early_group_blocks if early_group_blocks else len(blocks)
    for g in np.flatnonzero(ref["near_early"]):
        near_blk[g * gb:(g + 1) * gb] = True
    for j in range(len(blocks)):
        if near_blk[j]:
            near_row[j * B:(j + 1) * B] = True
    ok = ~near_row
    live = ~np.isnan(ref["conf"])
    g = {k: got[k][rows] for k in ("mask_state", "tokens", "conf", "argmax")}
    assert (g["argmax"][live] == ref["argmax"][live]).all(), f"{label}: argmax differs"
    assert (g["argmax"][~live] == -1).all(), f"{label}: committed rows were written"
    assert (g["mask_state"][ok] == ref["mask_state"][ok]).all(), f"{label}: mask_state differs"
    assert (g["tokens"][ok] == ref["tokens"][ok]).all(), f"{label}: tokens differ"
    blk_ok = np.array([not near_row[j * B:(j + 1) * B].any() for j in range(len(blocks))], bool)
    bsel = np.array(blocks)
    assert (got["n_committed"][bsel][blk_ok] == ref["n_committed"][blk_ok]).all(), label
    assert (got["block_complete"][bsel][blk_ok] == ref["block_complete"][blk_ok]).all(), label
    fin = live & np.isfinite(ref["conf"])
    cerr = float(np.abs(g["conf"][fin] - ref["conf"][fin]).max()) if fin.any() else 0.0
    # a one-entry row has an infinite logit gap on both sides
    assert (g["conf"][live & ~fin] == ref["conf"][live & ~fin]).all(), f"{label}: conf differs"
    stats = dict(rows=len(rows), live=int(live.sum()), near_tau=int(ref["near_tau"].sum()),
                 near_topk=int(ref["near_topk"].sum()), near_early=int(ref["near_early"].sum()),
                 early=int(ref["early"].sum()), conf_max_err=cerr,
                 committed=int(ref["n_committed"].sum()))
    say(f"[commit {label}] {stats}")
    # conf itself: within the measure's decision band (1e-6 for probabilities)
    assert cerr <= OC.NEAR[measure], stats
    return stats


def poisoned_inputs(shape, seed=0, layer=0):
    return W.attn_inputs(shape, layer=layer, device="cuda", seed=seed, poison=True)


def to_pages(sh, x, seed, spare=3):
    """Scatter a contiguous cache and window into randomly numbered pages (on
    the device); unused pages hold NaN."""
    B, nb = sh.block_size, sh.batch
    hkv, d = x["k_cache"].shape[1], x["k_cache"].shape[3]
    need = sum(p // B for p in sh.prefix_len) + sum(sh.n_win_blocks)
    n_pages = need + spare
    g = torch.Generator().manual_seed(seed)
    perm = torch.randperm(n_pages, generator=g).tolist()
    kp = torch.full((n_pages, hkv, B, d), float("nan"), dtype=x["k_cache"].dtype, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    ts = max(p // B for p in sh.prefix_len) + 2
    pt = torch.full((nb, ts), -1, dtype=torch.int32)
    wp = torch.full((nb, sh.max_win_blocks), -1, dtype=torch.int32)
    for b in range(nb):
        for i in range(sh.prefix_len[b] // B):
            pg = perm.pop()
            pt[b, i] = pg
            kp[pg] = x["k_cache"][b, :, i * B:(i + 1) * B]
            vp[pg] = x["v_cache"][b, :, i * B:(i + 1) * B]
        for k in range(sh.n_win_blocks[b]):
            pg = perm.pop()
            wp[b, k] = pg
            kp[pg] = x["k_win"][b, :, k * B:(k + 1) * B]
            vp[pg] = x["v_win"][b, :, k * B:(k + 1) * B]
    return kp, vp, pt.cuda(), wp.cuda()
