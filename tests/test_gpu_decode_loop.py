"""Multi-step D2F decoding with the active-window schedule, run through the
library (attention per layer, the commit pass, d2f_decode_advance) and, on
the same synthetic inputs, through the oracle (attention, commit, window
schedule, KV append), step by step.

Compared at every step: attention outputs and LSE (bf16 tolerances), the
commit decisions (bit-exact; the inputs are checked to hold no near-threshold
ties), per-block commit counts, the schedule's transitions and phases, the
device slot rows (mask state, tokens, phases) and the prefix lengths.  At the
end: the decoded sequences and the KV caches of every layer (byte-exact)."""
import numpy as np
import pytest
import torch

import block_causal_attention_d2f_amd as d2f
import workloads as W
from oracle import attention as OA
from oracle import commit as OC
from oracle import kv_cache as OK
from oracle import window as OW
from parity import LSE_BF16, MAX_BF16, MEAN_BF16, say

pytestmark = pytest.mark.gpu

MASK_ID = 126336
MASKED, COMMITTED = 0, 1


def _run(nb, hq, hkv, d, B, mw, total, prompt, vocab, tau, k_aggr, tau_add, tau_act, layers,
         seed, paged=False):
    dev = "cuda"
    cap = max(prompt) + total * B
    wmax = mw * B
    g = torch.Generator().manual_seed(seed)
    kc0 = torch.randn((layers, nb, hkv, cap, d), generator=g).to(torch.bfloat16)
    vc0 = torch.randn((layers, nb, hkv, cap, d), generator=g).to(torch.bfloat16)
    kc, vc = kc0.to(dev), vc0.to(dev)
    okc = kc0.float().numpy().copy()          # bf16 values are exact in f32
    ovc = vc0.float().numpy().copy()
    q = torch.zeros((layers, nb, hq, wmax, d), dtype=torch.bfloat16, device=dev)
    kw = torch.zeros((layers, nb, hkv, wmax, d), dtype=torch.bfloat16, device=dev)
    vw = torch.zeros_like(kw)
    out = torch.zeros((nb, hq, wmax, d), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((nb, hq, wmax), dtype=torch.float32, device=dev)
    # device slot state, set up as the header asks before the first step
    ms = torch.full((nb, wmax), COMMITTED, dtype=torch.uint8)
    ms[:, :B] = MASKED
    ms = ms.reshape(-1).to(dev)
    tk = torch.full((nb * wmax,), MASK_ID, dtype=torch.int32, device=dev)
    ph = torch.zeros((nb, mw), dtype=torch.uint8)
    ph[:, 0] = 1
    ph = ph.reshape(-1).to(dev)
    ncd = torch.zeros(nb * mw, dtype=torch.int32, device=dev)
    outt = torch.full((nb, total * B), -1, dtype=torch.int32, device=dev)
    logits = torch.full((nb * wmax, vocab), float("nan"), dtype=torch.float32)
    P, oP = list(prompt), list(prompt)
    if paged:
        # one page per block, randomly numbered; the prompt's pages first,
        # then a free list from which every appended block takes one
        assert all(p % B == 0 for p in prompt)
        n_pages = sum(p // B for p in prompt) + nb * (total + 1) + 3
        order = torch.randperm(n_pages, generator=torch.Generator().manual_seed(seed + 77)).tolist()
        kp = torch.full((layers, n_pages, hkv, B, d), float("nan"), dtype=torch.bfloat16,
                        device=dev)
        vp = torch.full_like(kp, float("nan"))
        ts = max(prompt) // B + total
        pt = torch.full((nb, ts), -1, dtype=torch.int32)
        wpg = torch.full((nb, mw), -1, dtype=torch.int32)
        for b in range(nb):
            for i in range(prompt[b] // B):
                pg = order.pop()
                pt[b, i] = pg
                kp[:, pg] = kc[:, b, :, i * B:(i + 1) * B]
                vp[:, pg] = vc[:, b, :, i * B:(i + 1) * B]
            wpg[b, 0] = order.pop()
        pt, wpg = pt.to(dev), wpg.to(dev)
        free = order
    wins = [d2f.Window(B, mw, total, tau_add, tau_act) for _ in range(nb)]
    owins = [OW.Window(B, mw, total, tau_add, tau_act) for _ in range(nb)]
    omask = [np.zeros(B, np.uint8) for _ in range(nb)]
    otok = [np.full(B, MASK_ID, np.int64) for _ in range(nb)]
    odec = [[] for _ in range(nb)]
    born = [{0: 0} for _ in range(nb)]
    step, worst = 0, 0.0
    while not all(w.done for w in owins):
        assert step < 60 * total, "decoding did not finish"
        live = [b for b in range(nb) if not owins[b].done]
        nwin = [owins[b].n_win for b in range(nb)]   # 0 once a request is finished (idle)
        # -- attention, every layer ----------------------------------------------------
        for l in range(layers):
            for b in live:
                pos = [owins[b].first * B + r for r in range(owins[b].n_win * B)]
                s = seed + 1000 * l + b
                q[l, b, :, :len(pos)] = W.decode_window_kv(hq, d, pos, step, 1, seed=s).to(dev)
                kw[l, b, :, :len(pos)] = W.decode_window_kv(hkv, d, pos, step, 2, seed=s).to(dev)
                vw[l, b, :, :len(pos)] = W.decode_window_kv(hkv, d, pos, step, 3, seed=s).to(dev)
            pl_attn = list(P)
            if paged:
                wh = wpg.cpu()
                for b in live:   # the model writes the window's K/V into its pages
                    for k in range(owins[b].n_win):
                        pg = int(wh[b, k])
                        kp[l, pg] = kw[l, b, :, k * B:(k + 1) * B]
                        vp[l, pg] = vw[l, b, :, k * B:(k + 1) * B]
                d2f.d2f_block_attn_paged(q[l], kp[l], vp[l], pt, wpg, pl_attn, nwin, out=out,
                                         lse=lse)
            else:
                d2f.d2f_block_attn(q[l], kc[l], vc[l], kw[l], vw[l], pl_attn, nwin, B, out=out,
                                   lse=lse)
            torch.cuda.synchronize()
            ro, rl = OA.block_attn(q[l].cpu(), okc[l], ovc[l], kw[l].cpu(), vw[l].cpu(), pl_attn,
                                   nwin, B, pairs=[(b, h) for b in live for h in range(hq)])
            for b in live:
                rows = owins[b].n_win * B
                err = np.abs(out[b, :, :rows].float().cpu().numpy() - ro[b, :, :rows])
                worst = max(worst, float(err.max()))
                assert err.max() <= MAX_BF16 and err.mean() <= MEAN_BF16, (step, l, b)
                lerr = np.abs(lse[b, :, :rows].cpu().numpy() - rl[b, :, :rows]).max()
                assert lerr <= LSE_BF16, (step, l, b, lerr)
        # -- commit pass over every slot ---------------------------------------------------
        o_rows, o_phase = [], []
        for b in live:
            pos = [owins[b].first * B + r for r in range(owins[b].n_win * B)]
            ages = [step - born[b][p // B] for p in pos]
            logits[b * wmax:b * wmax + len(pos)] = W.decode_rows(vocab, pos, ages, step,
                                                                 seed=seed + 10 * b)
            o_rows.extend(range(b * wmax, b * wmax + len(pos)))
            o_phase.extend(owins[b].phase)
        ref = OC.confidence_commit(logits[o_rows], np.concatenate([omask[b] for b in live]),
                                   np.concatenate([otok[b] for b in live]), np.array(o_phase),
                                   B, tau, k_aggr, MASK_ID)
        assert not ref["near_tau"].any() and not ref["near_topk"].any(), \
            "synthetic inputs hold a near tie; pick another seed"
        res = d2f.d2f_confidence_commit(logits.to(dev), ms, tk, ph, B, tau, k_aggr, MASK_ID,
                                        n_committed=ncd)
        ms_h, tk_h = ms.cpu().numpy(), tk.cpu().numpy().astype(np.int64)
        nc_h = ncd.cpu().numpy()
        o = 0
        for b in live:
            n = owins[b].n_win
            sl = slice(o * B, (o + n) * B)
            assert np.array_equal(ms_h[b * wmax:b * wmax + n * B], ref["mask_state"][sl]), step
            assert np.array_equal(tk_h[b * wmax:b * wmax + n * B], ref["tokens"][sl]), step
            assert np.array_equal(nc_h[b * mw:b * mw + n], ref["n_committed"][o:o + n]), step
            omask[b], otok[b] = ref["mask_state"][sl].copy(), ref["tokens"][sl].copy()
            o += n
        del res
        # -- the step's bookkeeping ----------------------------------------------------------
        okw = kw.float().cpu().numpy()
        ovw = vw.float().cpu().numpy()
        if paged:
            new_pages = [free.pop() for _ in range(nb)]
            pers, app = d2f.d2f_decode_advance_paged(pt, wpg, new_pages, wins, P, ncd, ms, tk, ph,
                                                     outt, MASK_ID, n_heads_kv=hkv, head_dim=d)
            free.extend(pg for pg, a in zip(new_pages, app) if not a)
        else:
            pers, app = d2f.d2f_decode_advance(kc, vc, kw, vw, wins, P, ncd, ms, tk, ph, outt,
                                               MASK_ID)
        o = 0
        for b in range(nb):
            if owins[b].done:
                assert (pers[b], app[b]) == (0, 0)
                continue
            n = owins[b].n_win
            ncb = [int(x) for x in ref["n_committed"][o:o + n]]
            o += n
            p, a = owins[b].after_commit(ncb)
            assert (pers[b], app[b]) == (p, a), (step, b)
            for _ in range(p):
                for l in range(layers):
                    okc[l], ovc[l], pl2 = OK.kv_commit(okc[l], ovc[l], okw[l], ovw[l], oP, b, B)
                    okw[l] = OK.drop_oldest_block(okw[l], b, B)
                    ovw[l] = OK.drop_oldest_block(ovw[l], b, B)
                oP = pl2
                odec[b].extend(int(t) for t in otok[b][:B])
                omask[b], otok[b] = omask[b][B:], otok[b][B:]
            if a:
                born[b][owins[b].first + owins[b].n_win - 1] = step + 1
                omask[b] = np.concatenate([omask[b], np.full(B, MASKED, np.uint8)])
                otok[b] = np.concatenate([otok[b], np.full(B, MASK_ID, np.int64)])
        assert P == oP, step
        ms_h, tk_h, ph_h = ms.cpu().numpy(), tk.cpu().numpy(), ph.cpu().numpy()
        for b in range(nb):
            w, ow = wins[b], owins[b]
            assert (w.first, w.n_win, w.started, w.persisted, w.committed, w.phase) == \
                   (ow.first, ow.n_win, ow.started, ow.persisted, ow.committed, ow.phase), (step, b)
            n = ow.n_win * B
            assert np.array_equal(ms_h[b * wmax:b * wmax + n], omask[b])
            assert np.array_equal(tk_h[b * wmax:b * wmax + n], otok[b])
            assert (ms_h[b * wmax + n:(b + 1) * wmax] == COMMITTED).all()
            assert (tk_h[b * wmax + n:(b + 1) * wmax] == MASK_ID).all()
            assert list(ph_h[b * mw:(b + 1) * mw]) == list(ow.phase) + [0] * (mw - ow.n_win)
        step += 1
    # -- end state -------------------------------------------------------------------------
    outh = outt.cpu().numpy()
    for b in range(nb):
        assert len(odec[b]) == total * B and MASK_ID not in odec[b]
        assert list(outh[b]) == odec[b]
        assert P[b] == prompt[b] + total * B
    if paged:   # the cache is the pages the table lists, in order
        pth = pt.cpu()
        for b in range(nb):
            ids = [int(i) for i in pth[b, :P[b] // B]]
            assert -1 not in ids and len(set(ids)) == len(ids)
            gk = torch.cat([kp[:, i] for i in ids], dim=2).float().cpu().numpy()
            gv = torch.cat([vp[:, i] for i in ids], dim=2).float().cpu().numpy()
            assert np.array_equal(gk, okc[:, b, :, :P[b]])
            assert np.array_equal(gv, ovc[:, b, :, :P[b]])
        assert (wpg.cpu() == -1).all()
    else:
        assert np.array_equal(kc.float().cpu().numpy(), okc)
        assert np.array_equal(vc.float().cpu().numpy(), ovc)
    tokens = nb * total * B
    say(f"[decode-loop{' paged' if paged else ''}] nb={nb} L={layers} B={B} window={mw} "
        f"blocks={total}: {step} steps, "
        f"{tokens / step:.2f} tokens per step, worst attention error {worst:.2e}")
    return step


@pytest.mark.parametrize("case", [
    # nb, hq, hkv, d, B, window, total, prompt, vocab, tau, k_aggr, tau_add, tau_act, layers, seed
    (1, 4, 2, 64, 16, 3, 5, [40], 3000, 0.9, 2, 0.25, 0.75, 2, 1),
    (2, 4, 4, 128, 16, 4, 4, [64, 23], 2000, 0.9, 1, 0.1, 0.95, 1, 2),
    (1, 2, 1, 64, 8, 1, 4, [17], 1500, 0.8, 3, 0.5, 0.5, 1, 3),      # one-block window
    (3, 2, 2, 64, 4, 2, 3, [0, 9, 5], 800, 0.95, 1, 0.0, 0.3, 1, 4),  # empty prompt, tau_add 0
], ids=["two-layers", "gqa-free-d128", "one-block-window", "three-requests"])
def test_decode_loop_matches_oracle(case):
    nb, hq, hkv, d, B, mw, total, prompt, vocab, tau, k, ta, tc, layers, seed = case
    say(f"[decode-loop] start {case}")
    steps = _run(nb, hq, hkv, d, B, mw, total, prompt, vocab, tau, k, ta, tc, layers, seed)
    assert steps >= total


def test_decode_loop_more_requests_than_one_launch():
    """70 requests: the bookkeeping runs as two launches (64 + 6 requests)."""
    say("[decode-loop] start 70 requests")
    prompt = [(7 * b) % 23 for b in range(70)]
    _run(70, 2, 1, 64, 4, 2, 2, prompt, 300, 0.9, 1, 0.25, 0.75, 1, 5)


@pytest.mark.parametrize("case", [
    # nb, hq, hkv, d, B, window, total, prompt, vocab, tau, k_aggr, tau_add, tau_act, layers, seed
    (2, 4, 2, 64, 16, 3, 5, [48, 16], 3000, 0.9, 2, 0.25, 0.75, 2, 6),
    (3, 8, 8, 128, 8, 2, 4, [0, 24, 8], 2000, 0.9, 1, 0.1, 0.9, 1, 7),
], ids=["paged-two-layers", "paged-B8"])
def test_paged_decode_loop_matches_oracle(case):
    """The same loop over a paged cache: window blocks live in pages, the
    persist moves page ids, and the cache gathered through the page table
    equals the oracle's byte for byte."""
    nb, hq, hkv, d, B, mw, total, prompt, vocab, tau, k, ta, tc, layers, seed = case
    say(f"[decode-loop paged] start {case}")
    _run(nb, hq, hkv, d, B, mw, total, prompt, vocab, tau, k, ta, tc, layers, seed, paged=True)



def _draw_loop(seed, paged):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(1, 6))
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4]))
    B = int(rng.choice([8, 16] if paged else [2, 4, 8, 16]))
    mw = int(rng.integers(1, 5))
    total = int(rng.integers(mw, mw + 4))
    prompt = [int(rng.integers(0, 6)) * B if paged else int(rng.integers(0, 80)) for _ in range(nb)]
    return (nb, hq, hkv, int(rng.choice([64, 128])), B, mw, total, prompt,
            int(rng.integers(500, 4000)), float(rng.choice([0.8, 0.9, 0.95])),
            int(rng.integers(1, 4)), float(rng.choice([0.0, 0.25, 0.5])),
            float(rng.choice([0.3, 0.75, 0.95])), int(rng.integers(1, 3)), seed)


@pytest.mark.parametrize("paged", [False, True], ids=["contiguous", "paged"])
@pytest.mark.parametrize("k", range(2))
def test_random_decode_loops_match_oracle(paged, k):
    """Seeded random loops: batch, heads, block size, window, sequence length,
    prompts (whole blocks when paged), vocabulary, thresholds, k_aggr, layers."""
    case = _draw_loop(13000 + 10 * k + (5 if paged else 0), paged)
    say(f"[decode-loop random] start {case} paged={paged}")
    nb, hq, hkv, d, B, mw, total, prompt, vocab, tau, ka, ta, tc, layers, seed = case
    steps = _run(nb, hq, hkv, d, B, mw, total, prompt, vocab, tau, ka, ta, tc, layers, seed,
                 paged=paged)
    assert steps >= total
