"""GPU parity of d2f_confidence_commit (through the C ABI) against the oracle:
argmax and every commit/remask decision bit-exact, near-ties reported."""
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from parity import compare_commit, run_commit, say

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg_case(name, bsz=None, tau=None, blocks=None):
    c = W.config(name, block_size=bsz)
    ci = W.config_commit_inputs(c, device="cuda")
    taus = c["taus"] if tau is None else [tau]
    for t in taus:
        got = run_commit(ci, t, c["k_aggr"])
        compare_commit(ci, got, t, c["k_aggr"], blocks=blocks, label=f"{name}-B{bsz}-tau{t}")


def test_tiny_f32():
    _cfg_case("tiny_f32")


def test_llada_p512_single_step():
    _cfg_case("llada_p512")


def test_llada_batch16():
    _cfg_case("llada_batch16")


@pytest.mark.parametrize("bsz", [16, 32, 64])
def test_dream_gqa_vocab(bsz):
    # every block of the 8 requests x 3 window blocks, at both thresholds
    _cfg_case("dream_gqa", bsz=bsz)


def test_llada_p32k_window_rows():
    _cfg_case("llada_p32k")


@pytest.mark.parametrize("vocab,ld_pad", [(1, 0), (7, 0), (513, 3), (8192, 0), (8193, 0),
                                          (20001, 5), (126464, 4)])
def test_vocab_sizes_and_strides(vocab, ld_pad):
    # vocab not a multiple of 4 and padded row strides take the scalar-load path
    rows, B = 32, 8
    g = torch.Generator(device="cuda").manual_seed(vocab)
    full = torch.randn((rows, vocab + ld_pad), generator=g, device="cuda") * 3
    logits = full[:, :vocab]
    phases = [W.AGGRESSIVE, W.CONSERVATIVE, W.AGGRESSIVE, W.CONSERVATIVE]
    ci = W.commit_inputs(rows, vocab, B, phases, 1.0, False, committed_frac=0.25,
                         device="cuda", seed=vocab)
    ci.logits = logits
    for tau in (0.0, 0.5, 0.9):
        got = run_commit(ci, tau, 2)
        compare_commit(ci, got, tau, 2, label=f"V{vocab}-ld{vocab + ld_pad}-tau{tau}")


def test_committed_rows_are_not_read_and_ties():
    rows, V, B = 16, 300, 4
    logits = torch.zeros((rows, V), device="cuda")
    logits[0, 5] = 2.0
    logits[0, 9] = 2.0           # tie: lowest index wins
    logits[1].fill_(1.5)         # all equal: conf = 1/V, argmax 0
    logits[2, 299] = 50.0        # last column, conf ~ 1
    logits[4:8] = float("nan")   # committed rows below: never read
    ms = torch.zeros(rows, dtype=torch.uint8)
    ms[4:8] = W.COMMITTED
    tok = torch.full((rows,), 999, dtype=torch.int32)
    tok[4:8] = torch.tensor([1, 2, 3, 4], dtype=torch.int32)
    ci = W.CommitInputs(logits, ms.cuda(), tok.cuda(),
                        torch.tensor([W.AGGRESSIVE, W.CONSERVATIVE, W.AGGRESSIVE, W.AGGRESSIVE],
                                     dtype=torch.uint8).cuda(), B, 999)
    got = run_commit(ci, 0.9, 1)
    assert got["argmax"][0] == 5 and got["argmax"][1] == 0 and got["argmax"][2] == 299
    assert abs(got["conf"][1] - 1.0 / V) < 1e-9
    assert list(got["tokens"][4:8]) == [1, 2, 3, 4] and (got["mask_state"][4:8] == 1).all()
    assert got["block_complete"][1] == 1 and got["n_committed"][1] == 0
    compare_commit(ci, got, 0.9, 1, label="ties/committed")


@pytest.mark.parametrize("k_aggr,tau", [(0, 0.9), (3, 0.9), (64, 0.9), (1, 1.5), (2, -1.0)])
def test_k_aggr_and_threshold_extremes(k_aggr, tau):
    ci = W.commit_inputs(64, 5000, 16, [W.AGGRESSIVE, W.CONSERVATIVE, W.AGGRESSIVE,
                                        W.AGGRESSIVE], 3.0, True, committed_frac=0.3,
                         device="cuda", seed=k_aggr + 7)
    got = run_commit(ci, tau, k_aggr)
    compare_commit(ci, got, tau, k_aggr, label=f"k{k_aggr}-tau{tau}")


@pytest.mark.parametrize("bsz", [1, 3, 64, 200])
def test_block_sizes(bsz):
    n_blocks = 5
    phases = [W.AGGRESSIVE if k % 2 == 0 else W.CONSERVATIVE for k in range(n_blocks)]
    ci = W.commit_inputs(bsz * n_blocks, 3000, bsz, phases, 3.0, True, committed_frac=0.2,
                         device="cuda", seed=bsz)
    got = run_commit(ci, 0.8, 2)
    compare_commit(ci, got, 0.8, 2, label=f"B{bsz}")


def test_large_vocab_and_largest_block():
    # vocab 300000: 37 chunk partials per row (the decide folds them in three
    # batches); block 1024: four rows per decide thread.
    ci = W.commit_inputs(32, 300000, 16, [W.AGGRESSIVE, W.CONSERVATIVE], 3.0, True,
                         committed_frac=0.2, device="cuda", seed=300)
    got = run_commit(ci, 0.8, 2)
    compare_commit(ci, got, 0.8, 2, label="V300000")
    ci = W.commit_inputs(2048, 700, 1024, [W.AGGRESSIVE, W.CONSERVATIVE], 1.5, True,
                         committed_frac=0.3, device="cuda", seed=1024)
    got = run_commit(ci, 0.5, 5)
    compare_commit(ci, got, 0.5, 5, label="B1024")


@pytest.mark.parametrize("vocab", [1, 96])
def test_many_blocks(vocab):
    # 4096 blocks of 16 rows (65536 rows): a reduce grid of 65536 workgroups
    # and a decide grid of 4096, with mixed phases and committed rows.
    nb = 4096
    phases = [W.AGGRESSIVE if k % 3 else W.CONSERVATIVE for k in range(nb)]
    ci = W.commit_inputs(16 * nb, vocab, 16, phases, 2.0, True, committed_frac=0.3,
                         device="cuda", seed=4096 + vocab)
    got = run_commit(ci, 0.5, 2)
    compare_commit(ci, got, 0.5, 2, label=f"blocks{nb}-V{vocab}")


def test_hand_worked_fixture_on_gpu():
    rows, params, phases, blocks = [], {}, [], None
    for line in open(os.path.join(GOLDEN, "commit_worked_example.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        p = line.split()
        if p[0] == "params":
            params = {k: float(v) for k, v in (s.split("=") for s in p[1:])}
        elif p[0] == "phases":
            phases = [W.AGGRESSIVE if s == "A" else W.CONSERVATIVE for s in p[1:]]
        elif p[0] == "blocks":
            blocks = [int(v) for v in p[1:]]
        else:
            rows.append(p)
    logits = torch.tensor([[math.log(float(r[3])), math.log(float(r[4])), math.log(float(r[5]))]
                           for r in rows], dtype=torch.float32, device="cuda")
    ms = torch.tensor([0 if r[1] == "M" else 1 for r in rows], dtype=torch.uint8, device="cuda")
    tok = torch.tensor([int(r[2]) for r in rows], dtype=torch.int32, device="cuda")
    ci = W.CommitInputs(logits, ms, tok, torch.tensor(phases, dtype=torch.uint8, device="cuda"),
                        int(params["block_size"]), int(params["mask_token_id"]))
    got = run_commit(ci, params["tau"], int(params["k_aggr"]))
    for i, r in enumerate(rows):
        want = float(r[6])
        if not math.isnan(want):
            assert abs(got["conf"][i] - want) < 1e-6
        assert got["argmax"][i] == int(r[7])
        assert got["mask_state"][i] == (0 if r[8] == "M" else 1)
        assert got["tokens"][i] == int(r[9])
    assert list(got["n_committed"]) == blocks[0::2]
    assert list(got["block_complete"]) == blocks[1::2]
    say("[commit fixture] ok")


def test_deterministic():
    ci = W.config_commit_inputs(W.config("llada_p512"), device="cuda")
    a = run_commit(ci, 0.9, 1)
    b = run_commit(ci, 0.9, 1)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
