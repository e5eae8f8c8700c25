"""GPU parity of the other confidence measures (top-probability margin,
negative entropy, logit gap) and of Prophet's early commit, through
d2f_confidence_commit_ex, against the fp64 oracle: argmax and every
decision bit-exact outside each measure's near-tie band (reported)."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import compare_commit, run_commit, say

pytestmark = pytest.mark.gpu

# A threshold per measure that splits the synthetic rows (N(0, 3) logits, one
# column raised by U(2, 8) above the rest) into committed and remasked.
TAUS = {"margin": 0.5, "neg_entropy": -2.0, "logit_gap": 5.0}


@pytest.mark.parametrize("measure", ["margin", "neg_entropy", "logit_gap"])
@pytest.mark.parametrize("cfg,bsz", [("tiny_f32", None), ("llada_p512", None), ("dream_gqa", 16), ("dream_gqa", 64),
                                     ("llada_p32k", None)])
def test_measures_on_the_workloads(measure, cfg, bsz):
    c = W.config(cfg, block_size=bsz)
    ci = W.config_commit_inputs(c, device="cuda", seed=7)
    tau = TAUS[measure]
    got = run_commit(ci, tau, c["k_aggr"], measure=measure)
    st = compare_commit(ci, got, tau, c["k_aggr"], label=f"{measure}-{cfg}-B{bsz}",
                        measure=measure)
    assert st["live"] > 0


@pytest.mark.parametrize("measure", ["margin", "neg_entropy", "logit_gap"])
@pytest.mark.parametrize("vocab,ld_pad", [(1, 0), (2, 0), (7, 1), (8193, 0), (126464, 4)])
def test_measures_vocab_sizes_and_ties(measure, vocab, ld_pad):
    """Scalar and vector loads, one-entry rows (gap +inf), and rows whose
    maximum is repeated (margin and gap exactly 0)."""
    rows, B = 32, 8
    g = torch.Generator(device="cuda").manual_seed(vocab + 11)
    full = torch.randn((rows, vocab + ld_pad), generator=g, device="cuda") * 3
    if vocab >= 2:
        full[::4, vocab - 1] = full[::4, :vocab].max(dim=1).values  # repeated maximum
        full[1::4, 0] = full[1::4, :vocab].max(dim=1).values
    logits = full[:, :vocab]
    phases = [W.AGGRESSIVE, W.CONSERVATIVE, W.AGGRESSIVE, W.CONSERVATIVE]
    ci = W.commit_inputs(rows, vocab, B, phases, 1.0, False, committed_frac=0.25,
                         device="cuda", seed=vocab)
    ci.logits = logits
    tau = {"margin": 0.05, "neg_entropy": -3.0, "logit_gap": 1.0}[measure]
    got = run_commit(ci, tau, 2, measure=measure)
    compare_commit(ci, got, tau, 2, label=f"{measure}-V{vocab}", measure=measure)


def _slot_batch(n_req, win_blocks, B, vocab, seed):
    """Slot layout of several requests' windows: win_blocks blocks each,
    newest block conservative."""
    phases = []
    for _ in range(n_req):
        phases += [W.AGGRESSIVE] * (win_blocks - 1) + [W.CONSERVATIVE]
    return W.commit_inputs(n_req * win_blocks * B, vocab, B, phases, 3.0, True,
                           committed_frac=0.2, device="cuda", seed=seed)


@pytest.mark.parametrize("measure", ["maxprob", "margin", "logit_gap"])
def test_prophet_early_commit(measure):
    """Per-request groups (4 blocks of 16 rows each, 12 requests) with a mix
    of thresholds so that some groups fire and some do not."""
    ci = _slot_batch(12, 4, 16, 20000, seed=21)
    # the smallest raised margin of a group is near 2; thresholds straddle it
    thr = [0.5, 7.5, 1.0, 5.0, 2.5, 0.0, 1.5, 7.5, 0.25, 3.0, 2.0, 1.75]
    tau = {"maxprob": 0.9, "margin": 0.8, "logit_gap": 5.0}[measure]
    got = run_commit(ci, tau, 1, measure=measure, early_gap=thr, early_group_blocks=4)
    st = compare_commit(ci, got, tau, 1, label=f"prophet-{measure}", measure=measure,
                        early_gap=thr, early_group_blocks=4)
    assert 0 < st["early"] < 12, st


def test_prophet_one_group_and_ragged_last_group():
    ci = _slot_batch(5, 3, 8, 3000, seed=22)   # 15 blocks, groups of 4: last group has 3
    for thr, gb in (([1.0], 0), ([0.5, 9.0, 1.0, 0.1], 4)):
        got = run_commit(ci, 0.95, 1, measure="logit_gap", early_gap=thr, early_group_blocks=gb)
        compare_commit(ci, got, 0.95, 1, label=f"prophet-groups{gb}", measure="logit_gap",
                       early_gap=thr, early_group_blocks=gb)


def test_maxprob_through_the_extended_entry_matches_the_plain_one():
    """measure "maxprob" with an early threshold that never fires takes the
    second-largest accumulator path; its decisions equal the plain call's."""
    c = W.config("llada_p512")
    ci = W.config_commit_inputs(c, device="cuda", seed=3)
    a = run_commit(ci, 0.9, 1)
    b = run_commit(ci, 0.9, 1, measure="maxprob", early_gap=[1e30])
    for k in ("mask_state", "tokens", "n_committed", "block_complete", "argmax"):
        assert np.array_equal(a[k], b[k]), k
    say("[prophet] maxprob paths agree")
