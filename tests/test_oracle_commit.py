"""Pins for the fp64 commit oracle (CPU only).

Closed forms of the softmax maximum, a hand-worked fixture, torch's softmax
on tie-free rows, and an exhaustive check of the block rule against a
rank-counting restatement on tiny blocks.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import commit as OC

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
M, C = OC.MASKED, OC.COMMITTED
A, K = OC.AGGRESSIVE, OC.CONSERVATIVE


def test_all_equal_row():
    for v in (1, 2, 7, 512, 126464):
        conf, a = OC.row_confidence(np.full((1, v), 3.25, dtype=np.float32))
        assert a[0] == 0
        assert abs(conf[0] - 1.0 / v) <= 1e-15 / v * 10


@pytest.mark.parametrize("V,L,j", [(2, 0.5, 1), (512, 4.0, 300), (126464, 9.0, 126463),
                                   (152064, -3.0, 0)])
def test_one_raised_entry_closed_form(V, L, j):
    row = np.zeros((1, V))
    row[0, j] = L
    conf, a = OC.row_confidence(row)
    if L > 0:
        assert a[0] == j
        expect = math.exp(L) / (math.exp(L) + V - 1)
    else:
        assert a[0] == (1 if j == 0 else 0)
        expect = 1.0 / (math.exp(L) + V - 1)
    assert abs(conf[0] - expect) <= 1e-14 * max(expect, 1e-300) + 1e-15


def test_argmax_ties_go_to_lowest_index():
    row = np.array([[1.0, 5.0, -2.0, 5.0, 5.0]])
    conf, a = OC.row_confidence(row)
    assert a[0] == 1
    expect = 1.0 / (3 + math.exp(-4.0) + math.exp(-7.0))
    assert abs(conf[0] - expect) < 1e-15


def test_against_torch_softmax_on_tie_free_rows():
    g = torch.Generator().manual_seed(1)
    x = (torch.randn(64, 4097, generator=g) * 3).to(torch.float32)
    conf, a = OC.row_confidence(x)
    p = torch.softmax(x.double(), dim=1)
    mx, idx = p.max(dim=1)
    np.testing.assert_allclose(conf, mx.numpy(), rtol=1e-13, atol=0)
    np.testing.assert_array_equal(a, idx.numpy())


def _row_with_conf(V, target):
    """Row of zeros with entry 0 raised so that its softmax max equals target:
    e^L / (e^L + V - 1) = target  <=>  L = ln(target (V - 1) / (1 - target))."""
    row = np.zeros(V)
    row[0] = math.log(target * (V - 1) / (1 - target))
    return row


def test_threshold_is_strict_and_taken_as_float32():
    V, B = 1000, 4
    tau = 0.9
    t32 = OC.tau_as_received(tau)
    assert t32 != tau and abs(t32 - tau) < 3e-8
    confs = [t32 + 1e-5, t32 - 1e-5, 0.99, 0.5]
    logits = np.stack([_row_with_conf(V, c) for c in confs])
    r = OC.confidence_commit(logits, np.zeros(B, np.uint8), np.full(B, 7), np.array([K]), B,
                             tau, 1, -1)
    np.testing.assert_allclose(r["conf"], confs, rtol=1e-12)
    assert list(r["mask_state"]) == [C, M, C, M]
    assert list(r["tokens"]) == [0, -1, 0, -1]
    assert not r["near_tau"].any()
    # A confidence between float32(0.9) and 0.9 clears the threshold as received.
    mid = (t32 + tau) / 2
    r = OC.confidence_commit(_row_with_conf(V, mid)[None, :], np.zeros(1, np.uint8), [0],
                             np.array([K]), 1, tau, 1, -1)
    assert r["mask_state"][0] == C and r["near_tau"][0]


def _fixture():
    rows, blocks, params, phases = [], None, {}, []
    with open(os.path.join(GOLDEN, "commit_worked_example.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "params":
                params = {k: float(v) for k, v in (p.split("=") for p in parts[1:])}
            elif parts[0] == "phases":
                phases = [A if p == "A" else K for p in parts[1:]]
            elif parts[0] == "blocks":
                blocks = [int(v) for v in parts[1:]]
            else:
                rows.append(parts)
    return params, phases, rows, blocks


def test_hand_worked_fixture():
    params, phases, rows, blocks = _fixture()
    V, B = int(params["vocab"]), int(params["block_size"])
    logits = np.array([[math.log(float(r[3])), math.log(float(r[4])), math.log(float(r[5]))]
                       for r in rows], dtype=np.float32)
    ms = np.array([M if r[1] == "M" else C for r in rows], np.uint8)
    tok = np.array([int(r[2]) for r in rows])
    out = OC.confidence_commit(logits, ms, tok, np.array(phases, np.uint8), B, params["tau"],
                               int(params["k_aggr"]), int(params["mask_token_id"]))
    assert logits.shape[1] == V
    for i, r in enumerate(rows):
        want_conf = float(r[6])
        if math.isnan(want_conf):
            assert math.isnan(out["conf"][i])
        else:
            assert abs(out["conf"][i] - want_conf) < 1e-6
        assert out["argmax"][i] == int(r[7])
        assert out["mask_state"][i] == (M if r[8] == "M" else C)
        assert out["tokens"][i] == int(r[9])
    assert list(out["n_committed"]) == blocks[0::2]
    assert list(out["block_complete"]) == blocks[1::2]


def _rank_rule(confs, states, phase, tau, k_aggr):
    """Restatement of the block rule by counting: masked position p is
    committed iff conf_p > tau, or the block is aggressive and fewer than
    k_aggr masked positions q rank above p (higher conf, or equal conf and
    q < p)."""
    out = []
    for p, (c, s) in enumerate(zip(confs, states)):
        if s != M:
            out.append(None)
            continue
        above = sum(1 for q, (cq, sq) in enumerate(zip(confs, states))
                    if sq == M and (cq > c or (cq == c and q < p)))
        out.append(c > tau or (phase == A and above < k_aggr))
    return out


def test_exhaustive_small_blocks():
    V = 2
    level = [0.55, 0.7, 0.7, 0.95, 0.6, 0.99]  # includes an exact tie and values above tau
    tau = 0.9
    t32 = OC.tau_as_received(tau)
    n_cases = 0
    for B in (1, 2, 3, 4):
        confs = level[:B]
        # Row [L, 0] has softmax maximum e^L / (e^L + 1); pick L for each conf.
        logits = np.array([[math.log(c / (1 - c)), 0.0] for c in confs], dtype=np.float64)
        got_conf, _ = OC.row_confidence(logits)
        for states in itertools.product((M, C), repeat=B):
            for phase in (A, K):
                for k_aggr in range(B + 1):
                    r = OC.confidence_commit(logits, np.array(states, np.uint8), np.zeros(B),
                                             np.array([phase], np.uint8), B, tau, k_aggr, 9)
                    want = _rank_rule(list(got_conf), states, phase, t32, k_aggr)
                    for p in range(B):
                        if want[p] is None:
                            assert r["mask_state"][p] == C and r["tokens"][p] == 0
                        else:
                            assert r["mask_state"][p] == (C if want[p] else M)
                            assert r["tokens"][p] == (0 if want[p] else 9)
                    assert r["n_committed"][0] == sum(1 for w in want if w)
                    assert r["block_complete"][0] == int(all(w is None or w for w in want))
                    n_cases += 1
    assert n_cases == sum(2 ** b * 2 * (b + 1) for b in (1, 2, 3, 4))
    assert V == 2


def test_committed_rows_are_not_read():
    # A committed row full of NaN must not disturb anything.
    logits = np.array([[np.nan] * 4, [0.0, 3.0, 0.0, 0.0]])
    r = OC.confidence_commit(logits, np.array([C, M], np.uint8), np.array([5, 9]),
                             np.array([A], np.uint8), 2, 0.9, 1, 9)
    assert list(r["mask_state"]) == [C, C] and list(r["tokens"]) == [5, 1]
    assert math.isnan(r["conf"][0]) and r["argmax"][0] == -1
    assert r["block_complete"][0] == 1 and r["n_committed"][0] == 1


def test_near_topk_flag():
    V = 50
    c1 = 0.5
    logits = np.stack([_row_with_conf(V, c1), _row_with_conf(V, c1 + 2e-7), _row_with_conf(V, 0.2)])
    logits = np.concatenate([logits, _row_with_conf(V, 0.1)[None]])
    r = OC.confidence_commit(logits, np.zeros(4, np.uint8), np.zeros(4), np.array([A], np.uint8),
                             4, 0.9, 1, -1)
    assert r["near_topk"][0]
    assert list(r["mask_state"]) == [M, C, M, M]


def test_confidence_exactly_at_threshold_is_not_committed():
    # All-equal rows have softmax maximum exactly 1/V (a power of two here),
    # which float32 also holds exactly: "exceeds" must leave them masked.
    for V, tau in ((2, 0.5), (4, 0.25), (8, 0.125)):
        r = OC.confidence_commit(np.zeros((1, V)), np.zeros(1, np.uint8), [3], np.array([K]), 1,
                                 tau, 1, 3)
        assert r["conf"][0] == tau
        assert r["mask_state"][0] == M and r["tokens"][0] == 3 and r["near_tau"][0]
