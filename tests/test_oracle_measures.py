"""Pins of the oracle's other confidence measures (maximum probability is
pinned in test_oracle_commit.py): negative entropy, top-probability margin,
logit gap, and Prophet's early commit.  Each is checked against something
other than the oracle's own formula: closed forms, scipy and sorting on
random rows, and a hand-worked fixture."""
import math
import os

import numpy as np
import pytest
import scipy.stats
import torch

from oracle import commit as OC

M, C = OC.MASKED, OC.COMMITTED
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("V,a", [(2, 0.5), (7, 3.0), (1000, 9.25), (126464, 12.0)])
def test_one_raised_entry_closed_form(V, a):
    """V - 1 zeros and one entry a: every measure in closed form."""
    row = np.zeros((1, V))
    row[0, V // 2] = a
    r = OC.row_measures(row)
    Z = math.exp(a) + (V - 1)
    p1, p2 = math.exp(a) / Z, 1.0 / Z
    assert r["argmax"][0] == V // 2
    assert math.isclose(r["maxprob"][0], p1, rel_tol=1e-12)
    assert math.isclose(r["margin"][0], p1 - p2, rel_tol=1e-12)
    assert math.isclose(r["neg_entropy"][0], p1 * math.log(p1) + (V - 1) * p2 * math.log(p2),
                        rel_tol=1e-12)
    assert r["logit_gap"][0] == a


@pytest.mark.parametrize("V", [1, 2, 5, 4096])
def test_uniform_row(V):
    r = OC.row_measures(np.full((1, V), 0.3))
    assert math.isclose(r["neg_entropy"][0], -math.log(V), rel_tol=1e-12, abs_tol=1e-15)
    assert r["maxprob"][0] == pytest.approx(1.0 / V, rel=1e-12)
    if V > 1:
        assert r["margin"][0] == 0.0 and r["logit_gap"][0] == 0.0
    assert r["argmax"][0] == 0


def test_repeated_maximum_counts_twice():
    row = np.array([[1.0, 4.0, 2.0, 4.0, 0.0]])
    r = OC.row_measures(row)
    assert r["argmax"][0] == 1 and r["margin"][0] == 0.0 and r["logit_gap"][0] == 0.0


def test_against_scipy_and_sorting_on_random_rows():
    g = np.random.default_rng(3)
    rows = g.normal(0.0, 3.0, size=(40, 3001))
    rows[::3, 17] += 11.0
    r = OC.row_measures(rows)
    for i, x in enumerate(rows):
        p = np.exp(x - x.max())
        p /= p.sum()
        assert math.isclose(r["neg_entropy"][i], -scipy.stats.entropy(p), rel_tol=1e-10)
        ps = np.sort(p)
        assert math.isclose(r["margin"][i], ps[-1] - ps[-2], rel_tol=1e-9, abs_tol=1e-15)
        xs = np.sort(x)
        assert r["logit_gap"][i] == xs[-1] - xs[-2]
    t2 = torch.topk(torch.from_numpy(rows), 2, dim=1).values
    assert np.array_equal(r["logit_gap"], (t2[:, 0] - t2[:, 1]).numpy())
    sm = torch.softmax(torch.from_numpy(rows), dim=1)
    assert np.allclose(r["maxprob"], sm.max(dim=1).values.numpy(), rtol=1e-12)


def test_measures_order_a_one_parameter_family_alike():
    """Raising one entry makes every measure larger (a sanity invariant)."""
    base = np.random.default_rng(5).normal(0, 1, 50)
    rows = np.stack([np.concatenate([[base.max() + d], base]) for d in (0.1, 1.0, 3.0, 8.0)])
    r = OC.row_measures(rows)
    for k in OC.MEASURES:
        assert np.all(np.diff(r[k]) > 0), k


@pytest.mark.parametrize("measure", OC.MEASURES)
def test_block_rule_uses_the_measure(measure):
    """The commit rule ranks and thresholds by the chosen measure: rows built
    so that the measures disagree on the order."""
    # row a: one clear maximum among many small values; row b: two large
    # values close together (high max-probability share, small margin).
    a = np.full(20, 0.0); a[3] = 4.0
    b = np.full(20, -30.0); b[5] = 6.0; b[6] = 5.9
    logits = np.stack([a, b]).astype(np.float32)
    r = OC.row_measures(logits)
    order = np.argsort(-r[measure], kind="stable")
    out = OC.confidence_commit(logits, np.zeros(2, np.uint8), np.zeros(2, np.int64),
                               np.array([OC.AGGRESSIVE], np.uint8), 2, 1e9, 1, 99,
                               measure=measure)
    committed = np.flatnonzero(out["mask_state"] == C)
    assert list(committed) == [order[0]]


def _read_cases():
    cases, cur = {}, None
    with open(os.path.join(HERE, "golden", "prophet_early_commit.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "case":
                cur = cases.setdefault(parts[1], {"rows": []})
            elif parts[0] == "blocks":
                cur["blocks"] = [int(v) for v in parts[1:]]
            elif parts[0] == "early":
                cur["early"] = [int(v) for v in parts[1:]]
            else:
                cur["rows"].append(parts)
    return cases


@pytest.mark.parametrize("name", ["A", "B"])
def test_prophet_hand_worked_fixture(name):
    case = _read_cases()[name]
    rows = case["rows"]
    logits = np.array([[float(v) for v in r[3:7]] for r in rows], np.float32)
    ms = np.array([M if r[1] == "M" else C for r in rows], np.uint8)
    tok = np.array([int(r[2]) for r in rows])
    out = OC.confidence_commit(logits, ms, tok, np.zeros(2, np.uint8), 2, 3.0, 0, 99,
                               measure="logit_gap", early_gap=[2.5, 2.5], early_group_blocks=1)
    for i, r in enumerate(rows):
        want = float(r[7])
        assert (math.isnan(out["conf"][i]) if math.isnan(want) else out["conf"][i] == want)
        assert out["mask_state"][i] == (M if r[8] == "M" else C)
        assert out["tokens"][i] == int(r[9])
    assert list(out["n_committed"]) == case["blocks"][0::2]
    assert list(out["block_complete"]) == case["blocks"][1::2]
    assert list(out["early"]) == case["early"]


def test_prophet_threshold_steps():
    assert [OC.prophet_threshold(p) for p in (0.0, 0.2, 0.34, 0.5, 0.67, 0.9, 1.0)] == \
        [7.5, 7.5, 5.0, 5.0, 2.5, 2.5, 2.5]


def test_prophet_on_top_of_max_probability():
    """The early test reads the logit gap while max probability drives the
    ordinary rule (tau 2 lets nothing through on its own)."""
    rows = _read_cases()["A"]["rows"]
    logits = np.array([[float(v) for v in r[3:7]] for r in rows], np.float32)
    out = OC.confidence_commit(logits, np.zeros(4, np.uint8), np.full(4, 99), np.zeros(2, np.uint8),
                               2, 2.0, 0, 99, measure="maxprob", early_gap=[2.5, 2.5],
                               early_group_blocks=1)
    assert list(out["mask_state"]) == [C, C, M, M]
    assert list(out["tokens"]) == [0, 1, 99, 99]
    assert list(out["n_committed"]) == [2, 0] and list(out["block_complete"]) == [1, 0]
    assert list(out["early"]) == [1, 0]
    with pytest.raises(AssertionError):
        OC.confidence_commit(logits, np.zeros(4, np.uint8), np.full(4, 99), np.zeros(2, np.uint8),
                             2, 2.0, 0, 99, measure="neg_entropy", early_gap=2.5)
