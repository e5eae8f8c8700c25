"""The library's active-window scheduler (host code behind the C ABI, no GPU
needed) against the oracle's, transition by transition, and its errors."""
import random

import pytest

import block_causal_attention_d2f_amd as d2f
from block_causal_attention_d2f_amd import _binding as B
from oracle import window as OW


@pytest.fixture(scope="module")
def lib():
    import os
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libd2f.so not built")
    return d2f.load()


def _same(w, o):
    assert (w.first, w.n_win, w.started, w.persisted) == (o.first, o.n_win, o.started, o.persisted)
    assert w.committed == o.committed and w.phase == o.phase


@pytest.mark.parametrize("seed", range(40))
def test_matches_oracle_on_random_schedules(lib, seed):
    rng = random.Random(1000 + seed)
    Bs = rng.choice([1, 3, 16, 64])
    max_win = rng.choice([1, 2, 3, 8])
    total = rng.randint(1, 12)
    tau_add = rng.choice([0.0, 0.1, 0.25, 0.5, 0.7, 0.95, 1.0])
    tau_act = rng.choice([0.0, 0.5, 0.7, 0.9, 0.95, 1.0])
    w = d2f.Window(Bs, max_win, total, tau_add, tau_act)
    o = OW.Window(Bs, max_win, total, tau_add, tau_act)
    _same(w, o)
    steps = 0
    while not o.done:
        steps += 1
        assert steps < 5000
        nc = [rng.randint(0, Bs - c) if rng.random() < 0.6 else 0 for c in o.committed]
        if sum(nc) == 0:
            nc[next(i for i, c in enumerate(o.committed) if c < Bs)] = 1
        assert w.after_commit(nc) == o.after_commit(nc)
        _same(w, o)
    assert w.done


def test_hand_worked_trace_through_the_library(lib):
    # The same trace as tests/golden/window_schedule_trace.txt.
    w = d2f.Window(4, 3, 4, 0.25, 0.7)
    A, C = B.AGGRESSIVE, B.CONSERVATIVE
    for nc, exp in [([2], (0, 1, 0, [A, C], [2, 0])),
                    ([0, 2], (0, 1, 0, [A, C, C], [2, 2, 0])),
                    ([0, 1, 3], (0, 0, 0, [A, C, A], [2, 3, 3])),
                    ([2, 0, 0], (1, 1, 1, [A, A, A], [3, 3, 0])),
                    ([0, 1, 4], (0, 0, 1, [A, A, A], [3, 4, 4])),
                    ([1, 0, 0], (3, 0, 4, [], []))]:
        p, a = w.after_commit(nc)
        assert (p, a, w.first, w.phase, w.committed) == exp
    assert w.done


def test_errors_leave_state_unchanged(lib):
    with pytest.raises(d2f.D2FError):
        d2f.Window(0, 2, 3, 0.5, 0.5)
    with pytest.raises(d2f.D2FError):
        d2f.Window(4, 65, 3, 0.5, 0.5)
    with pytest.raises(d2f.D2FError):
        d2f.Window(4, 2, 3, float("nan"), 0.5)
    w = d2f.Window(4, 2, 2, 0.5, 0.5)
    before = (w.first, w.n_win, w.committed, w.phase)
    with pytest.raises(d2f.D2FError):
        w.after_commit([5])          # more than the block holds
    with pytest.raises(d2f.D2FError):
        w.after_commit([-1])
    assert (w.first, w.n_win, w.committed, w.phase) == before
    w.after_commit([4])              # block 0 done -> persisted, block 1 started
    w.after_commit([4])              # block 1 done -> everything persisted
    assert w.done
    with pytest.raises(d2f.D2FError):
        w.after_commit([0])
