"""The oracle's active-window scheduler against a hand-worked trace and
invariants of the rules it follows (see oracle/window.py for the passages)."""
import os
import random

import pytest

from oracle import window as OW

HERE = os.path.dirname(os.path.abspath(__file__))


def _kv(tokens):
    return dict(t.split("=", 1) for t in tokens)


def _ints(s):
    return [int(x) for x in s.split(",")] if s else []


def _phases(s):
    return [OW.AGGRESSIVE if x == "A" else OW.CONSERVATIVE for x in s.split(",")] if s else []


def test_hand_worked_trace():
    lines = [l.split("#")[0].strip() for l in open(os.path.join(HERE, "golden", "window_schedule_trace.txt"))]
    lines = [l for l in lines if l]
    p = _kv(lines[0].split()[1:])
    w = OW.Window(int(p["block_size"]), int(p["max_win_blocks"]), int(p["total_blocks"]),
                  float(p["tau_add"]), float(p["tau_act"]))
    init = _kv(lines[1].split()[1:])
    assert w.first == int(init["first"]) and w.phase == _phases(init["phases"])
    assert w.committed == _ints(init["committed"])
    for line in lines[2:]:
        head, tail = line.split("->")
        commit = _ints(_kv(head.split()[2:])["commit"])
        exp = _kv(tail.split())
        persisted, appended = w.after_commit(commit)
        assert persisted == int(exp["persisted"]), line
        assert appended == int(exp["appended"]), line
        assert w.first == int(exp["first"]), line
        assert w.phase == _phases(exp["phases"]), line
        assert w.committed == _ints(exp["committed"]), line
    assert w.done


@pytest.mark.parametrize("seed", range(20))
def test_invariants_under_random_progress(seed):
    rng = random.Random(seed)
    B = rng.choice([1, 4, 16])
    max_win = rng.choice([1, 2, 4])
    total = rng.randint(1, 9)
    tau_add, tau_act = rng.choice([0.0, 0.1, 0.5, 0.9]), rng.choice([0.0, 0.5, 0.95])
    w = OW.Window(B, max_win, total, tau_add, tau_act)
    prev_phase = {}  # absolute block -> phase seen last step
    persisted_order = []
    steps = 0
    while not w.done:
        steps += 1
        assert steps < 10000
        assert 1 <= w.n_win <= max_win
        # committed per block: a random part of what is still masked (at least
        # one position somewhere, so the schedule advances)
        nc = [rng.randint(0, B - c) if rng.random() < 0.7 else 0 for c in w.committed]
        if sum(nc) == 0:
            k = next(i for i, c in enumerate(w.committed) if c < B)
            nc[k] = 1
        first_before, last_before = w.first, w.committed[-1] + nc[-1]
        n_before, started_before = w.n_win, w.started
        p, a = w.after_commit(nc)
        persisted_order.extend(range(first_before, first_before + p))
        # persist happens oldest first and only for complete blocks
        assert w.first == first_before + p
        # an append needs room, blocks left, and the last block past tau_add
        if a:
            assert n_before - p < max_win and started_before < total
            if n_before - p > 0:
                assert last_before > tau_add * B - 1e-9 or p == n_before
        # the oldest block is aggressive; aggressive is absorbing
        if w.n_win:
            assert w.phase[0] == OW.AGGRESSIVE
        for k in range(w.n_win):
            b = w.first + k
            if prev_phase.get(b) == OW.AGGRESSIVE:
                assert w.phase[k] == OW.AGGRESSIVE
            prev_phase[b] = w.phase[k]
    assert persisted_order == list(range(total))
    assert w.started == total


def test_single_block_window_is_sequential_decoding():
    # max_win_blocks 1: blocks are decoded strictly one after another and each
    # is aggressive (the classic block-by-block semi-autoregressive schedule).
    w = OW.Window(4, 1, 3, 0.0, 0.0)
    seen = []
    while not w.done:
        assert w.n_win == 1 and w.phase == [OW.AGGRESSIVE]
        seen.append(w.first)
        w.after_commit([4 - w.committed[0]])
    assert seen == [0, 1, 2]
