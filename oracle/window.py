"""Reference active-window scheduler of D2F's pipelined decoding.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages state ([D2F-review] "핵심 메시지", last point, and "쉽게
이해하기", inference paragraph; [D2F-wiki] "인터블록 병렬 디코딩" and
"운영 관점", KV cache management):
  * decoding keeps a window of active blocks; when the progress of the last
    block in the window passes a threshold, a new (fully masked) block is
    added behind it, so that the window size stays bounded;
  * a newly added block starts conservative; once the block before it has
    progressed far enough it switches to the aggressive commit rule;
  * blocks are processed in order between blocks: a completed block's K/V
    become permanent cache entries (the completion event is the signal to
    persist them), and the window then no longer holds it.

Readings taken where the pages are silent (each is listed in the design notes):
  * progress of a block = committed positions / block size;
  * "passes a threshold" is strict (progress > tau_add, progress > tau_act),
    compared as committed > tau * B in float64 of the float32 thresholds;
  * at most one block is appended per step, only while the window holds
    fewer than max_win_blocks blocks and fewer than total_blocks blocks have
    been started;
  * the oldest block of the window is aggressive (its predecessor is complete
    and cached); the block after it turns aggressive once its predecessor's
    progress passes tau_act, and stays aggressive;
  * after a commit pass, the complete blocks at the front of the window are
    persisted oldest first (a complete block behind an incomplete one waits);
    the append decision is taken after persisting, on the window that remains;
  * phases for the next step are decided last, on the updated window;
  * the first block is started when decoding starts.
"""
import numpy as np

CONSERVATIVE = 0
AGGRESSIVE = 1


def _passes(committed, tau, block_size):
    return committed > float(np.float32(tau)) * block_size


class Window:
    """State: absolute index of the oldest window block, per-window-block
    committed counts and phases, blocks started and blocks persisted."""

    def __init__(self, block_size, max_win_blocks, total_blocks, tau_add, tau_act):
        assert block_size >= 1 and max_win_blocks >= 1 and total_blocks >= 1
        self.B = block_size
        self.max_win = max_win_blocks
        self.total = total_blocks
        self.tau_add = tau_add
        self.tau_act = tau_act
        self.first = 0            # absolute index of the oldest window block
        self.committed = [0]      # per window block
        self.phase = [AGGRESSIVE]  # the first block is the oldest
        self.started = 1
        self.persisted = 0

    @property
    def n_win(self):
        return len(self.committed)

    @property
    def done(self):
        return self.persisted == self.total

    def after_commit(self, n_committed):
        """Apply one commit pass (positions committed in it, per window
        block); returns (blocks persisted now, blocks appended now)."""
        assert len(n_committed) == self.n_win
        for k, c in enumerate(n_committed):
            self.committed[k] += int(c)
            assert 0 <= self.committed[k] <= self.B
        persisted = 0
        while self.committed and self.committed[0] == self.B:
            self.committed.pop(0)
            self.phase.pop(0)
            self.first += 1
            self.persisted += 1
            persisted += 1
        appended = 0
        if self.started < self.total and self.n_win < self.max_win:
            if self.n_win == 0 or _passes(self.committed[-1], self.tau_add, self.B):
                self.committed.append(0)
                self.phase.append(CONSERVATIVE)
                self.started += 1
                appended = 1
        for k in range(self.n_win):
            if k == 0 or _passes(self.committed[k - 1], self.tau_act, self.B):
                self.phase[k] = AGGRESSIVE
        return persisted, appended

