"""Seeded random commit passes, for breadth beyond the workloads and the
hand-picked cases: d2f_confidence_commit (through the C ABI) against the
oracle over vocabulary size (including 1 and the 8192-logit chunk edges),
padded row strides, block size 1..1024, masked fraction, per-block phases,
k_aggr, the threshold, the four confidence measures and Prophet's early
commit with random groups and thresholds.  Decisions are compared bit for bit
outside each measure's band around the threshold."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import compare_commit, run_commit, say

pytestmark = pytest.mark.gpu

MAX_LOGITS = 20_000_000  # keeps the fp64 oracle at a few seconds per case
N_DRAWS = 16
TAUS = {"maxprob": [-1.0, 0.0, 0.3, 0.5, 0.9, 0.99, 1.0],
        "margin": [0.0, 0.2, 0.5, 0.8, 1.0],
        "neg_entropy": [-6.0, -2.0, -0.5, -0.05, 0.0],
        "logit_gap": [0.0, 0.5, 2.5, 5.0, 7.5]}


def draw(seed):
    rng = np.random.default_rng(seed)
    vocab = int(rng.choice([1, 2, 5, 4096, 8191, 8192, 8193, 30000, 126464]))
    sizes = [b for b in (1, 2, 3, 8, 16, 32, 64, 200, 1024) if b * vocab <= MAX_LOGITS]
    bsz = int(rng.choice(sizes))
    n_blocks = int(rng.integers(1, max(1, min(12, MAX_LOGITS // (bsz * vocab))) + 1))
    measure = str(rng.choice(list(TAUS)))
    early = measure != "neg_entropy" and rng.random() < 0.4
    group_blocks = int(rng.integers(1, n_blocks + 1)) if early else 0
    n_groups = -(-n_blocks // group_blocks) if early else 0
    return dict(
        vocab=vocab, bsz=bsz, n_blocks=n_blocks, measure=measure,
        ld_pad=int(rng.choice([0, 0, 1, 3, 4])),
        std=float(rng.choice([0.5, 2.0, 3.0, 8.0])), boost=bool(rng.random() < 0.5),
        committed_frac=float(rng.choice([0.0, 0.1, 0.5, 0.9])),
        phases=[int(p) for p in rng.integers(0, 2, n_blocks)],
        k_aggr=int(rng.choice([0, 1, 2, 3, bsz])),
        tau=float(rng.choice(TAUS[measure])),
        early_gap=[float(rng.choice([0.0, 0.5, 1.0, 2.5, 5.0, 7.5, 1e30])) for _ in range(n_groups)]
        if early else None,
        group_blocks=group_blocks)


@pytest.mark.parametrize("k", range(N_DRAWS))
def test_random_commit_against_oracle(k):
    seed = 5000 + 37 * k
    c = draw(seed)
    say(f"--- random commit case seed={seed}: {c}")
    rows = c["bsz"] * c["n_blocks"]
    ci = W.commit_inputs(rows, c["vocab"], c["bsz"], c["phases"], c["std"], c["boost"],
                         committed_frac=c["committed_frac"], device="cuda", seed=seed)
    if c["ld_pad"]:
        # the same logits in rows of a wider buffer whose padding is NaN
        full = torch.full((rows, c["vocab"] + c["ld_pad"]), float("nan"), device="cuda")
        full[:, :c["vocab"]] = ci.logits
        ci.logits = full[:, :c["vocab"]]
    kw = dict(measure=c["measure"], early_gap=c["early_gap"], early_group_blocks=c["group_blocks"])
    got = run_commit(ci, c["tau"], c["k_aggr"], **kw)
    compare_commit(ci, got, c["tau"], c["k_aggr"], label=f"random-{seed}", **kw)
