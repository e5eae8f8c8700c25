"""fp64 oracle: per-position confidence and the block commit/remask rule.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What is computed, and where the pages say so:

* [D2F-review] section "쉽게 이해하기" (inference paragraph) and "핵심 메시지":
  a block newly added to the active window behaves conservatively and commits
  only tokens whose confidence exceeds a threshold; once the block before it
  has progressed far enough it turns aggressive and commits the relatively
  most confident tokens even when they are not very confident; tokens that
  were not committed are masked again and predicted again at the next step.
* [dLLM-survey] section "양방향 어텐션과 사라진 KV 캐시" (LLaDA's
  low-confidence remasking: predict every mask, keep the confident ones,
  re-mask the rest) and section "답을 미리 안다: 조기 확정 디코딩(Prophet)"
  (the top-probability ordering, i.e. the maximum softmax probability, is
  LLaDA's default confidence).

Other confidence measures, all from the same vocabulary row:

* [dLLM-survey] section "신뢰도를 넘어서: 궤적 일관성 디코딩(CCD)": standard
  decoding picks positions by the local confidence or by the negative
  entropy of the predicted distribution; section "토큰 순서의 이론" (the
  ordering oracles): top-probability (LLaDA's default, the max probability)
  and the top-probability margin (the gap between the two largest
  probabilities); Dream uses the negative entropy.
* [dLLM-survey] section "답을 미리 안다: 조기 확정 디코딩(Prophet)": the
  confidence gap is the difference of the two largest logits; once it
  passes a threshold, every remaining mask is filled with its argmax at once;
  the threshold is lowered in steps (7.5, 5.0, 2.5) as decoding progresses.

Readings taken where the pages are silent:
  * confidence = max softmax probability at temperature 1; token = argmax;
    ties in the argmax go to the lowest vocabulary index;
  * "exceeds the threshold" is strict: conf > tau, with tau taken as the
    float32 value a caller passes through the C interface;
  * aggressive = the threshold rule plus the k_aggr most confident MASKED
    positions of the block (ties to the lower position);
  * a position already COMMITTED on entry is absorbing and is not read;
  * a MASKED position that is not committed gets mask_token_id (remask);
  * every measure drives the same block rule (conf > tau; aggressive blocks
    also take the k_aggr largest); the second-largest logit counts a repeated
    maximum again (two equal maxima: margin 0, gap 0);
  * Prophet's early commit tests the logit gap whatever measure drives the
    ordinary rule (Prophet sits on top of the model's own decoder); it is
    evaluated per group of consecutive blocks (one request's window): it
    fires when the smallest logit gap over the group's
    positions that were MASKED on entry is strictly above the group's
    threshold, after the ordinary rule has run, and commits the group's
    remaining MASKED positions with their argmax; its threshold steps are
    taken at thirds of the progress.
"""
import numpy as np

from .common import as_f64, as_int

MASKED = 0
COMMITTED = 1
CONSERVATIVE = 0
AGGRESSIVE = 1

MEASURES = ("maxprob", "margin", "neg_entropy", "logit_gap")
# Width of the band around a threshold inside which fp32 and fp64 may decide
# differently, per measure (see the design notes for the error bounds).
NEAR = {"maxprob": 1e-6, "margin": 1e-6, "neg_entropy": 5e-5, "logit_gap": 1e-5}
PROPHET_STEPS = (7.5, 5.0, 2.5)


def tau_as_received(tau: float) -> float:
    """The threshold as the interface carries it: rounded to float32."""
    return float(np.float32(tau))


def row_confidence(rows: np.ndarray):
    """Softmax max-probability and first-index argmax of each row, in fp64.

    conf = 1 / sum_j exp(l_j - max_j l_j); argmax = smallest j with l_j = max.
    """
    rows = as_f64(rows)
    m = rows.max(axis=1)
    is_max = rows == m[:, None]
    first = is_max.argmax(axis=1)  # index of the first True
    conf = 1.0 / np.exp(rows - m[:, None]).sum(axis=1)
    return conf, first.astype(np.int64)


def row_measures(rows: np.ndarray) -> dict:
    """Every confidence measure of each row, in fp64, from the definitions.

    p = softmax(l); maxprob = max p; margin = p(1) - p(2), the two largest
    probabilities; neg_entropy = sum_j p_j log p_j (0 log 0 = 0); logit_gap =
    l(1) - l(2), the two largest logits; argmax = first index of the maximum.
    The second largest entries are taken with the first argmax removed, so a
    repeated maximum counts again."""
    rows = as_f64(rows)
    n, V = rows.shape
    m = rows.max(axis=1)
    first = (rows == m[:, None]).argmax(axis=1)
    e = np.exp(rows - m[:, None])
    S = e.sum(axis=1)
    p = e / S[:, None]
    if V > 1:
        rest = rows.copy()
        rest[np.arange(n), first] = -np.inf
        second = rest.max(axis=1)
    else:
        second = np.full(n, -np.inf)
    plogp = np.where(p > 0, p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    return dict(maxprob=1.0 / S, margin=1.0 / S - np.exp(second - m) / S,
                neg_entropy=plogp.sum(axis=1), logit_gap=m - second,
                argmax=first.astype(np.int64))


def prophet_threshold(progress: float) -> float:
    """Early-commit threshold for a decoding progress in [0, 1]: the three
    steps at thirds of the progress."""
    k = min(2, int(np.floor(3.0 * float(progress))))
    return PROPHET_STEPS[max(0, k)]


def take_rows(logits, rows: np.ndarray) -> np.ndarray:
    """Rows of a torch tensor or array, widened to float64."""
    try:
        import torch
        if isinstance(logits, torch.Tensor):
            idx = torch.as_tensor(rows, dtype=torch.long, device=logits.device)
            return as_f64(logits.index_select(0, idx))
    except ImportError:  # pragma: no cover
        pass
    return as_f64(np.asarray(logits)[rows])


def confidence_commit(logits, mask_state, tokens, block_phase, block_size, tau, k_aggr,
                      mask_token_id, measure="maxprob", early_gap=None, early_group_blocks=0):
    """One commit pass over a window (several requests' blocks concatenated).

    logits [n_rows][V]; mask_state, tokens [n_rows]; block_phase [n_rows/B].
    ``measure`` names the confidence (see row_measures).  ``early_gap``:
    per-group thresholds of Prophet's early commit (tested on the logit gap
    whatever the measure; not with "neg_entropy"), groups of
    ``early_group_blocks`` consecutive blocks (0: one group); None disables
    it.
    Returns a dict with the updated mask_state (uint8) and tokens (int64),
    conf (fp64; NaN for rows COMMITTED on entry), argmax (-1 likewise),
    n_committed and block_complete per block, early (per group: 1 when the
    early commit fired), and the near-tie flags: near_tau[p] when
    |conf_p - tau| is within NEAR[measure], near_topk[k] when an aggressive
    block's k_aggr-th and (k_aggr+1)-th confidences are, near_early[g] when a
    group's smallest gap is that close to its threshold.
    """
    assert measure in MEASURES
    ms = as_int(mask_state, np.uint8).copy()
    tok = as_int(tokens, np.int64).copy()
    phase = as_int(block_phase, np.uint8)
    n_rows = ms.shape[0]
    B = int(block_size)
    assert n_rows % B == 0
    n_blocks = n_rows // B
    t = tau_as_received(tau)
    band = NEAR[measure]

    conf = np.full(n_rows, np.nan)
    amax = np.full(n_rows, -1, dtype=np.int64)
    gap = np.full(n_rows, np.nan)
    live = np.flatnonzero(ms == MASKED)
    if live.size:
        r = row_measures(take_rows(logits, live))
        conf[live] = r[measure]
        amax[live] = r["argmax"]
        gap[live] = r["logit_gap"]
    live_on_entry = ms == MASKED

    n_committed = np.zeros(n_blocks, dtype=np.int64)
    block_complete = np.zeros(n_blocks, dtype=np.uint8)
    near_tau = np.zeros(n_rows, dtype=bool)
    near_topk = np.zeros(n_blocks, dtype=bool)
    for k in range(n_blocks):
        rows = range(k * B, (k + 1) * B)
        cand = [p for p in rows if ms[p] == MASKED]
        chosen = {p for p in cand if conf[p] > t}
        for p in cand:
            near_tau[p] = abs(conf[p] - t) <= band
        if phase[k] == AGGRESSIVE and k_aggr > 0:
            order = sorted(cand, key=lambda p: (-conf[p], p))
            chosen |= set(order[:k_aggr])
            if len(order) > k_aggr and (conf[order[k_aggr - 1]] == conf[order[k_aggr]] or
                                        abs(conf[order[k_aggr - 1]] - conf[order[k_aggr]]) <= band):
                near_topk[k] = True
        for p in cand:
            if p in chosen:
                ms[p] = COMMITTED
                tok[p] = amax[p]
            else:
                tok[p] = mask_token_id
        n_committed[k] = len(chosen)
        block_complete[k] = 1 if all(ms[p] == COMMITTED for p in rows) else 0

    gb = int(early_group_blocks) if early_group_blocks else n_blocks
    n_groups = (n_blocks + gb - 1) // gb if n_blocks else 0
    early = np.zeros(n_groups, dtype=np.uint8)
    near_early = np.zeros(n_groups, dtype=bool)
    if early_gap is not None:
        assert measure != "neg_entropy"
        thr = np.broadcast_to(np.asarray(early_gap, dtype=np.float32).astype(np.float64),
                              (n_groups,))
        for g in range(n_groups):
            rows = np.arange(g * gb * B, min(n_rows, (g + 1) * gb * B))
            entry = rows[live_on_entry[rows]]
            if entry.size == 0:
                continue
            gmin = gap[entry].min()
            near_early[g] = abs(gmin - thr[g]) <= NEAR["logit_gap"]
            if gmin > thr[g]:
                early[g] = 1
                for p in rows:
                    if ms[p] == MASKED:
                        ms[p] = COMMITTED
                        tok[p] = amax[p]
                        n_committed[p // B] += 1
                for k in range(g * gb, min(n_blocks, (g + 1) * gb)):
                    block_complete[k] = 1
    return dict(mask_state=ms, tokens=tok, conf=conf, argmax=amax, n_committed=n_committed,
                block_complete=block_complete, early=early, near_tau=near_tau,
                near_topk=near_topk, near_early=near_early)
