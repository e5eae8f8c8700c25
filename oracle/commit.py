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

Readings taken where the pages are silent:
  * confidence = max softmax probability at temperature 1; token = argmax;
    ties in the argmax go to the lowest vocabulary index;
  * "exceeds the threshold" is strict: conf > tau, with tau taken as the
    float32 value a caller passes through the C interface;
  * aggressive = the threshold rule plus the k_aggr most confident MASKED
    positions of the block (ties to the lower position);
  * a position already COMMITTED on entry is absorbing and is not read;
  * a MASKED position that is not committed gets mask_token_id (remask).
"""
import numpy as np

from .common import as_f64, as_int

MASKED = 0
COMMITTED = 1
CONSERVATIVE = 0
AGGRESSIVE = 1

NEAR_TIE = 1e-6


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
                      mask_token_id):
    """One commit pass over a window (several requests' blocks concatenated).

    logits [n_rows][V]; mask_state, tokens [n_rows]; block_phase [n_rows/B].
    Returns a dict with the updated mask_state (uint8) and tokens (int64),
    conf (fp64; NaN for rows COMMITTED on entry), argmax (-1 likewise),
    n_committed and block_complete per block, and the near-tie flags:
    near_tau[p] when |conf_p - tau| <= 1e-6, near_topk[k] when an aggressive
    block's k_aggr-th and (k_aggr+1)-th confidences are within 1e-6.
    """
    ms = as_int(mask_state, np.uint8).copy()
    tok = as_int(tokens, np.int64).copy()
    phase = as_int(block_phase, np.uint8)
    n_rows = ms.shape[0]
    B = int(block_size)
    assert n_rows % B == 0
    n_blocks = n_rows // B
    t = tau_as_received(tau)

    conf = np.full(n_rows, np.nan)
    amax = np.full(n_rows, -1, dtype=np.int64)
    live = np.flatnonzero(ms == MASKED)
    if live.size:
        c, a = row_confidence(take_rows(logits, live))
        conf[live] = c
        amax[live] = a

    n_committed = np.zeros(n_blocks, dtype=np.int64)
    block_complete = np.zeros(n_blocks, dtype=np.uint8)
    near_tau = np.zeros(n_rows, dtype=bool)
    near_topk = np.zeros(n_blocks, dtype=bool)
    for k in range(n_blocks):
        rows = range(k * B, (k + 1) * B)
        cand = [p for p in rows if ms[p] == MASKED]
        chosen = {p for p in cand if conf[p] > t}
        for p in cand:
            near_tau[p] = abs(conf[p] - t) <= NEAR_TIE
        if phase[k] == AGGRESSIVE and k_aggr > 0:
            order = sorted(cand, key=lambda p: (-conf[p], p))
            chosen |= set(order[:k_aggr])
            if len(order) > k_aggr and abs(conf[order[k_aggr - 1]] - conf[order[k_aggr]]) <= NEAR_TIE:
                near_topk[k] = True
        for p in cand:
            if p in chosen:
                ms[p] = COMMITTED
                tok[p] = amax[p]
            else:
                tok[p] = mask_token_id
        n_committed[k] = len(chosen)
        block_complete[k] = 1 if all(ms[p] == COMMITTED for p in rows) else 0
    return dict(mask_state=ms, tokens=tok, conf=conf, argmax=amax, n_committed=n_committed,
                block_complete=block_complete, near_tau=near_tau, near_topk=near_topk)
