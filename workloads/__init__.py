"""Seeded synthetic inputs for one D2F denoising step.

This module only draws random tensors and lays them out; it holds none of
the method's arithmetic (no attention, no softmax, no commit rule).  Both the
fp64 oracle (``oracle/``) and the HIP library's tests and benchmark draw
their inputs from here, so the two sides see the same bits.

The shapes follow the workloads the D2F pages report on: LLaDA-8B attention
heads (32 query heads, 32 KV heads, head_dim 128), a Dream-7B-like grouped
variant (28 query heads over 4 KV heads), block size 16 as the reported
balance point with 32/64 as the larger-B sweep, vocabularies of 126464 and
152064 entries.  No benchmark item, prompt or model weight is reproduced:
every tensor is Gaussian noise with the stated mean and standard deviation.

Every tensor has its own generator, seeded ``1000 * layer + tid`` (plus a
per-config base seed), so one tensor can be regenerated without drawing the
others.  Integer host-side draws (prefix lengths, window sizes, mask states)
always use a CPU generator so that they are identical on every machine.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import torch

# Byte encodings shared by the C ABI and the oracle (data format, not arithmetic).
MASKED = 0
COMMITTED = 1
CONSERVATIVE = 0
AGGRESSIVE = 1

TID = dict(q=1, k_cache=2, v_cache=3, k_win=4, v_win=5, logits=6, boost_col=7,
           boost_delta=8, mask_state=9, prefix_len=10, n_win=11, tokens=12)


def _gen(device, seed: int, layer: int, tid: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) + 1000 * int(layer) + int(tid))
    return g


def _torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@dataclasses.dataclass
class AttnShape:
    """Geometry of one attention call (one layer).

    Layouts (row-major, innermost last):
      q, out      [batch][n_heads_q][max_win_blocks*block_size][head_dim]
      k/v cache   [batch][n_heads_kv][cache_capacity][head_dim]
      k/v window  [batch][n_heads_kv][max_win_blocks*block_size][head_dim]
    """
    batch: int
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    block_size: int
    max_win_blocks: int
    cache_capacity: int
    dtype: str  # "f32" or "bf16"
    prefix_len: List[int]
    n_win_blocks: List[int]

    @property
    def w_max(self) -> int:
        return self.max_win_blocks * self.block_size

    def win_rows(self, b: int) -> int:
        return self.n_win_blocks[b] * self.block_size


def make_shape(batch, n_heads_q, n_heads_kv, head_dim, block_size, prefix_len,
               n_win_blocks, dtype="bf16", max_win_blocks=None, extra_capacity=0,
               cache_capacity=None) -> AttnShape:
    prefix_len = [int(p) for p in prefix_len]
    n_win_blocks = [int(n) for n in n_win_blocks]
    if max_win_blocks is None:
        max_win_blocks = max(n_win_blocks) if n_win_blocks else 1
    if cache_capacity is None:
        need = max([p + n * block_size for p, n in zip(prefix_len, n_win_blocks)] or [0])
        cache_capacity = max(need + int(extra_capacity), 1)
    return AttnShape(batch, n_heads_q, n_heads_kv, head_dim, block_size,
                     max_win_blocks, int(cache_capacity), dtype, prefix_len, n_win_blocks)


def attn_inputs(shape: AttnShape, layer: int = 0, device="cpu", seed: int = 0,
                poison: bool = False, tid_offset: int = 0) -> Dict[str, torch.Tensor]:
    """q, k_cache, v_cache, k_win, v_win ~ N(0, 1), cast to the shape's dtype.

    bf16 tensors are drawn in fp32 and rounded to nearest-even by ``.to``.
    With ``poison`` every slot that the step must not read (cache slots at or
    past prefix_len[b], window rows at or past n_win_blocks[b]*block_size) is
    set to NaN, so a kernel that reads one produces NaN outputs.
    """
    dt = _torch_dtype(shape.dtype)
    nb, hq, hkv, d = shape.batch, shape.n_heads_q, shape.n_heads_kv, shape.head_dim
    w = shape.w_max
    cap = shape.cache_capacity

    def draw(name, dims):
        g = _gen(device, seed + tid_offset, layer, TID[name])
        return torch.randn(dims, generator=g, device=device, dtype=torch.float32).to(dt)

    out = dict(
        q=draw("q", (nb, hq, w, d)),
        k_cache=draw("k_cache", (nb, hkv, cap, d)),
        v_cache=draw("v_cache", (nb, hkv, cap, d)),
        k_win=draw("k_win", (nb, hkv, w, d)),
        v_win=draw("v_win", (nb, hkv, w, d)),
    )
    if poison:
        nan = float("nan")
        for b in range(nb):
            p, wb = shape.prefix_len[b], shape.win_rows(b)
            out["k_cache"][b, :, p:, :] = nan
            out["v_cache"][b, :, p:, :] = nan
            out["k_win"][b, :, wb:, :] = nan
            out["v_win"][b, :, wb:, :] = nan
            out["q"][b, :, wb:, :] = nan
    return out


def fresh_block(shape: AttnShape, name: str, it: int, device="cpu", seed: int = 0,
                layer: int = 0) -> torch.Tensor:
    """One newly appended window block for tensor ``name`` (q, k_win or v_win):
    [batch][heads][block_size][head_dim], drawn with tid + 100*it."""
    heads = shape.n_heads_q if name == "q" else shape.n_heads_kv
    g = _gen(device, seed, layer, TID[name] + 100 * (it + 1))
    x = torch.randn((shape.batch, heads, shape.block_size, shape.head_dim), generator=g,
                    device=device, dtype=torch.float32)
    return x.to(_torch_dtype(shape.dtype))


@dataclasses.dataclass
class CommitInputs:
    logits: torch.Tensor       # [rows][vocab] fp32
    mask_state: torch.Tensor   # [rows] uint8
    tokens: torch.Tensor       # [rows] int32
    block_phase: torch.Tensor  # [rows // block_size] uint8
    block_size: int
    mask_token_id: int


def logits_normal(rows: int, vocab: int, std: float, boost: bool, device="cpu",
                  seed: int = 0, layer: int = 0, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 logits ~ N(0, std) (std is the standard deviation).

    With ``boost``, one column per row, uniform over the vocabulary, is raised
    to (largest of the row's other entries) + delta with delta ~ U(2, 8), so
    that the rows' top probabilities spread over roughly 0.15 .. 0.99.
    """
    g = _gen(device, seed, layer, TID["logits"])
    if out is None:
        out = torch.empty((rows, vocab), device=device, dtype=torch.float32)
    out.normal_(0.0, std, generator=g)
    if boost and rows > 0 and vocab > 1:  # one column: no other entries to exceed
        gc = _gen("cpu", seed, layer, TID["boost_col"])
        gd = _gen("cpu", seed, layer, TID["boost_delta"])
        cols = torch.randint(0, vocab, (rows,), generator=gc)
        delta = torch.rand((rows,), generator=gd, dtype=torch.float32) * 6.0 + 2.0
        cols_d = cols.to(device)
        ar = torch.arange(rows, device=device)
        out[ar, cols_d] = -float("inf")
        top = out.max(dim=1).values
        out[ar, cols_d] = top + delta.to(device)
    return out


def commit_inputs(rows: int, vocab: int, block_size: int, phases: Sequence[int], std: float,
                  boost: bool, committed_frac: float = 0.0, device="cpu", seed: int = 0,
                  layer: int = 0, mask_token_id: Optional[int] = None) -> CommitInputs:
    """Logits plus the per-position mask state and per-block phase of a window.

    A fraction ``committed_frac`` of positions (Bernoulli per position) start
    COMMITTED with a random token; the rest are MASKED and hold mask_token_id.
    """
    assert rows % block_size == 0 and len(phases) == rows // block_size
    if mask_token_id is None:
        mask_token_id = vocab  # a synthetic id outside the logit columns
    logits = logits_normal(rows, vocab, std, boost, device, seed, layer)
    gm = _gen("cpu", seed, layer, TID["mask_state"])
    committed = torch.rand((rows,), generator=gm) < committed_frac
    mask_state = torch.where(committed, COMMITTED, MASKED).to(torch.uint8)
    gt = _gen("cpu", seed, layer, TID["tokens"])
    tok = torch.randint(0, vocab, (rows,), generator=gt, dtype=torch.int32)
    tokens = torch.where(committed, tok, torch.full_like(tok, mask_token_id))
    phase = torch.tensor(list(phases), dtype=torch.uint8)
    return CommitInputs(logits, mask_state.to(device), tokens.to(device), phase.to(device),
                        block_size, int(mask_token_id))


def window_phases(n_win_blocks: Sequence[int]) -> List[int]:
    """Per-block phases of a batch's windows, concatenated request by request:
    the newest block of each window is CONSERVATIVE, older ones AGGRESSIVE."""
    out = []
    for n in n_win_blocks:
        out += [AGGRESSIVE] * (n - 1) + [CONSERVATIVE]
    return out


# ---------------------------------------------------------------------------
# The five workloads.
# ---------------------------------------------------------------------------

def ragged_batch(batch: int, p_lo: int, p_hi: int, nw_lo: int, nw_hi: int, seed: int = 0):
    """Prefix lengths ~ U{p_lo..p_hi} and window sizes ~ U{nw_lo..nw_hi}."""
    gp = _gen("cpu", seed, 0, TID["prefix_len"])
    gn = _gen("cpu", seed, 0, TID["n_win"])
    prefix = torch.randint(p_lo, p_hi + 1, (batch,), generator=gp).tolist()
    nwin = torch.randint(nw_lo, nw_hi + 1, (batch,), generator=gn).tolist()
    return prefix, nwin


def config(name: str, block_size: Optional[int] = None) -> dict:
    """Parameters of a named workload.  ``block_size`` picks one point of the
    Dream-shaped B sweep (16, 32 or 64)."""
    if name == "tiny_f32":
        shape = make_shape(1, 2, 2, 32, 16, [48], [3], dtype="f32")
        return dict(name=name, workload="tiny fp32 D2F step", shape=shape, layers=1,
                    vocab=512, logit_std=2.0, boost=False, committed_frac=0.3,
                    phases=[AGGRESSIVE, AGGRESSIVE, CONSERVATIVE], taus=[0.9], k_aggr=1)
    if name == "llada_p512":
        shape = make_shape(1, 32, 32, 128, 16, [512], [2], dtype="bf16")
        return dict(name=name, workload="LLaDA-8B-shaped single step", shape=shape, layers=1,
                    vocab=126464, logit_std=3.0, boost=True, committed_frac=0.0,
                    phases=window_phases([2]), taus=[0.9], k_aggr=1)
    if name == "llada_batch16":
        prefix, nwin = ragged_batch(16, 256, 4096, 1, 4)
        shape = make_shape(16, 32, 32, 128, 16, prefix, nwin, dtype="bf16", max_win_blocks=4)
        return dict(name=name, workload="batched ragged decode at LLaDA-8B shape", shape=shape,
                    layers=32, vocab=126464, logit_std=3.0, boost=True, committed_frac=0.0,
                    phases=window_phases(nwin), taus=[0.9], k_aggr=1)
    if name == "dream_gqa":
        b = 16 if block_size is None else int(block_size)
        assert b in (16, 32, 64)
        shape = make_shape(8, 28, 4, 128, b, [2048] * 8, [3] * 8, dtype="bf16")
        return dict(name=name, workload=f"Dream-7B-shaped GQA step, B={b}", shape=shape,
                    layers=1, vocab=152064, logit_std=3.0, boost=True, committed_frac=0.0,
                    phases=window_phases([3] * 8), taus=[0.8, 0.95], k_aggr=1)
    if name == "llada_p32k":
        shape = make_shape(1, 32, 32, 128, 16, [32768], [4], dtype="bf16", extra_capacity=1024)
        return dict(name=name, workload="long-context step, 32K prefix", shape=shape, layers=1,
                    vocab=126464, logit_std=3.0, boost=True, committed_frac=0.0,
                    phases=window_phases([4]), taus=[0.9], k_aggr=1, n_kv_commits=64)
    if name == "llada_p128k":
        # The pages' open question about 100K+ token contexts, at the LLaDA shape.
        shape = make_shape(1, 32, 32, 128, 16, [131072], [4], dtype="bf16", extra_capacity=1024)
        return dict(name=name, workload="long-context step, 128K prefix", shape=shape, layers=1,
                    vocab=126464, logit_std=3.0, boost=True, committed_frac=0.0,
                    phases=window_phases([4]), taus=[0.9], k_aggr=1)
    raise KeyError(name)


def config_commit_inputs(cfg: dict, device="cpu", seed: int = 0) -> CommitInputs:
    shape = cfg["shape"]
    rows = sum(shape.win_rows(b) for b in range(shape.batch))
    return commit_inputs(rows, cfg["vocab"], shape.block_size, cfg["phases"], cfg["logit_std"],
                         cfg["boost"], cfg["committed_frac"], device=device, seed=seed)


def total_rows(shape: AttnShape) -> int:
    """Window positions of the whole batch (the commit pass's row count)."""
    return sum(shape.win_rows(b) for b in range(shape.batch))


# ---- Synthetic multi-step decoding (the active-window loop) ----

def decode_rows(vocab: int, positions: Sequence[int], ages: Sequence[int], step: int,
                seed: int = 0, std: float = 3.0) -> torch.Tensor:
    """fp32 logits of window rows for one synthetic decoding step (CPU).

    Row r belongs to absolute position positions[r] of a block that has been in
    the window for ages[r] steps.  Entries ~ N(0, std) drawn from a generator
    keyed by (seed, step, position); one column per position (fixed over
    steps, drawn from (seed, position)) is raised above the row's largest
    other entry by 1.5 * age + u, u ~ U(0, 2) from (seed, step, position), so
    that positions grow more confident the longer their block is active."""
    out = torch.empty((len(positions), vocab), dtype=torch.float32)
    for r, (pos, age) in enumerate(zip(positions, ages)):
        g = torch.Generator().manual_seed(int(seed) * 1_000_003 + int(step) * 7919 + int(pos) * 131)
        row = torch.randn(vocab, generator=g) * std
        gc = torch.Generator().manual_seed(int(seed) * 1_000_003 + 17 + int(pos) * 977)
        col = int(torch.randint(0, vocab, (1,), generator=gc))
        u = float(torch.rand(1, generator=g)) * 2.0
        row[col] = -float("inf")
        row[col] = float(row.max()) + 1.5 * int(age) + u
        out[r] = row
    return out


def decode_window_kv(n_heads: int, head_dim: int, positions: Sequence[int], step: int, tid: int,
                     seed: int = 0, dtype: str = "bf16") -> torch.Tensor:
    """[n_heads][len(positions)][head_dim] ~ N(0, 1) for the window rows of one
    synthetic decoding step (CPU), keyed by (seed, step, position, tensor)."""
    out = torch.empty((n_heads, len(positions), head_dim), dtype=torch.float32)
    for r, pos in enumerate(positions):
        g = torch.Generator().manual_seed(int(seed) * 1_000_003 + int(step) * 7919 + int(pos) * 131
                                          + 100_000 * int(tid))
        out[:, r, :] = torch.randn((n_heads, head_dim), generator=g)
    return out.to(_torch_dtype(dtype))
