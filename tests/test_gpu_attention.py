"""GPU parity of d2f_block_attn (through the C ABI) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import workloads as W
from parity import compare_attn, oracle_attn, poisoned_inputs, run_attn, say

pytestmark = pytest.mark.gpu


def _check(shape, seed=0, pairs=None, label="", layer=0):
    say(f"--- attention case {label}: {shape}")
    x = poisoned_inputs(shape, seed=seed, layer=layer)
    out, lse = run_attn(shape, x, out_fill=7.0)
    ref_o, ref_l = oracle_attn(shape, x, pairs=pairs)
    stats = compare_attn(shape, out, lse, ref_o, ref_l, pairs=pairs, label=label)
    # Rows past each request's window are left untouched.
    o = out.float().cpu().numpy()
    for b in range(shape.batch):
        assert (o[b, :, shape.win_rows(b):] == 7.0).all()
    return x, out, lse, stats


def test_tiny_f32():
    c = W.config("tiny_f32")
    _check(c["shape"], label="tiny_f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", [
    # (nb, Hq, Hkv, D, B, prefix, nwin)
    (1, 2, 2, 64, 16, [0], [1]),            # no cache, single block
    (1, 2, 2, 64, 16, [0], [4]),            # no cache, 4 blocks
    (1, 4, 4, 64, 1, [37], [9]),            # B = 1: causal attention
    (1, 2, 2, 128, 5, [77], [3]),           # B does not divide the tile; ragged prefix
    (2, 8, 2, 64, 16, [130, 5], [2, 3]),    # GQA group 4, ragged batch
    (3, 4, 1, 128, 8, [1000, 64, 999], [4, 1, 2]),   # many key splits, GQA 4
    (1, 2, 2, 128, 64, [129], [3]),         # large B: window 192 rows > one query tile
    (1, 6, 2, 64, 48, [10], [2]),           # group 3, block straddles query tiles
    (1, 4, 2, 64, 128, [300], [8]),         # 1024-row window: a block spans 4 query tiles
    (1, 2, 2, 128, 256, [0], [4]),          # no cache, 1024-row window of 256-row blocks
    (2, 3, 1, 64, 32, [65, 2000], [16, 7]), # 512-row window, group 3, ragged window lengths
])
def test_edge_shapes(dtype, case):
    nb, hq, hkv, d, b, prefix, nwin = case
    shape = W.make_shape(nb, hq, hkv, d, b, prefix, nwin, dtype=dtype, extra_capacity=3)
    _check(shape, seed=sum(prefix) + b, label=f"edge-{dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_idle_requests(dtype):
    """n_win_blocks = 0 marks a request idle: its rows stay untouched and the
    others are computed as usual; a batch of idle requests launches nothing."""
    shape = W.make_shape(3, 4, 2, 64, 16, [50, 300, 7], [2, 0, 1], dtype=dtype,
                         extra_capacity=3)
    _check(shape, seed=11, label=f"idle-{dtype}")
    shape = W.make_shape(2, 2, 2, 128, 16, [40, 9], [0, 0], dtype=dtype, max_win_blocks=2)
    x = poisoned_inputs(shape, seed=12)
    out, lse = run_attn(shape, x, out_fill=7.0)
    assert (out.float() == 7.0).all() and (lse == 7.0).all()


def test_fp32_head_dim_32_long_prefix():
    shape = W.make_shape(2, 2, 2, 32, 16, [2100, 33], [3, 2], dtype="f32")
    _check(shape, label="f32-d32-split")


def test_explicit_softmax_scale():
    shape = W.make_shape(1, 2, 2, 64, 16, [100], [2], dtype="f32")
    x = poisoned_inputs(shape, seed=3)
    out, lse = run_attn(shape, x, softmax_scale=0.3)
    ro, rl = oracle_attn(shape, x, scale=0.3)
    compare_attn(shape, out, lse, ro, rl, label="scale0.3")


@pytest.mark.parametrize("d", [128, 64])
def test_many_groups_with_one_long_request(d):
    # More (request, KV head) groups than CUs selects the two-stage ring; the
    # long request is still cut into key ranges and merged.
    nb = 20 if d == 128 else 40
    hkv = 16 if d == 128 else 8
    prefix = [6000] + [100 + 37 * i for i in range(nb - 1)]
    shape = W.make_shape(nb, hkv, hkv, d, 16, prefix, [2] * nb, dtype="bf16")
    pairs = [(0, h) for h in range(0, hkv, 3)] + [(b, b % hkv) for b in range(1, nb, 4)]
    _check(shape, pairs=pairs, label=f"many-groups-d{d}")


def test_llada_p512_single_step():
    c = W.config("llada_p512")
    _check(c["shape"], label="llada_p512")


def test_llada_batch16_layers():
    c = W.config("llada_batch16")
    sh = c["shape"]
    _check(sh, label="llada_batch16-L0", layer=0)
    rng = np.random.default_rng(3)
    pairs = [(int(b), int(h)) for b, h in zip(rng.integers(0, sh.batch, 24),
                                              rng.integers(0, sh.n_heads_q, 24))]
    _check(sh, pairs=pairs, label="llada_batch16-L31-sampled", layer=31)


@pytest.mark.parametrize("bsz", [16, 32, 64])
def test_dream_gqa(bsz):
    c = W.config("dream_gqa", block_size=bsz)
    sh = c["shape"]
    pairs = [(0, h) for h in range(sh.n_heads_q)] + [(5, h) for h in (0, 6, 7, 13, 20, 27)]
    _check(sh, pairs=pairs, label=f"dream_gqa-B{bsz}")


def test_llada_p32k():
    c = W.config("llada_p32k")
    sh = c["shape"]
    pairs = [(0, h) for h in (0, 9, 17, 31)]
    _check(sh, pairs=pairs, label="llada_p32k")


def test_long_prefix_ranges_on_eight_waves():
    """A 16384-token prefix over 32 heads: the plan cuts each head's keys into
    8 ranges of ~33 tiles, one eight-wave unit per CU, merged exactly.
    Sampled heads against the oracle; two runs bit-identical."""
    shape = W.make_shape(1, 32, 32, 128, 16, [16384], [4], dtype="bf16")
    x, out, lse, _ = _check(shape, seed=21, pairs=[(0, 0), (0, 13), (0, 31)],
                            label="prefix16k-8ranges")
    o2, l2 = run_attn(shape, x, out_fill=7.0)
    assert torch.equal(out.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)


def test_context_128k():
    """A 131072-token prefix (the pages' open question about 100K+ contexts):
    sampled heads against the oracle; every unread slot is NaN."""
    shape = W.make_shape(1, 8, 8, 128, 16, [131072], [4], dtype="bf16")
    _check(shape, pairs=[(0, 0), (0, 5)], label="context-128k")


def test_deterministic_and_later_blocks_do_not_leak():
    shape = W.make_shape(2, 4, 2, 128, 16, [300, 1500], [4, 3], dtype="bf16")
    x = poisoned_inputs(shape, seed=11)
    o1, l1 = run_attn(shape, x, out_fill=0.0)
    o2, l2 = run_attn(shape, x, out_fill=0.0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # Re-draw q/K/V of window blocks >= 2: rows of blocks 0..1 must not change.
    y = {k: v.clone() for k, v in x.items()}
    lo = 2 * shape.block_size
    g = torch.Generator(device="cuda").manual_seed(99)
    for n in ("q", "k_win", "v_win"):
        for b in range(shape.batch):
            hi = shape.win_rows(b)
            r = torch.randn(y[n][b, :, lo:hi].shape, generator=g, device="cuda")
            y[n][b, :, lo:hi] = r.to(y[n].dtype)
    o3, l3 = run_attn(shape, y, out_fill=0.0)
    assert torch.equal(o3[:, :, :lo], o1[:, :, :lo])
    assert torch.equal(l3[:, :, :lo], l1[:, :, :lo])
    assert not torch.equal(o3[0, :, lo:64], o1[0, :, lo:64])
    say("[attn determinism/causality] ok")
