"""The C ABI from plain C: tests/c_consumer/consumer.c (C99; d2f.h and the
HIP runtime API only) runs one D2F step -- attention with a split key range,
the commit pass, the KV append -- and error calls, and writes its results to a
file.  Here the same inputs are regenerated from the published SplitMix64
definition and the results are compared with the fp64 oracle.  The consumer
is a shared library loaded in this process (no child process)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OA
from oracle import commit as OC
from oracle import kv_cache as OK
from parity import compare_attn, say

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "c_consumer", "libd2f_consumer.so")

# the consumer's problem (consumer.c)
NB, HQ, HKV, D, BS, MAXW, CAP = 2, 4, 2, 64, 16, 2, 2048
WMAX = MAXW * BS
PREFIX, NWIN = [37, 2000], [2, 1]
ROWS, VOCAB, MASK_ID, TAU, K_AGGR = 32, 1000, 1000, 0.5, 1
NAN_BF16, FILL_BF16 = 0x7FC0, 0x7F7F
D2F_OK, D2F_ERR_ORDER, D2F_ERR_WORKSPACE = 0, 3, 4


def splitmix64(seed, n):
    """Draws 1..n of SplitMix64 started at `seed` (Steele, Lea and Flood,
    OOPSLA 2014; 64-bit finaliser as published by Vigna), mod 2^64."""
    z = np.uint64(seed) + np.arange(1, n + 1, dtype=np.uint64) * np.uint64(0x9E3779B97F4A7C15)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def unit_values(seed, n):
    """2 (x >> 40) / 2^24 - 1 for each draw, exact in float32."""
    return ((splitmix64(seed, n) >> np.uint64(40)).astype(np.float32) * np.float32(2.0 ** -24)
            * np.float32(2.0) - np.float32(1.0))


def bf16_tensor(seed, shape):
    v = unit_values(seed, int(np.prod(shape))).reshape(shape)
    return torch.from_numpy(v).to(torch.bfloat16)  # round to nearest even


def inputs():
    q = bf16_tensor(1, (NB, HQ, WMAX, D))
    kc, vc = bf16_tensor(2, (NB, HKV, CAP, D)), bf16_tensor(3, (NB, HKV, CAP, D))
    kw, vw = bf16_tensor(4, (NB, HKV, WMAX, D)), bf16_tensor(5, (NB, HKV, WMAX, D))
    nan = torch.tensor(NAN_BF16, dtype=torch.int16).view(torch.bfloat16)
    for b in range(NB):
        kc[b, :, PREFIX[b]:] = nan
        vc[b, :, PREFIX[b]:] = nan
        kw[b, :, NWIN[b] * BS:] = nan
        vw[b, :, NWIN[b] * BS:] = nan
        q[b, :, NWIN[b] * BS:] = nan
    logits = (np.float32(4.0) * unit_values(6, ROWS * VOCAB)).reshape(ROWS, VOCAB)
    for r in range(0, ROWS, 3):
        logits[r, (r * 37) % VOCAB] += np.float32(10.0)
    xm, xt = splitmix64(7, ROWS), splitmix64(8, ROWS)
    committed = (xm >> np.uint64(62)) == 0
    mask = np.where(committed, W.COMMITTED, W.MASKED).astype(np.uint8)
    tokens = np.where(committed, (xt % np.uint64(VOCAB)).astype(np.int64), MASK_ID).astype(np.int32)
    phase = np.array([W.AGGRESSIVE, W.CONSERVATIVE], np.uint8)
    return q, kc, vc, kw, vw, logits, mask, tokens, phase


def read_results(path):
    nq, nl, nc = NB * HQ * WMAX * D, NB * HQ * WMAX, NB * HKV * CAP * D
    spec = [("status", np.int32, 8), ("out", np.uint16, nq), ("lse", np.float32, nl),
            ("conf", np.float32, ROWS), ("argmax", np.int32, ROWS), ("mask", np.uint8, ROWS),
            ("tokens", np.int32, ROWS), ("n_committed", np.int32, ROWS // BS),
            ("complete", np.uint8, ROWS // BS), ("k_cache", np.uint16, nc),
            ("v_cache", np.uint16, nc), ("prefix", np.int32, NB)]
    raw = open(path, "rb").read()
    res, off = {}, 0
    for name, dt, n in spec:
        res[name] = np.frombuffer(raw, dtype=dt, count=n, offset=off)
        off += n * np.dtype(dt).itemsize
    assert off == len(raw), (off, len(raw))
    return res


def test_consumer_library_exports_its_entry():
    if not os.path.exists(LIB):
        pytest.skip("libd2f_consumer.so not built")
    assert hasattr(ctypes.CDLL(LIB), "d2f_consumer_run")


@pytest.mark.gpu
def test_plain_c_consumer_against_oracle(tmp_path):
    import block_causal_attention_d2f_amd as d2f
    d2f.load()  # the library the consumer links (same file, loaded once)
    assert os.path.exists(LIB), f"{LIB} missing: build with __graft_entry__.build()"
    lib = ctypes.CDLL(LIB)
    lib.d2f_consumer_run.restype = ctypes.c_int
    lib.d2f_consumer_run.argtypes = [ctypes.c_char_p]
    path = str(tmp_path / "consumer.bin")
    say("--- C consumer: one step through the C ABI from plain C")
    rc = lib.d2f_consumer_run(path.encode())
    assert rc == 0, f"consumer returned {rc}"
    r = read_results(path)
    st = r["status"].tolist()
    assert st == [D2F_OK, D2F_ERR_WORKSPACE, D2F_OK, D2F_OK, D2F_OK, D2F_ERR_ORDER, D2F_OK, 0], st
    q, kc, vc, kw, vw, logits, mask, tokens, phase = inputs()

    # attention: the oracle on the same bits, the standard bf16 tolerances;
    # rows past each window keep the consumer's fill
    sh = W.make_shape(NB, HQ, HKV, D, BS, PREFIX, NWIN, dtype="bf16", max_win_blocks=MAXW,
                      cache_capacity=CAP)
    ref_o, ref_l = OA.block_attn(q, kc, vc, kw, vw, PREFIX, NWIN, BS)
    out_bits = r["out"].reshape(NB, HQ, WMAX, D)
    out = torch.from_numpy(out_bits.astype(np.int16)).view(torch.bfloat16)
    lse = torch.from_numpy(r["lse"].reshape(NB, HQ, WMAX).copy())
    compare_attn(sh, out, lse, ref_o, ref_l, label="c-consumer")
    for b in range(NB):
        assert (out_bits[b, :, NWIN[b] * BS:] == FILL_BF16).all()
        assert (lse[b, :, NWIN[b] * BS:] == 7.0).all()

    # commit: decisions bit-exact outside the band around tau
    ref = OC.confidence_commit(torch.from_numpy(logits), torch.from_numpy(mask),
                               torch.from_numpy(tokens), torch.from_numpy(phase), BS, TAU, K_AGGR,
                               MASK_ID)
    ok = ~ref["near_tau"]
    for j in range(ROWS // BS):
        if ref["near_topk"][j]:
            ok[j * BS:(j + 1) * BS] = False
    live = ~np.isnan(ref["conf"])
    assert (r["argmax"][live] == ref["argmax"][live]).all()
    assert (r["mask"][ok] == ref["mask_state"][ok]).all()
    assert (r["tokens"][ok] == ref["tokens"][ok]).all()
    assert np.abs(r["conf"][live] - ref["conf"][live]).max() <= OC.NEAR["maxprob"]
    if ok.all():
        assert (r["n_committed"] == ref["n_committed"]).all()
        assert (r["complete"] == ref["block_complete"]).all()
    say(f"[c-consumer commit] live={int(live.sum())} committed={int(ref['n_committed'].sum())} "
        f"near_tau={int(ref['near_tau'].sum())}")

    # KV append of request 0's oldest block: byte-exact, prefix 37 -> 53
    kb = kc.view(torch.int16).numpy().view(np.uint16)
    vb = vc.view(torch.int16).numpy().view(np.uint16)
    kwb = kw.view(torch.int16).numpy().view(np.uint16)
    vwb = vw.view(torch.int16).numpy().view(np.uint16)
    k2, v2, p2 = OK.kv_commit(kb, vb, kwb, vwb, PREFIX, 0, BS)
    assert r["prefix"].tolist() == p2 == [53, 2000]
    assert np.array_equal(r["k_cache"].reshape(k2.shape), k2)
    assert np.array_equal(r["v_cache"].reshape(v2.shape), v2)
