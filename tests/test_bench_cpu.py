"""Host logic of bench.py that runs without a GPU: the near-tie count it
reports next to the measurement, and the number of rotating input sets."""
import types

import torch

import bench


def _wl(conf, phases, block_size, k_aggr, tau=0.9, measure="maxprob", masked=None):
    n = len(conf)
    mask0 = torch.zeros(n, dtype=torch.uint8)
    if masked is not None:
        mask0 = torch.tensor([0 if m else 1 for m in masked], dtype=torch.uint8)
    return types.SimpleNamespace(measure=measure, tau=tau, k_aggr=k_aggr,
                                 conf=torch.tensor(conf, dtype=torch.float32), mask0=mask0,
                                 phases=torch.tensor(phases, dtype=torch.uint8),
                                 sh=types.SimpleNamespace(block_size=block_size))


def test_near_threshold_rows_are_counted():
    # 0.9000004 and 0.8999996 lie within 1e-6 of float32(0.9); 0.9 + 1e-5 does not
    wl = _wl([0.9000004, 0.8999996, 0.90001, 0.2], [0], 4, 0)
    r = bench.near_ties(wl)
    assert r["near_tau"] == 2 and r["near_topk"] == 0 and r["masked_rows"] == 4


def test_committed_rows_are_not_counted():
    wl = _wl([0.9000004, 0.9000004, 0.1, 0.2], [0], 4, 0, masked=[True, False, True, True])
    assert bench.near_ties(wl)["near_tau"] == 1


def test_near_topk_boundary_only_in_aggressive_blocks():
    # block 0 aggressive: 1st and 2nd confidences 4e-7 apart, below tau -> near
    # block 1 conservative: the same values do not count
    # block 2 aggressive: the 2nd clears tau, so the boundary decides nothing
    conf = [0.5000004, 0.5, 0.1, 0.05,
            0.5000004, 0.5, 0.1, 0.05,
            0.95, 0.9500004, 0.1, 0.05]
    wl = _wl(conf, [1, 0, 1], 4, 1)
    r = bench.near_ties(wl)
    assert r["near_topk"] == 1 and r["near_tau"] == 0


def test_k_aggr_two_and_measure_band():
    # logit gap: band 1e-5; the 2nd and 3rd gaps are 5e-6 apart, below tau = 5
    wl = _wl([3.0, 2.000005, 2.0, 0.5], [1], 4, 2, tau=5.0, measure="logit_gap")
    r = bench.near_ties(wl)
    assert r["near_topk"] == 1 and r["band"] == 1e-5
    wl = _wl([3.0, 2.1, 2.0, 0.5], [1], 4, 2, tau=5.0, measure="logit_gap")
    assert bench.near_ties(wl)["near_topk"] == 0


MB = 1 << 20


def _reuse_distance(n_sets, call_bytes):
    # a call cycling through n sets reads n - 1 others between two reads of one set
    return (n_sets - 1) * call_bytes


def test_input_sets_outrun_the_cache_for_the_step_and_each_call():
    # LLaDA single-step sizes: 25.6 MB read per step, 9.4 MB per attention call
    n = bench.input_set_count(25.6 * MB, 9.4 * MB, 26 * MB)
    assert _reuse_distance(n, 9.4 * MB) >= bench.ROTATE_BYTES
    assert _reuse_distance(n, 25.6 * MB) >= bench.ROTATE_BYTES
    assert n * 26 * MB <= bench.SET_BUDGET_BYTES


def test_input_sets_stay_within_the_budget_for_large_sets():
    # 35 GB sets (32 layers of a batched cache): the per-step rule alone applies
    n = bench.input_set_count(19_000 * MB, 324 * MB, 35_000 * MB)
    assert n == 2


def test_input_sets_budget_caps_the_per_call_rule():
    # per-call rule asks for 1 + ceil(640 / 1) = 641 sets; 1 GB sets cap it at 64
    n = bench.input_set_count(2_000 * MB, 1 * MB, 1 << 30)
    assert n == bench.SET_BUDGET_BYTES // (1 << 30)


def test_kernel_short_name_reads_mangled_and_demangled_names():
    import bench
    assert bench.kernel_short_name(
        "_ZN3d2f12_GLOBAL__N_117attn_merge_kernelILi128EDF16bEEvNS_8AttnArgsE") == \
        "attn_merge_kernel<128, __bf16>"
    assert bench.kernel_short_name(
        "void d2f::(anonymous namespace)::attn_bf16_kernel<128, 2, 0, 2>(d2f::AttnArgs)") == \
        "attn_bf16_kernel<128, 2, 0, 2>"
    assert bench.kernel_short_name(
        "_ZN3d2f12_GLOBAL__N_119vocab_reduce_kernelILb1ELi0EEEvNS_10CommitArgsE") == \
        "vocab_reduce_kernel<true, 0>"
    assert bench.kernel_short_name("void at::native::fill_kernel(int)") is None


def test_stall_breakdown_shares_and_per_wave_counts():
    """Shares are the wave-cycle counters over SQ_WAVE_CYCLES, counts are per
    wave, and the co-execution share is taken of the MFMA busy cycles."""
    v = {c: 0.0 for cs in bench.STALL_COUNTERS for c in cs}
    v.update({"SQ_WAVE_CYCLES": 1000.0, "SQ_ACTIVE_INST_ANY": 300.0, "SQ_WAIT_ANY": 400.0,
              "SQ_WAIT_INST_ANY": 250.0, "SQ_ACTIVE_INST_VALU": 200.0, "SQ_ACTIVE_INST_SCA": 50.0,
              "SQ_WAVES": 10.0, "SQ_INSTS_MFMA": 70.0, "SQ_INSTS_SALU": 35.0,
              "SQ_VALU_MFMA_BUSY_CYCLES": 2048.0, "SQ_VALU_MFMA_COEXEC_CYCLES": 512.0})
    r = bench.stall_breakdown(v)
    s = r["share_of_wave_cycles"]
    assert s["issuing_any"] == 0.3 and s["waiting_on_counters_or_barrier"] == 0.4
    assert s["waiting_to_issue"] == 0.25 and s["valu"] == 0.2 and s["scalar"] == 0.05
    assert r["instructions_per_wave"]["mfma"] == 7.0 and r["instructions_per_wave"]["salu"] == 3.5
    assert r["mfma_busy_cycles_per_simd"] == 2 and r["coexec_share_of_mfma_busy"] == 0.25
    assert all(len(cs) <= 8 for cs in bench.STALL_COUNTERS)  # one pass holds <= 8 SQ counters


def test_other_workloads_name_configs_the_targets_are_set_on():
    import workloads as W
    names = set()
    for name, bs in bench.OTHER_WORKLOADS:
        cfg = W.config(name, block_size=bs)
        sh = cfg["shape"]
        names.add((name, sh.block_size))
        if name == "dream_gqa":  # grouped-query, MFMA-bound at these shapes
            assert sh.n_heads_q > sh.n_heads_kv and sh.block_size == bs
            assert bench.attn_flops(sh) / bench.attn_bytes(sh) > 200
    assert {("dream_gqa", 16), ("dream_gqa", 32), ("dream_gqa", 64)} <= names
    assert any(n == "llada_p32k" for n, _ in names)
    import sys
    old = sys.argv  # parse() reads sys.argv
    try:
        sys.argv = ["bench.py", "--gpus", "1", "--steps", "20", "--warmup", "5"]
        a = bench.parse()
        assert a.other_workloads and a.config == "llada_batch16"
        sys.argv = ["bench.py", "--no-other-workloads"]
        assert not bench.parse().other_workloads
        # a run that names its workload (the profiling commands) times only that
        sys.argv = ["bench.py", "--config", "llada_batch16", "--steps", "2"]
        a = bench.parse()
        assert not a.other_workloads and a.config == "llada_batch16"
    finally:
        sys.argv = old
