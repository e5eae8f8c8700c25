"""The commit pass without a workspace (d2f_confidence_commit_noalloc, for
callers that cannot allocate) against the commit pass with a caller
workspace (d2f_confidence_commit): the same kernels, so every output must be
identical, on two calls in a row with the second one smaller (the scratch
array keeps the first call's partials); and its size limit."""
import ctypes
import os

import pytest
import torch

import workloads as W
from block_causal_attention_d2f_amd import _binding as B

OK, INVALID, WORKSPACE = 0, 1, 4
FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: these calls fail validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libd2f.so not built")
    return B.load()


def _need(lib, rows, vocab):
    n = ctypes.c_size_t(0)
    assert lib.d2f_confidence_commit_workspace_size(rows, vocab, ctypes.byref(n)) == OK
    return n.value


def _noalloc(lib, rows, vocab):
    return lib.d2f_confidence_commit_noalloc(FAKE, vocab, rows, vocab, FAKE, FAKE, FAKE, 16,
                                             ctypes.c_float(0.9), 1, 0, None, None, FAKE, FAKE,
                                             None)


def test_size_limit_and_argument_errors(lib):
    # 16384 rows over 32 vocabulary chunks: 8 MiB of partials plus two words a row
    assert _need(lib, 16384, 262144) > B.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, 16384, 262144) == WORKSPACE
    assert b"8388608" in lib.d2f_last_error()
    assert _need(lib, 8192, 262144) <= B.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, -16, 1000) == INVALID
    assert _noalloc(lib, 16, 0) == INVALID
    assert _noalloc(lib, 0, 1000) == OK  # no rows: nothing to do


def _case(name, bsz=None):
    c = W.config(name, block_size=bsz)
    return c, W.config_commit_inputs(c, device="cuda")


def _outputs(ci, n_blocks):
    rows = ci.mask_state.numel()
    return dict(mask_state=ci.mask_state.clone(), tokens=ci.tokens.clone(),
                n_committed=torch.full((n_blocks,), -7, dtype=torch.int32, device="cuda"),
                block_complete=torch.full((n_blocks,), 9, dtype=torch.uint8, device="cuda"),
                conf=torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda"),
                argmax=torch.full((rows,), -1, dtype=torch.int32, device="cuda"))


@pytest.mark.gpu
def test_noalloc_equals_the_workspace_call_on_two_calls():
    import sys
    # Dream-shaped B = 64 pass (1536 rows x 152064), then the LLaDA single step
    # (32 rows x 126464), smaller, on the same scratch array.
    # The first call on a device looks up the scratch array's address, which
    # may make the runtime load the array; from then on a call allocates
    # nothing, which the second call checks through the free device memory.
    for call, (label, (c, ci)) in enumerate((("dream_gqa B=64", _case("dream_gqa", 64)),
                                             ("llada_p512", _case("llada_p512")))):
        print(f"[no-alloc] {label}", file=sys.stderr, flush=True)
        B_ = ci.block_size
        rows = ci.mask_state.numel()
        n_blocks = rows // B_
        tau, k = c["taus"][0], c["k_aggr"]
        ref = _outputs(ci, n_blocks)
        B.d2f_confidence_commit(ci.logits, ref["mask_state"], ref["tokens"], ci.block_phase, B_,
                                tau, k, ci.mask_token_id, conf_out=ref["conf"],
                                argmax_out=ref["argmax"], n_committed=ref["n_committed"],
                                block_complete=ref["block_complete"])
        got = _outputs(ci, n_blocks)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        B.d2f_confidence_commit_noalloc(ci.logits, got["mask_state"], got["tokens"],
                                        ci.block_phase, B_, tau, k, ci.mask_token_id,
                                        conf_out=got["conf"], argmax_out=got["argmax"],
                                        n_committed=got["n_committed"],
                                        block_complete=got["block_complete"])
        torch.cuda.synchronize()
        if call > 0:
            assert torch.cuda.mem_get_info()[0] >= free0, label
        for key in ref:
            a, b = ref[key], got[key]
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (label, key)
        committed = int(got["n_committed"].sum())
        assert committed > 0, label
        print(f"[no-alloc] {label}: {rows} rows, {committed} committed, identical",
              file=sys.stderr, flush=True)
