"""paged_gqa_decode_noalloc through the C ABI against paged_gqa_decode (the
entry point with a workspace) and the oracle, on two calls in a row, the
second with a smaller input: outputs identical bit for bit to the workspace
call's (the same kernels on the same inputs), within 2e-3 of the oracle,
device errors reported through the caller's word, and a call whose split
records would not fit the library's scratch array refused before any
launch."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_transformer_amd as pkv
import synth
from gpu_util import attention_oracle, dev, say

pytestmark = pytest.mark.gpu

ATOL = 2e-3


def _run_both(w, batch, page_tokens=16):
    """The first `batch` sequences of an attention workload through both
    entry points; returns (noalloc out, workspace out, noalloc error bits,
    workspace error bits)."""
    shape = w["shape"]
    Hq, Hkv, D = shape.heads, shape.kv_heads, shape.head_dim
    q = dev(np.ascontiguousarray(w["q"][:batch]))
    bt = dev(np.ascontiguousarray(w["block_table"][:batch]))
    lens = dev(np.ascontiguousarray(w["lens"][:batch]))
    pool_t = dev(w["pool"])
    pool = pkv.kv_pool_create(pool_t, Hkv, head_dim=D, page_tokens=page_tokens)
    out_a = torch.full((batch, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    out_b = torch.full((batch, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    err_word = pkv.alloc_workspace(256)
    say("noalloc: batch %d, lens %s" % (batch, w["lens"][:batch].tolist()))
    pkv.paged_gqa_decode_noalloc(pool, q, bt, lens, w["scale"], out_a, err_word)
    ws = pkv.alloc_workspace(pkv.attention_workspace_bytes(Hq, Hkv, batch, bt.shape[1], head_dim=D,
                                                           page_tokens=page_tokens))
    pkv.paged_gqa_decode(pool, q, bt, lens, w["scale"], out_b, ws)
    return out_a.cpu().numpy(), out_b.cpu().numpy(), pkv.device_error(err_word), pkv.device_error(ws)


def test_noalloc_matches_the_workspace_call_twice_then_smaller():
    w = synth.attention_workload()  # Llama-3.2-1B heads, batch 16, lengths U[1,2048]
    ref = attention_oracle(w["pool"], 8, w["q"], w["block_table"], w["lens"], w["scale"])
    for batch in (16, 5):
        a, b, err, err_ws = _run_both(w, batch)
        assert err == 0 and err_ws == 0
        assert np.array_equal(a, b), "noalloc and workspace calls differ (batch %d)" % batch
        diff = float(np.abs(a - ref[:batch]).max())
        say("noalloc batch %d: bitwise equal to the workspace call, max-abs %.3g vs the oracle" % (batch, diff))
        assert diff <= ATOL


def test_noalloc_reports_device_errors_in_the_callers_word():
    w = synth.attention_workload(batch=4)
    w["block_table"] = w["block_table"].copy()
    w["block_table"][1, 0] = w["num_pages"] + 5  # outside the pool
    a, b, err, err_ws = _run_both(w, 4)
    assert err == err_ws == pkv.DEVERR_PAGE
    keep = [0, 2, 3]
    assert np.array_equal(a[keep], b[keep])


def test_noalloc_refuses_calls_beyond_its_scratch():
    """Split records of 64 sequences x 8 kv heads over 2048-token tables
    (8 splits of 16 tiles, 4224 bytes each) need 17.3 MB, more than the
    16 MiB array: the call returns -ENOSPC and launches nothing (out keeps
    its NaNs)."""
    Hq, Hkv, D, B, mp = 32, 8, 64, 64, 128
    pool_t = torch.zeros(4 * synth.page_elems(Hkv), dtype=torch.int16, device="cuda")
    pool = pkv.kv_pool_create(pool_t, Hkv)
    q = torch.zeros((B, Hq, D), dtype=torch.int16, device="cuda")
    bt = torch.zeros((B, mp), dtype=torch.int32, device="cuda")
    lens = torch.ones(B, dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    err_word = pkv.alloc_workspace(256)
    rc = pkv.lib().paged_gqa_decode_noalloc(ctypes.byref(pool), q.data_ptr(), Hq, bt.data_ptr(), mp,
                                            lens.data_ptr(), B, 0.125, out.data_ptr(), err_word.data_ptr(),
                                            torch.cuda.current_stream().cuda_stream)
    assert rc == -28  # -ENOSPC
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    # the same call over 1024-token tables (4 splits, 8.65 MB) fits and runs
    rc = pkv.lib().paged_gqa_decode_noalloc(ctypes.byref(pool), q.data_ptr(), Hq, bt.data_ptr(), 64,
                                            lens.data_ptr(), B, 0.125, out.data_ptr(), err_word.data_ptr(),
                                            torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    assert pkv.device_error(err_word) == 0
    assert not torch.isnan(out).any()
