"""GPU parity of prefill (one sequence's prompt into the pool) through the
C ABI.  Bars: the last token's logits max-abs <= 1e-2 * RMS(logits); the
argmax identical wherever the oracle's top-2 gap exceeds 1e-3; every K/V
value written within one BF16 ulp of the oracle's (or 1e-3 of their RMS)
and the rest of the pool untouched.  Against the library's own decode step
the prompt's pages and the last logits are bit-identical: each prompt token
goes through the arithmetic of a decode step at its position."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_transformer_amd as pkv
import synth
from gpu_util import check_argmax_rule, check_pool_after, dev, host_u16, say

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _rms(a):
    return float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))


def _inputs(shape, seed, start, T, weights=None):
    wl = synth.decode_workload("prefill", shape, seed, [start + T - 1])
    w = weights or synth.model_weights(shape, seed, sigma=0.05, norm_sigma=0.3)
    tokens = synth.rng(seed, "prompt").integers(0, shape.vocab, size=T).astype(np.int32)
    return w, wl.pool, wl.block_tables[:, 0], tokens


def prefill_gpu(shape, weights, pool_np, bts, start, tokens, model=None):
    T = len(tokens)
    mp = start + T
    cfg = pkv.make_config(shape, max_pos=mp)
    model = model or pkv.upload_model(weights, shape.theta, mp)
    pool_t = dev(pool_np)
    pool = pkv.kv_pool_create(pool_t, shape.kv_heads)
    bts = np.ascontiguousarray(bts, dtype=np.int32)
    ws = pkv.alloc_workspace(pkv.prefill_workspace_bytes(cfg, T, bts.shape[1]))
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    nxt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pkv.prefill(cfg, model, pool, dev(bts), start, dev(tokens), logits, nxt, ws)
    err = pkv.device_error(ws)
    return logits.cpu().numpy(), int(nxt.cpu()[0]), host_u16(pool_t), err


@pytest.mark.parametrize("start,T", [(0, 37), (11, 20), (5, 1)])
def test_prefill_tiny_model_matches_oracle(start, T):
    shape = synth.tiny_shape(hidden=128, layers=3, heads=4, kv_heads=2, inter=256, vocab=1000)
    w, pool, bts, tokens = _inputs(shape, 40 + start, start, T)
    logits, nxt, pool_after, err = prefill_gpu(shape, w, pool, bts, start, tokens)
    assert err == 0
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    ref, ref_tok, ref_pool = oracle.prefill_paged(shape, w, pool, geo, bts, start, tokens)
    diff = np.abs(logits - ref).max()
    say("prefill tiny start %d T %d: max|dlogit| %.3g (RMS %.3g)" % (start, T, diff, _rms(ref)))
    assert diff <= TOL * _rms(ref)
    check_argmax_rule(ref[None], np.array([nxt]))
    check_pool_after(pool_after, ref_pool, pool)


def test_prefill_pages_equal_successive_decode_steps_bitwise():
    """Prompt of 40 tokens after 6 cached: the pool and last logits of one
    prefill call equal those of 40 decode_step calls of batch 1."""
    shape = synth.tiny_shape(hidden=128, layers=2, heads=8, kv_heads=2, inter=256, vocab=700)
    start, T = 6, 40
    w, pool, bts, tokens = _inputs(shape, 77, start, T)
    mp = start + T
    model = pkv.upload_model(w, shape.theta, mp)
    logits_a, nxt_a, pool_a, err = prefill_gpu(shape, w, pool, bts, start, tokens, model)
    assert err == 0
    cfg = pkv.make_config(shape, max_pos=mp)
    pool_t = dev(pool)
    kpool = pkv.kv_pool_create(pool_t, shape.kv_heads)
    bt_dev = dev(np.ascontiguousarray(bts[:, None, :], dtype=np.int32))   # [L, 1, max_pages]
    ws = pkv.alloc_workspace(pkv.workspace_bytes(cfg, 1, bts.shape[1]))
    logits = torch.empty((1, shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")
    for t in range(T):
        pkv.decode_step(cfg, model, kpool, bt_dev, dev(np.array([start + t], np.int32)),
                        dev(tokens[t:t + 1]), logits, nxt, ws)
    assert pkv.device_error(ws) == 0
    pool_b = host_u16(pool_t)
    assert np.array_equal(pool_a, pool_b)
    assert np.array_equal(logits_a, logits.cpu().numpy()[0])
    assert nxt_a == int(nxt.cpu()[0])


def test_prefill_llama_shape_4_tokens_after_1006():
    """Llama-3.2-1B-shaped model: 4 prompt tokens at positions 1006..1009
    (crossing a page boundary) after 1006 cached tokens."""
    shape = synth.LLAMA1B
    w = synth.model_weights(shape, 1006)
    _, pool, bts, tokens = _inputs(shape, 1006, 1006, 4, weights=w)
    logits, nxt, pool_after, err = prefill_gpu(shape, w, pool, bts, 1006, tokens)
    assert err == 0
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    ref, ref_tok, ref_pool = oracle.prefill_paged(shape, w, pool, geo, bts, 1006, tokens)
    diff = np.abs(logits - ref).max()
    say("prefill llama 1006+4: max|dlogit| %.3g (RMS %.3g)" % (diff, _rms(ref)))
    assert diff <= TOL * _rms(ref)
    check_argmax_rule(ref[None], np.array([nxt]))
    check_pool_after(pool_after, ref_pool, pool)
