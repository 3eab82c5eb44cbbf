"""GPU parity of prefill (one sequence's prompt into the pool) through the
C ABI.  Prefill's projections take their activations as BF16 hi + lo halves
(~16 significant bits, as the decode projections do), so its bars are the
decode path's:
  * the last token's logits: max-abs <= 4e-4 for the full-size model,
    <= 5e-3 * RMS(logits) for the small test models (gpu_util's bars), and
    the argmax identical wherever the oracle's top-2 gap exceeds 1e-3;
  * every layer's K/V of every prompt token within one BF16 ulp or 1e-3 *
    RMS of the oracle's, the oracle being fed the GPU's own K/V of the
    earlier positions (teacher forcing: a token's K/V at a later layer then
    depend on earlier tokens only through values both sides share, so a
    BF16 rounding that fell on the other neighbour in an earlier token
    cannot spread); every other pool byte untouched;
  * placement, bitwise: the pool after prefill equals the original pool with
    the prefill's own K/V values written by kv_append at start_pos + t.
The 512-token prompt that bench.py times is compared with stored oracle
outputs in test_gpu_golden.py."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_transformer_amd as pkv
import synth
from gpu_util import assert_logits, check_argmax_rule, check_prefill_pool, dev, device_pool, host_u16, prompt_kv_bits, say

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _rms(a):
    return float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))


def _inputs(shape, seed, start, T, weights=None):
    wl = synth.decode_workload("prefill", shape, seed, [start + T - 1])
    w = weights or synth.model_weights(shape, seed, sigma=0.05, norm_sigma=0.3)
    tokens = synth.rng(seed, "prompt").integers(0, shape.vocab, size=T).astype(np.int32)
    return w, wl.pool, wl.block_tables[:, 0], tokens


def prefill_gpu(shape, weights, pool_np, bts, start, tokens, model=None, page_tokens=16):
    """prefill through the C ABI; returns (logits, next token, pool after as
    whole pages, device error bits).  pool_np: whole pages or a (K, V) pair."""
    T = len(tokens)
    mp = start + T
    cfg = pkv.make_config(shape, max_pos=mp)
    model = model or pkv.upload_model(weights, shape.theta, mp, head_dim=shape.head_dim)
    pool, read_pool = device_pool(pool_np, shape.kv_heads, shape.head_dim, page_tokens)
    bts = np.ascontiguousarray(bts, dtype=np.int32)
    ws = pkv.alloc_workspace(pkv.prefill_workspace_bytes(cfg, T, bts.shape[1]))
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    nxt = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    pkv.prefill(cfg, model, pool, dev(bts), start, dev(tokens), logits, nxt, ws)
    err = pkv.device_error(ws)
    return logits.cpu().numpy(), int(nxt.cpu()[0]), read_pool(), err


def _oracle_check(shape, w, pool, bts, start, tokens, logits, nxt, pool_after, label, full_size=False):
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    ref, ref_tok, _ = oracle.prefill_paged(shape, w, pool, geo, bts, start, tokens)
    kv_err = check_prefill_pool(pool_after, pool, geo, bts, start, tokens, shape, w)
    say("prefill %s start %d T %d: teacher-forced max|dKV| per layer %s" % (
        label, start, len(tokens), ["%.3g" % e for e in kv_err]))
    assert_logits(logits, ref, "prefill %s start %d T %d" % (label, start, len(tokens)), full_size)
    check_argmax_rule(ref[None], np.array([nxt]))


@pytest.mark.parametrize("start,T", [(0, 37), (11, 20), (5, 1), (0, 16), (13, 3)])
def test_prefill_tiny_model_matches_oracle(start, T):
    shape = synth.tiny_shape(hidden=128, layers=3, heads=4, kv_heads=2, inter=256, vocab=1000)
    w, pool, bts, tokens = _inputs(shape, 40 + start, start, T)
    logits, nxt, pool_after, err = prefill_gpu(shape, w, pool, bts, start, tokens)
    assert err == 0
    _oracle_check(shape, w, pool, bts, start, tokens, logits, nxt, pool_after, "tiny")


@pytest.mark.parametrize("head_dim,T", [(64, 40), (128, 23)])
def test_prefill_split_qkv_matches_oracle(head_dim, T):
    """Hidden 512 with a short prompt: the QKV projection splits K into
    partial sums and a second kernel finishes RoPE, q and the K/V append."""
    shape = synth.tiny_shape(hidden=512, layers=2, heads=4, kv_heads=2, inter=512, vocab=700,
                             head_dim=head_dim)
    start = 3
    w, pool, bts, tokens = _inputs(shape, 60 + head_dim, start, T)
    logits, nxt, pool_after, err = prefill_gpu(shape, w, pool, bts, start, tokens)
    assert err == 0
    _oracle_check(shape, w, pool, bts, start, tokens, logits, nxt, pool_after, "split-qkv")


@pytest.mark.parametrize("heads,kv_heads", [(2, 2), (14, 2), (16, 1)])
def test_prefill_group_sizes(heads, kv_heads):
    """GQA groups of 1, 7 and 16 heads: 16, 2 and 1 tokens per wave."""
    shape = synth.tiny_shape(hidden=128, layers=2, heads=heads, kv_heads=kv_heads, inter=256,
                             vocab=500)
    start, T = 9, 23
    w, pool, bts, tokens = _inputs(shape, 60 + heads, start, T)
    logits, nxt, pool_after, err = prefill_gpu(shape, w, pool, bts, start, tokens)
    assert err == 0
    _oracle_check(shape, w, pool, bts, start, tokens, logits, nxt, pool_after, "G=%d" % (heads // kv_heads))


@pytest.mark.parametrize("start,T", [(3, 250), (0, 400)])
def test_prefill_wide_tiles_match_oracle(start, T):
    """Prompts through an 8192-wide MLP.  250 tokens: the gate/up projection
    takes the 128 x 128 tile (128 row tiles x 2 token tiles, the second
    ragged); 400 tokens: the 256 x 128 tile (64 x 4, the last ragged); the
    other projections the smaller tiles."""
    shape = synth.tiny_shape(hidden=256, layers=1, heads=4, kv_heads=2, inter=8192, vocab=1000)
    w, pool, bts, tokens = _inputs(shape, 91 + T, start, T)
    logits, nxt, pool_after, err = prefill_gpu(shape, w, pool, bts, start, tokens)
    assert err == 0
    _oracle_check(shape, w, pool, bts, start, tokens, logits, nxt, pool_after, "wide")


def _prompt_kv(pool, geo, bts, start, T):
    """BF16 bits of the K and V the pool holds at positions start .. start+T-1,
    per layer: [L][T][Hkv][D] each."""
    ks, vs = [], []
    for l in range(bts.shape[0]):
        k, v = prompt_kv_bits(pool, geo, bts[l], start, T)
        ks.append(k.reshape(T, geo.kv_heads, geo.head_dim))
        vs.append(v.reshape(T, geo.kv_heads, geo.head_dim))
    return ks, vs


def test_prefill_placement_equals_kv_append_bitwise():
    """Prompt of 40 tokens after 6 cached: the pool after prefill is the
    original pool with the prompt's K/V written by kv_append."""
    shape = synth.tiny_shape(hidden=128, layers=2, heads=8, kv_heads=2, inter=256, vocab=700)
    start, T = 6, 40
    w, pool, bts, tokens = _inputs(shape, 77, start, T)
    _, _, pool_a, err = prefill_gpu(shape, w, pool, bts, start, tokens)
    assert err == 0
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    ks, vs = _prompt_kv(pool_a, geo, bts, start, T)
    pool_t = dev(pool)
    kpool = pkv.kv_pool_create(pool_t, shape.kv_heads, head_dim=shape.head_dim)
    pos = dev(np.arange(start, start + T, dtype=np.int32))
    for l in range(shape.layers):
        table = dev(np.ascontiguousarray(np.repeat(bts[l][None], T, axis=0), dtype=np.int32))
        pkv.kv_append(kpool, table, pos, dev(ks[l]), dev(vs[l]))
    torch.cuda.synchronize()
    assert np.array_equal(pool_a, host_u16(pool_t))


def test_prefill_llama_shape_4_tokens_after_1006():
    """Llama-3.2-1B-shaped model: 4 prompt tokens at positions 1006..1009
    (crossing a page boundary) after 1006 cached tokens."""
    shape = synth.LLAMA1B
    w = synth.model_weights(shape, 1006)
    _, pool, bts, tokens = _inputs(shape, 1006, 1006, 4, weights=w)
    logits, nxt, pool_after, err = prefill_gpu(shape, w, pool, bts, 1006, tokens)
    assert err == 0
    _oracle_check(shape, w, pool, bts, 1006, tokens, logits, nxt, pool_after, "llama", full_size=True)
