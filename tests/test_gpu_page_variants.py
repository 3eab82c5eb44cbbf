"""GPU parity of the page-geometry variants of the three-stage engine's
paged KV cache (its section 3.2: fixed-length pages such as 256 tokens,
K and V kept in two caches under one page number), through the C ABI:
pages of 256 tokens, and separate K and V pools, at head widths 64 and 128.

Bars as for 16-token pages: kv_append and placement bit-exact; attention
max-abs <= 2e-3 against the oracle; layers within 1e-2 * RMS with the
appended K/V within one BF16 ulp (or 1e-3 * RMS); logits within
1e-2 * RMS with the argmax rule.  The kernels work on 16-token tiles in the
same order whatever the page size or pool kind, so the same tokens give
bitwise the same attention output in every geometry; that is checked too."""
import numpy as np
import pytest
import torch

import brute
import oracle
import paged_kv_transformer_amd as pkv
import synth
from gpu_util import (appended_mask, assert_layer_out, assert_logits, attention_gpu, attention_oracle,
                      check_argmax_rule, check_pool_after,
                      check_prefill_pool, dev, device_pool, expected_pool_after, layer_gpu, say,
                      step_gpu, whole)

pytestmark = pytest.mark.gpu

ATOL = 2e-3
TOL = 1e-2


def _rms(a):
    return float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))


def _pool(seed, npages, kv_heads, D, PT, split):
    pe = synth.page_elems(kv_heads, head_dim=D, page_tokens=PT)
    if split:
        return synth.random_split_pools(seed, npages, pe)
    return synth.random_pool(seed, npages, pe)


GEOMETRIES = [  # (page tokens, separate K/V pools, head width)
    (256, False, 64), (16, True, 64), (256, True, 64), (256, False, 128), (16, True, 128),
]
IDS = ["pt%d-%s-d%d" % (pt, "split" if sp else "whole", d) for pt, sp, d in GEOMETRIES]


@pytest.mark.parametrize("PT,split,D", GEOMETRIES, ids=IDS)
def test_kv_append_bit_exact(PT, split, D):
    kv_heads = 2
    positions = np.array([0, 15, 16, 255, 256, 300, 1000], dtype=np.int32)
    say("kv_append", PT, split, D)
    g = np.random.default_rng([7, PT, D])
    npages = int(synth.pages_for(positions + 1, PT).sum()) + 3
    pool = _pool(31, npages, kv_heads, D, PT, split)
    bt = synth.block_tables(32, 1, positions + 1, npages, page_tokens=PT)[0]
    k = synth.to_bf16_bits(g.standard_normal((len(positions), kv_heads * D)).astype(np.float32))
    v = synth.to_bf16_bits(g.standard_normal((len(positions), kv_heads * D)).astype(np.float32))
    geo = oracle.PoolGeometry(kv_heads, D, PT)
    want = whole(pool, geo).copy()
    for b, p in enumerate(positions):
        oracle.pool_append(want, geo, bt[b], int(p), k[b], v[b])
    P, read = device_pool(pool, kv_heads, D, PT)
    pkv.kv_append(P, dev(bt), dev(positions), dev(k), dev(v))
    torch.cuda.synchronize()
    assert np.array_equal(read(), want)


@pytest.mark.parametrize("PT,split,D", GEOMETRIES, ids=IDS)
def test_attention_matches_oracle(PT, split, D):
    """Ragged lengths around tile and page edges, one sequence past 2048
    tokens (several splits), GQA group 4."""
    Hq, Hkv = 8, 2
    lens = np.array([0, 1, 15, 16, 17, 255, 256, 257, 700, 2100], dtype=np.int32)
    say("attention", PT, split, D)
    npages = int(synth.pages_for(lens, PT).sum()) + 2
    pool = _pool(41, npages, Hkv, D, PT, split)
    bt = synth.block_tables(42, 1, lens, npages, page_tokens=PT)[0]
    q = synth.bf16_normal(43, "q", (len(lens), Hq, D))
    scale = 1.0 / np.sqrt(D)
    out, err = attention_gpu(pool, Hkv, q, bt, lens, scale, page_tokens=PT)
    ref = attention_oracle(pool, Hkv, q, bt, lens, scale, page_tokens=PT)
    assert err == 0
    diff = np.abs(out - ref).max()
    say("  max-abs %.3g" % diff)
    assert diff <= ATOL
    assert np.all(out[lens == 0] == 0)


@pytest.mark.parametrize("D", [64, 128])
def test_attention_full_size_256_token_pages(D):
    """32/8 heads, batch 16, lengths U[1,2048], 128 MiB pool of 256-token
    pages with shuffled tables."""
    shape = synth.LLAMA1B if D == 64 else synth.LLAMA8B
    w = synth.attention_workload(shape=shape, page_tokens=256)
    say(w["name"])
    out, err = attention_gpu(w["pool"], 8, w["q"], w["block_table"], w["lens"], w["scale"],
                             page_tokens=256)
    ref = attention_oracle(w["pool"], 8, w["q"], w["block_table"], w["lens"], w["scale"],
                           page_tokens=256)
    assert err == 0
    diff = np.abs(out - ref).max()
    say("  max-abs %.3g" % diff)
    assert diff <= ATOL


def test_attention_same_tokens_same_bits_in_every_geometry():
    """The same K/V tokens laid out in 16-token pages, 256-token pages, and
    separate K and V pools of either size give bitwise equal outputs."""
    Hq, Hkv, D = 16, 4, 64
    lens = np.array([1, 200, 1500, 2048, 3000], dtype=np.int32)
    g = np.random.default_rng(51)
    n_max = int(lens.max())
    K = synth.to_bf16_bits(g.standard_normal((len(lens), n_max, Hkv * D)).astype(np.float32))
    V = synth.to_bf16_bits(g.standard_normal((len(lens), n_max, Hkv * D)).astype(np.float32))
    q = synth.bf16_normal(52, "q", (len(lens), Hq, D))
    outs = []
    for PT in (16, 256):
        npages = int(synth.pages_for(lens, PT).sum())
        bt = synth.block_tables(53, 1, lens, npages, page_tokens=PT)[0]
        # the pages through the numpy views of the page layout (16-token
        # tiles: K [page][tile][head][d / 8][slot % 16][d % 8], V
        # [page][tile][head][d][slot % 16])
        pages = np.zeros(npages * 2 * Hkv * PT * D, np.uint16)
        kv, vv = brute.pool_view(pages, Hkv, D, PT)
        for b, n in enumerate(lens):
            t = np.arange(n)
            kv[bt[b][t // PT], (t % PT) // 16, :, :, t % 16, :] = K[b, :n].reshape(n, Hkv, D // 8, 8)
            vv[bt[b][t // PT], (t % PT) // 16, :, :, t % 16] = V[b, :n].reshape(n, Hkv, D)
        geo = oracle.PoolGeometry(Hkv, D, PT)
        for p in (pages, oracle.split_pools(pages, geo)):
            out, err = attention_gpu(p, Hkv, q, bt, lens, 0.125, page_tokens=PT)
            assert err == 0
            outs.append(out)
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def _layer_inputs(shape, batch, seed, PT, split):
    positions = synth.rng(seed, "lens").integers(0, 600, size=batch).astype(np.int32)
    positions[:3] = [0, 255, 256]
    wl = synth.decode_workload("variant", shape, seed, positions, layers=1, page_tokens=PT,
                               with_pool=not split)
    if split:
        wl.pool = synth.random_split_pools(seed, wl.num_pages,
                                           synth.page_elems(shape, page_tokens=PT))
    lw = synth.layer_weights(shape, seed, 0, sigma=0.05, norm_sigma=0.3)
    hidden = synth.rng(seed, "hidden").standard_normal((batch, shape.hidden)).astype(np.float32)
    return wl, lw, hidden


@pytest.mark.parametrize("PT,split,D", GEOMETRIES, ids=IDS)
@pytest.mark.parametrize("batch", [3, 70])
def test_layer_matches_oracle(PT, split, D, batch):
    """Both projection paths (batch 3: weight streaming; 70: tiled)."""
    shape = synth.tiny_shape(hidden=256, heads=4, kv_heads=2, inter=512, head_dim=D, name="tiny-geo")
    wl, lw, hidden = _layer_inputs(shape, batch, 800 + batch + PT + D, PT, split)
    geo = oracle.PoolGeometry(shape.kv_heads, D, PT)
    base = whole(wl.pool, geo)
    bt = wl.block_tables[0]
    got, pool_after, err = layer_gpu(shape, lw, hidden, wl.pool, bt, wl.positions, page_tokens=PT)
    assert err == 0
    ref, k_new, v_new = oracle.layer_decode_paged(shape, lw, hidden, base, geo, bt, wl.positions)
    assert_layer_out(got, ref, hidden, "layer pt%d split %s d%d B=%d" % (PT, split, D, batch))
    want = expected_pool_after(base, geo, bt, wl.positions, k_new, v_new)
    touched = appended_mask(base, geo, [bt[b] for b in range(batch)], wl.positions)
    check_pool_after(pool_after, want, base, touched=touched)


@pytest.mark.parametrize("PT,split", [(256, False), (256, True), (16, True)])
@pytest.mark.parametrize("batch", [5, 64])
def test_step_matches_oracle(PT, split, batch):
    shape = synth.tiny_shape(hidden=128, layers=3, heads=4, kv_heads=2, inter=256, vocab=1000,
                             name="tiny-geo-step")
    seed = 900 + batch + PT
    positions = synth.rng(seed, "lens").integers(0, 600, size=batch).astype(np.int32)
    positions[:3] = [0, 255, 256]
    weights = synth.model_weights(shape, seed, sigma=0.05, norm_sigma=0.3)
    wl = synth.decode_workload("geo-step", shape, seed, positions, page_tokens=PT, with_pool=not split)
    if split:
        wl.pool = synth.random_split_pools(seed, wl.num_pages, synth.page_elems(shape, page_tokens=PT))
    tokens = synth.rng(seed, "tokens").integers(0, shape.vocab, size=batch)
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim, PT)
    base = whole(wl.pool, geo)
    logits, nxt, pool_after, err = step_gpu(shape, weights, wl.pool, wl.block_tables, wl.positions,
                                            tokens, page_tokens=PT)
    assert err == 0
    ref, _, k_new, v_new = oracle.decode_step_paged(shape, weights, base, geo, wl.block_tables,
                                                    wl.positions, tokens)
    checked = check_argmax_rule(ref, nxt)
    assert_logits(logits, ref, "step pt%d split %s B=%d (argmax checked %d)" % (PT, split, batch, checked))
    # placement: every byte the step did not append is unchanged
    rows = [wl.block_tables[l, b] for l in range(shape.layers) for b in range(batch)]
    pos = [wl.positions[b] for l in range(shape.layers) for b in range(batch)]
    touched = appended_mask(base, geo, rows, pos)
    assert np.array_equal(pool_after[~touched], base[~touched])


@pytest.mark.parametrize("PT,split,start,T", [(256, False, 0, 37), (256, True, 250, 20),
                                               (16, True, 11, 20)])
def test_prefill_matches_oracle(PT, split, start, T):
    from test_gpu_prefill import prefill_gpu
    shape = synth.tiny_shape(hidden=128, layers=2, heads=4, kv_heads=2, inter=256, vocab=1000,
                             name="tiny-geo-prefill")
    seed = 950 + start
    wl = synth.decode_workload("prefill", shape, seed, [start + T - 1], page_tokens=PT,
                               with_pool=not split)
    if split:
        wl.pool = synth.random_split_pools(seed, wl.num_pages, synth.page_elems(shape, page_tokens=PT))
    w = synth.model_weights(shape, seed, sigma=0.05, norm_sigma=0.3)
    tokens = synth.rng(seed, "prompt").integers(0, shape.vocab, size=T).astype(np.int32)
    bts = wl.block_tables[:, 0]
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim, PT)
    base = whole(wl.pool, geo)
    logits, nxt, pool_after, err = prefill_gpu(shape, w, wl.pool, bts, start, tokens, page_tokens=PT)
    assert err == 0
    ref, _, ref_pool = oracle.prefill_paged(shape, w, base, geo, bts, start, tokens)
    assert_logits(logits, ref, "prefill pt%d split %s start %d T %d" % (PT, split, start, T))
    check_argmax_rule(ref[None], np.array([nxt]))
    check_prefill_pool(pool_after, base, geo, bts, start, tokens, shape, w)


def test_length_past_a_256_token_table_is_reported():
    Hq, Hkv, D, PT = 4, 1, 64, 256
    pool = _pool(61, 3, Hkv, D, PT, False)
    q = synth.bf16_normal(62, "q", (1, Hq, D))
    bt = np.array([[0, 1]], dtype=np.int32)
    _, err = attention_gpu(pool, Hkv, q, bt, [513], 0.125, page_tokens=PT)  # 513 > 2 * 256
    assert err & pkv.DEVERR_LENGTH
    _, err = attention_gpu(pool, Hkv, q, bt, [512], 0.125, page_tokens=PT)
    assert err == 0
