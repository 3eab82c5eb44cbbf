"""GPU parity at head width 128 (the head-width variant of the page
geometry: 16-token pages of 128-wide K and V rows), through the C ABI and
against the oracle, with the bars of the 64-wide tests: attention max-abs
<= 2e-3; kv_append and page placement bit-exact; layer outputs max-abs <=
1e-2 * RMS; logits max-abs <= 1e-2 * RMS and the argmax identical wherever
the oracle's top-2 gap exceeds 1e-3."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_transformer_amd as pkv
import synth
from gpu_util import (appended_mask, assert_layer_out, assert_logits, attention_gpu, attention_oracle,
                      check_argmax_rule,
                      check_pool_after, check_prefill_pool, dev, expected_pool_after, host_u16,
                      layer_gpu, say, step_gpu)

pytestmark = pytest.mark.gpu

D = 128
ATOL = 2e-3
TOL = 1e-2


def _rms(a):
    return float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))


def test_rope_table_d128_matches_oracle():
    theta, max_pos = 5e5, 2100
    c, s = pkv.rope_table(theta, max_pos, head_dim=D)
    c, s = c.cpu().numpy(), s.cpu().numpy()
    assert c.shape == (max_pos, D // 2)
    rc, rs = np.empty_like(c), np.empty_like(s)
    for p in range(max_pos):
        for j in range(D // 2):
            rc[p, j], rs[p, j] = oracle.rope_cos_sin(p, j, D, theta)
    ulp_c = np.abs(c.view(np.int32).astype(np.int64) - rc.view(np.int32).astype(np.int64))
    ulp_s = np.abs(s.view(np.int32).astype(np.int64) - rs.view(np.int32).astype(np.int64))
    assert ulp_c.max() <= 1 and ulp_s.max() <= 1
    assert (ulp_c > 0).sum() + (ulp_s > 0).sum() <= 2


@pytest.mark.parametrize("kv_heads,positions", [(8, [0, 15, 16, 31, 100, 2047]), (2, [5, 17, 18])])
def test_kv_append_d128_bit_exact(kv_heads, positions):
    say("kv_append d128", kv_heads, positions)
    g = np.random.default_rng([5, kv_heads, len(positions)])
    positions = np.asarray(positions, dtype=np.int32)
    pe = synth.page_elems(kv_heads, head_dim=D)
    npages = int(synth.pages_for(positions + 1).sum()) + 7
    pool = synth.random_pool(13, npages, pe)
    bt = synth.block_tables(14, 1, positions + 1, npages)[0]
    k = synth.to_bf16_bits(g.standard_normal((len(positions), kv_heads * D)).astype(np.float32))
    v = synth.to_bf16_bits(g.standard_normal((len(positions), kv_heads * D)).astype(np.float32))
    geo = oracle.PoolGeometry(kv_heads, D)
    want = pool.copy()
    for b, p in enumerate(positions):
        oracle.pool_append(want, geo, bt[b], int(p), k[b], v[b])
    pool_t = dev(pool)
    P = pkv.kv_pool_create(pool_t, kv_heads, head_dim=D)
    pkv.kv_append(P, dev(bt), dev(positions), dev(k), dev(v))
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(pool_t), want)


def test_attention_d128_llama8b_heads_full_size():
    """32/8 heads of width 128, batch 16, lengths U[1,2048], 128 MiB pool of
    64 KiB pages, shuffled tables."""
    w = synth.attention_workload(shape=synth.LLAMA8B)
    say(w["name"], "lens", w["lens"].tolist())
    out, err = attention_gpu(w["pool"], 8, w["q"], w["block_table"], w["lens"], w["scale"])
    ref = attention_oracle(w["pool"], 8, w["q"], w["block_table"], w["lens"], w["scale"])
    assert err == 0
    diff = np.abs(out - ref).max()
    say("d128 full-size max-abs error %.3g" % diff)
    assert diff <= ATOL


def test_attention_d128_large_call():
    """48 sequences x 8 kv heads over a 128-page table take 4 tiles per wave."""
    Hq, Hkv, B = 32, 8, 48
    lens = synth.rng(91, "lens").integers(1, 2049, size=B).astype(np.int32)
    lens[:4] = [1, 256, 257, 2048]
    pe = synth.page_elems(Hkv, head_dim=D)
    npages = int(synth.pages_for(lens).sum())
    pool = synth.random_pool(92, npages, pe)
    bt = synth.block_tables(93, 1, lens, npages, max_pages=128)[0]
    q = synth.bf16_normal(94, "q", (B, Hq, D))
    scale = 1.0 / np.sqrt(D)
    out, err = attention_gpu(pool, Hkv, q, bt, lens, scale)
    ref = attention_oracle(pool, Hkv, q, bt, lens, scale)
    assert err == 0
    assert np.abs(out - ref).max() <= ATOL


@pytest.mark.parametrize("Hq,Hkv,lens,max_pages", [
    (4, 1, [1], 1),
    (4, 2, [0, 1, 2, 15, 16, 17], 4),
    (32, 8, [128, 129, 255, 1000], 70),
    (28, 4, [127, 128, 2049], 140),
    (16, 1, [77, 300], 20),
    (8, 8, [33, 513], 40),
])
def test_attention_d128_small_cases(Hq, Hkv, lens, max_pages):
    say("attention d128", Hq, Hkv, lens, max_pages)
    lens = np.asarray(lens, dtype=np.int32)
    pe = synth.page_elems(Hkv, head_dim=D)
    npages = int(synth.pages_for(lens).sum()) + 5
    pool = synth.random_pool(25, npages, pe)
    bt = synth.block_tables(26, 1, lens, npages, max_pages=max_pages)[0]
    q = synth.bf16_normal(27, "q", (len(lens), Hq, D))
    scale = 1.0 / np.sqrt(D)
    out, err = attention_gpu(pool, Hkv, q, bt, lens, scale)
    ref = attention_oracle(pool, Hkv, q, bt, lens, scale)
    assert err == 0
    assert np.abs(out - ref).max() <= ATOL
    assert np.all(out[lens == 0] == 0)


def test_attention_d128_single_token_is_v0_exactly():
    Hq, Hkv = 8, 2
    pool = synth.random_pool(44, 3, synth.page_elems(Hkv, head_dim=D))
    bt = np.array([[1]], dtype=np.int32)
    q = synth.bf16_normal(45, "q", (1, Hq, D))
    out, _ = attention_gpu(pool, Hkv, q, bt, [1], 0.09)
    _, vc = oracle.pool_gather(pool, oracle.PoolGeometry(Hkv, D), bt[0], 1)
    assert np.array_equal(out[0], np.repeat(vc.reshape(Hkv, D), Hq // Hkv, axis=0))


def _layer_case(shape, batch, seed, pos_hi=300):
    g = synth.rng(seed, "lens")
    positions = g.integers(0, pos_hi, size=batch).astype(np.int32)
    positions[0] = 0
    if batch > 2:
        positions[1:3] = [15, 16]
    wl = synth.decode_workload("d128", shape, seed, positions, layers=1)
    lw = synth.layer_weights(shape, seed, 0, sigma=0.05, norm_sigma=0.3)
    hidden = synth.rng(seed, "hidden").standard_normal((batch, shape.hidden)).astype(np.float32)
    return wl, lw, hidden


def _check_layer(shape, wl, lw, hidden, seqs=None):
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    bt = wl.block_tables[0]
    got, pool_after, err = layer_gpu(shape, lw, hidden, wl.pool, bt, wl.positions)
    assert err == 0
    ref, k_new, v_new = oracle.layer_decode_paged(shape, lw, hidden, wl.pool, geo, bt, wl.positions,
                                                  seqs)
    rows = list(range(len(wl.positions))) if seqs is None else list(seqs)
    assert_layer_out(got[rows], ref[rows], hidden[rows], "layer %s B=%d" % (shape.name, len(wl.positions)))
    want = expected_pool_after(wl.pool, geo, bt, wl.positions, k_new, v_new, seqs)
    if seqs is None:
        check_pool_after(pool_after, want, wl.pool)
    else:
        # every sequence appends; the sampled ones are compared with the
        # oracle, the rest of the pool must be untouched
        B = len(wl.positions)
        every = appended_mask(wl.pool, geo, [bt[b] for b in range(B)], list(wl.positions))
        assert np.array_equal(pool_after[~every], wl.pool[~every])
        sampled = appended_mask(wl.pool, geo, [bt[b] for b in seqs], [wl.positions[b] for b in seqs])
        mixed = np.where(sampled, pool_after, wl.pool)
        check_pool_after(mixed, want, wl.pool, touched=sampled)


@pytest.mark.parametrize("batch,hkv,heads", [(1, 2, 4), (17, 1, 8), (40, 2, 6), (70, 2, 4)])
def test_layer_d128_tiny_shapes(batch, hkv, heads):
    """Batches below 64 take the weight-streaming projections, 70 the tiled
    ones; the QKV weight is packed with the 128-wide head layout."""
    shape = synth.tiny_shape(hidden=256, heads=heads, kv_heads=hkv, inter=512, head_dim=D,
                             name="tiny-d128")
    wl, lw, hidden = _layer_case(shape, batch, 500 + batch)
    _check_layer(shape, wl, lw, hidden)


def test_layer_d128_llama8b_shape_sampled():
    """One Llama-3-8B-shaped layer (hidden 4096, 32/8 heads of 128, SwiGLU
    14336), batch 16, contexts U[1,1024]; four sequences against the oracle
    computed here (every sequence is compared with the stored oracle outputs
    in test_gpu_golden.py)."""
    shape = synth.LLAMA8B
    batch, seed = 16, 1010
    positions = synth.rng(seed, "lens").integers(0, 1024, size=batch).astype(np.int32)
    wl = synth.decode_workload("d128 8b layer", shape, seed, positions, layers=1)
    lw = synth.layer_weights(shape, seed, 0)
    hidden = synth.rng(seed, "hidden").standard_normal((batch, shape.hidden)).astype(np.float32)
    _check_layer(shape, wl, lw, hidden, seqs=[0, 5, 10, 15])


def _check_step(shape, weights, wl, tokens):
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    logits, nxt, _, err = step_gpu(shape, weights, wl.pool, wl.block_tables, wl.positions, tokens,
                                   want_pool=False)
    assert err == 0
    ref, _, _, _ = oracle.decode_step_paged(shape, weights, wl.pool, geo, wl.block_tables,
                                            wl.positions, tokens)
    checked = check_argmax_rule(ref, nxt)
    assert_logits(logits, ref, "step %s B=%d (argmax checked %d)" % (shape.name, len(tokens), checked))


@pytest.mark.parametrize("batch", [5, 64])
def test_step_d128_tiny_model(batch):
    shape = synth.tiny_shape(hidden=256, layers=3, heads=4, kv_heads=2, inter=512, vocab=1000,
                             head_dim=D, name="tiny-d128")
    seed = 600 + batch
    positions = synth.rng(seed, "lens").integers(0, 300, size=batch).astype(np.int32)
    positions[:3] = [0, 15, 16]
    weights = synth.model_weights(shape, seed, sigma=0.05, norm_sigma=0.3)
    wl = synth.decode_workload("tiny-d128-step", shape, seed, positions)
    tokens = synth.rng(seed, "tokens").integers(0, shape.vocab, size=batch)
    _check_step(shape, weights, wl, tokens)


@pytest.mark.parametrize("start,T", [(0, 37), (11, 20)])
def test_prefill_d128_tiny_model(start, T):
    from test_gpu_prefill import prefill_gpu
    shape = synth.tiny_shape(hidden=256, layers=2, heads=4, kv_heads=2, inter=512, vocab=1000,
                             head_dim=D, name="tiny-d128")
    seed = 700 + start
    wl = synth.decode_workload("prefill", shape, seed, [start + T - 1])
    w = synth.model_weights(shape, seed, sigma=0.05, norm_sigma=0.3)
    tokens = synth.rng(seed, "prompt").integers(0, shape.vocab, size=T).astype(np.int32)
    bts = wl.block_tables[:, 0]
    logits, nxt, pool_after, err = prefill_gpu(shape, w, wl.pool, bts, start, tokens)
    assert err == 0
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    ref, _, ref_pool = oracle.prefill_paged(shape, w, wl.pool, geo, bts, start, tokens)
    assert_logits(logits, ref, "prefill d128 start %d T %d" % (start, T))
    check_argmax_rule(ref[None], np.array([nxt]))
    check_prefill_pool(pool_after, wl.pool, geo, bts, start, tokens, shape, w)


def test_head_dim_mismatch_is_rejected():
    """A 64-wide pool with a 128-wide config is refused before any launch."""
    shape = synth.tiny_shape(hidden=256, heads=4, kv_heads=2, inter=512, head_dim=D)
    cfg = pkv.make_config(shape, max_pos=64, layers=1)
    pool_t = torch.zeros(4 * synth.page_elems(2), dtype=torch.int16, device="cuda")
    pool = pkv.kv_pool_create(pool_t, 2)  # 64-wide
    ws = pkv.alloc_workspace(pkv.workspace_bytes(cfg, 1, 4))
    lw = pkv.upload_layer(synth.layer_weights(shape, 3, 0), head_dim=D)
    c, s = pkv.rope_table(shape.theta, 64, head_dim=D)
    bt = dev(np.zeros((1, 4), np.int32))
    h = torch.zeros((1, shape.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError):
        pkv.decoder_layer_decode(cfg, lw, c, s, pool, bt, dev(np.zeros(1, np.int32)), h, ws)
