"""GPU parity of the RoPE table, kv_append and paged_gqa_decode against the
oracle, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_transformer_amd as pkv
import synth
from gpu_util import attention_gpu, attention_oracle, dev, host_u16, say

pytestmark = pytest.mark.gpu

ATOL = 2e-3  # attention outputs, max-abs


@pytest.mark.parametrize("theta,max_pos", [(1e6, 4100), (5e5, 2049), (1e4, 300)])
def test_rope_table_matches_oracle(theta, max_pos):
    say("rope table", theta, max_pos)
    c, s = pkv.rope_table(theta, max_pos)
    c, s = c.cpu().numpy(), s.cpu().numpy()
    rc = np.empty_like(c)
    rs = np.empty_like(s)
    for p in range(max_pos):
        for j in range(32):
            rc[p, j], rs[p, j] = oracle.rope_cos_sin(p, j, 64, theta)
    # both evaluate in double and round to FP32; allow at most one FP32 ulp
    # (a double result within one ulp of a rounding boundary), report any
    ulp_c = np.abs(c.view(np.int32).astype(np.int64) - rc.view(np.int32).astype(np.int64))
    ulp_s = np.abs(s.view(np.int32).astype(np.int64) - rs.view(np.int32).astype(np.int64))
    assert ulp_c.max() <= 1 and ulp_s.max() <= 1
    assert (ulp_c > 0).sum() + (ulp_s > 0).sum() <= 2


@pytest.mark.parametrize("kv_heads,positions", [
    (8, [0, 15, 16, 31, 100, 2047]),
    (2, [5]),
    (2, [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16]),
])
def test_kv_append_bit_exact(kv_heads, positions):
    say("kv_append", kv_heads, positions)
    g = np.random.default_rng([3, kv_heads, len(positions)])
    positions = np.asarray(positions, dtype=np.int32)
    pe = synth.page_elems(kv_heads)
    need = int(synth.pages_for(positions + 1).sum())
    npages = need + 7  # untouched canary pages too
    pool = synth.random_pool(11, npages, pe)
    bt = synth.block_tables(12, 1, positions + 1, npages)[0]
    k = synth.to_bf16_bits(g.standard_normal((len(positions), kv_heads * 64)).astype(np.float32))
    v = synth.to_bf16_bits(g.standard_normal((len(positions), kv_heads * 64)).astype(np.float32))
    geo = oracle.PoolGeometry(kv_heads, 64)
    want = pool.copy()
    for b, p in enumerate(positions):
        oracle.pool_append(want, geo, bt[b], int(p), k[b], v[b])
    pool_t = dev(pool)
    P = pkv.kv_pool_create(pool_t, kv_heads)
    pkv.kv_append(P, dev(bt), dev(positions), dev(k), dev(v))
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(pool_t), want)


def test_kv_append_reports_bad_positions_and_pages():
    """Four sequences: two good ones, one whose position lies past its
    table (PKV_DEVERR_LENGTH) and one whose table entry lies outside the
    pool (PKV_DEVERR_PAGE).  The bad ones write nothing, the good ones are
    written exactly as the oracle's append, and the bits land in the error
    word read by device_error."""
    kv_heads, npages = 2, 12
    pe = synth.page_elems(kv_heads)
    pool = synth.random_pool(21, npages, pe)
    bt = np.array([[3, 4], [5, 6], [7, 8], [9, npages + 40]], dtype=np.int32)
    positions = np.array([17, 2, 32, 20], dtype=np.int32)  # seq 2: page 2 of a 2-page table
    g = np.random.default_rng(22)
    k = synth.to_bf16_bits(g.standard_normal((4, kv_heads * 64)).astype(np.float32))
    v = synth.to_bf16_bits(g.standard_normal((4, kv_heads * 64)).astype(np.float32))
    geo = oracle.PoolGeometry(kv_heads, 64)
    want = pool.copy()
    for b in (0, 1):
        oracle.pool_append(want, geo, bt[b], int(positions[b]), k[b], v[b])
    pool_t = dev(pool)
    P = pkv.kv_pool_create(pool_t, kv_heads)
    ws = pkv.alloc_workspace(256)
    say("kv_append with a bad position and a bad page")
    pkv.kv_append(P, dev(bt), dev(positions), dev(k), dev(v), dev_error=ws)
    err = pkv.device_error(ws)
    assert err == pkv.DEVERR_LENGTH | pkv.DEVERR_PAGE
    assert np.array_equal(host_u16(pool_t), want)
    assert pkv.device_error(ws) == 0  # read and cleared
    # without an error word the same call still skips the bad sequences
    pool_t2 = dev(pool)
    pkv.kv_append(pkv.kv_pool_create(pool_t2, kv_heads), dev(bt), dev(positions), dev(k), dev(v))
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(pool_t2), want)


def test_attention_full_size_llama1b_heads_batch16():
    """Paged GQA attention, 32/8 heads, batch 16, lengths U[1,2048], 128 MiB pool."""
    w = synth.attention_workload()
    say("attention, lens", w["lens"].tolist())
    out, err = attention_gpu(w["pool"], 8, w["q"], w["block_table"], w["lens"], w["scale"])
    ref = attention_oracle(w["pool"], 8, w["q"], w["block_table"], w["lens"], w["scale"])
    assert err == 0
    diff = np.abs(out - ref).max()
    say("attention max-abs error %.3g" % diff)
    assert diff <= ATOL


CASES = [
    # (Hq, Hkv, lens, max_pages)
    (4, 1, [1], 1),
    (4, 2, [0, 1, 2, 15, 16, 17], 4),
    (32, 8, [128, 129, 255, 256, 257, 1000], 70),
    (14, 2, [127, 128, 4097], 300),
    (16, 1, [77, 300], 20),
    (8, 8, [33, 513], 40),
    (6, 2, [16, 160, 161], 11),
    (8, 2, [64, 63, 1], 4),          # a sequence fills its whole block table
    (8, 1, [16384, 5], 1024),        # 128 splits of one sequence in the merge
]


@pytest.mark.parametrize("Hq,Hkv,lens,max_pages", CASES)
def test_attention_small_cases(Hq, Hkv, lens, max_pages):
    _small_case(Hq, Hkv, lens, max_pages, 0.125)


@pytest.mark.parametrize("scale", [0.2, -0.125, 0.0])
def test_attention_other_scales(scale):
    """Any finite scale: a larger one, a negative one (the softmax favours
    the most negative scores) and zero (every token weighs the same)."""
    _small_case(8, 2, [1, 15, 16, 17, 300], 20, scale)


def _small_case(Hq, Hkv, lens, max_pages, scale):
    say("attention", Hq, Hkv, lens, max_pages, scale)
    lens = np.asarray(lens, dtype=np.int32)
    pe = synth.page_elems(Hkv)
    npages = int(synth.pages_for(lens).sum()) + 5
    pool = synth.random_pool(21, npages, pe)
    bt = synth.block_tables(22, 1, lens, npages, max_pages=max_pages)[0]
    q = synth.bf16_normal(23, "q", (len(lens), Hq, 64))
    out, err = attention_gpu(pool, Hkv, q, bt, lens, scale)
    ref = attention_oracle(pool, Hkv, q, bt, lens, scale)
    assert err == 0
    assert np.abs(out - ref).max() <= ATOL
    assert np.all(out[lens == 0] == 0)


def test_attention_large_call_four_tiles_per_wave():
    """64 sequences x 8 kv heads over a 128-page table: enough workgroups
    that the call takes 4 tiles per wave (16 per split); lengths U[1,2048]
    plus the edge lengths of a 16-tile split."""
    Hq, Hkv, B = 32, 8, 64
    lens = synth.rng(81, "lens").integers(1, 2049, size=B).astype(np.int32)
    lens[:8] = [1, 16, 255, 256, 257, 512, 2047, 2048]
    pe = synth.page_elems(Hkv)
    npages = int(synth.pages_for(lens).sum())
    pool = synth.random_pool(82, npages, pe)
    bt = synth.block_tables(83, 1, lens, npages, max_pages=128)[0]
    q = synth.bf16_normal(84, "q", (B, Hq, 64))
    out, err = attention_gpu(pool, Hkv, q, bt, lens, 0.125)
    ref = attention_oracle(pool, Hkv, q, bt, lens, 0.125)
    assert err == 0
    diff = np.abs(out - ref).max()
    say("large call max-abs %.3g" % diff)
    assert diff <= ATOL


def test_attention_paged_equals_contiguous_bitwise():
    Hq, Hkv = 32, 8
    lens = np.array([1, 200, 1500, 2048], dtype=np.int32)
    pe = synth.page_elems(Hkv)
    need = synth.pages_for(lens)
    npages = int(need.sum())
    logical = synth.random_pool(31, npages, pe)
    ident_bt = np.full((4, 128), -1, np.int32)
    start = 0
    for b, k in enumerate(need):
        ident_bt[b, :k] = np.arange(start, start + k)
        start += k
    perm = np.random.default_rng(32).permutation(npages)
    shuffled = np.empty_like(logical)
    perm_bt = np.full_like(ident_bt, -1)
    for b, k in enumerate(need):
        for lp in range(k):
            src = ident_bt[b, lp]
            dst = perm[src]
            shuffled[dst * pe:(dst + 1) * pe] = logical[src * pe:(src + 1) * pe]
            perm_bt[b, lp] = dst
    q = synth.bf16_normal(33, "q", (4, Hq, 64))
    a, _ = attention_gpu(logical, Hkv, q, ident_bt, lens, 0.125)
    b, _ = attention_gpu(shuffled, Hkv, q, perm_bt, lens, 0.125)
    assert np.array_equal(a, b)


def test_attention_single_token_is_v0_exactly():
    Hq, Hkv = 8, 2
    pool = synth.random_pool(41, 3, synth.page_elems(Hkv))
    bt = np.array([[2]], dtype=np.int32)
    q = synth.bf16_normal(42, "q", (1, Hq, 64))
    out, _ = attention_gpu(pool, Hkv, q, bt, [1], 0.125)
    geo = oracle.PoolGeometry(Hkv, 64)
    _, vc = oracle.pool_gather(pool, geo, bt[0], 1)
    assert np.array_equal(out[0], np.repeat(vc.reshape(Hkv, 64), Hq // Hkv, axis=0))


def test_attention_zero_query_gives_mean_of_v():
    Hq, Hkv, n = 4, 1, 300
    pool = synth.random_pool(43, 19, synth.page_elems(Hkv))
    bt = np.arange(19, dtype=np.int32)[None]
    q = np.zeros((1, Hq, 64), np.uint16)
    out, _ = attention_gpu(pool, Hkv, q, bt, [n], 0.125)
    _, vc = oracle.pool_gather(pool, oracle.PoolGeometry(Hkv, 64), bt[0], n)
    np.testing.assert_allclose(out[0], np.repeat(vc.astype(np.float64).mean(0)[None], Hq, 0), atol=1e-5)


def test_attention_ignores_nan_in_unused_slots():
    Hq, Hkv = 8, 2
    lens = np.array([17, 40], dtype=np.int32)
    pe = synth.page_elems(Hkv)
    pool = synth.random_pool(51, 8, pe)
    bt = np.array([[0, 1, -1], [2, 3, 4]], dtype=np.int32)
    q = synth.bf16_normal(52, "q", (2, Hq, 64))
    clean, _ = attention_gpu(pool, Hkv, q, bt, lens, 0.125)
    poisoned = np.full_like(pool, 0x7FC0)  # BF16 quiet NaN everywhere ...
    geo = oracle.PoolGeometry(Hkv, 64)
    for b, n in enumerate(lens):            # ... except the live tokens
        kc, vc = oracle.pool_gather(pool, geo, bt[b], int(n))
        for t in range(n):
            oracle.pool_append(poisoned, geo, bt[b], t, oracle.f32_to_bf16(kc[t]),
                               oracle.f32_to_bf16(vc[t]))
    dirty, _ = attention_gpu(poisoned, Hkv, q, bt, lens, 0.125)
    assert np.array_equal(clean, dirty)


def test_attention_workspace_reuse_is_deterministic():
    w = synth.attention_workload(batch=4)
    ws = pkv.alloc_workspace(pkv.attention_workspace_bytes(32, 8, 4, 128))
    a, _ = attention_gpu(w["pool"], 8, w["q"], w["block_table"], w["lens"], 0.125, ws=ws)
    b, _ = attention_gpu(w["pool"], 8, w["q"], w["block_table"], w["lens"], 0.125, ws=ws)
    assert np.array_equal(a, b)


def test_attention_device_errors_are_reported():
    Hq, Hkv = 4, 1
    pool = synth.random_pool(61, 4, synth.page_elems(Hkv))
    q = synth.bf16_normal(62, "q", (2, Hq, 64))
    bt = np.array([[0, 99], [1, 2]], dtype=np.int32)  # 99 is outside the pool
    _, err = attention_gpu(pool, Hkv, q, bt, [20, 5], 0.125)
    assert err & pkv.DEVERR_PAGE
    _, err = attention_gpu(pool, Hkv, q, bt, [20, 33], 0.125)  # 33 > 2 pages * 16
    assert err & pkv.DEVERR_LENGTH
