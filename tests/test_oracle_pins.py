"""Pins of the CPU oracle to facts other than itself (CPU only).

Each test names the plausible mistake it is there to catch.
"""
import math

import numpy as np
import pytest
import torch

import brute
import oracle
import synth


def _rng(*k):
    return np.random.default_rng([77, *k])


# ------------------------------------------------------------------ BF16 ---

@pytest.mark.parametrize("value,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                 # exact tie, kept value even -> stays
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # exact tie, kept value odd -> up to even
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),    # just above the tie -> up
    (1.0 + 2.0 ** -8 - 2.0 ** -20, 0x3F80),    # just below the tie -> down
    (-1.5, 0xBFC0),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (float(np.finfo(np.float32).max), 0x7F80),   # FP32 max rounds past the largest BF16 -> inf
    (3.3895313892515355e38, 0x7F7F),          # the largest finite BF16 is kept
    (2.0 ** -133, 0x0001),                     # subnormal kept exactly
])
def test_bf16_round_cases(value, bits):
    # catches: truncation instead of rounding, ties away from zero, lost carry
    assert int(oracle.f32_to_bf16(np.array([value], dtype=np.float32))[0]) == bits


def test_bf16_nan_stays_nan():
    h = oracle.f32_to_bf16(np.array([np.nan, -np.nan], dtype=np.float32))
    assert np.all(np.isnan(oracle.bf16_to_f32(h)))


def test_bf16_matches_torch_rne():
    # library routine: torch's float32 -> bfloat16 conversion is round-to-nearest-even
    g = _rng(1)
    x = np.concatenate([g.standard_normal(200000).astype(np.float32) * s
                        for s in (1e-30, 1e-3, 1.0, 1e3, 1e30)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(x), ref)
    assert np.array_equal(oracle.bf16_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(
        torch.bfloat16).to(torch.float32).numpy())


# --------------------------------------------------------------- RMSNorm ---

def test_rmsnorm_unit_weight_closed_form():
    # catches: eps outside the root, sum instead of mean, missing sqrt
    g = _rng(2)
    for H, eps in ((896, 1e-6), (2048, 1e-5), (64, 0.5)):
        x = g.standard_normal(H).astype(np.float32) * 3
        w = np.full(H, 0x3F80, dtype=np.uint16)
        y = oracle.rmsnorm(x, w, eps).astype(np.float64)
        ms = np.mean(x.astype(np.float64) ** 2)
        assert math.isclose(np.sqrt(np.mean(y * y)), math.sqrt(ms / (ms + eps)), rel_tol=2e-6)


def test_rmsnorm_scale_invariant_without_eps():
    g = _rng(3)
    x = g.standard_normal(512).astype(np.float32)
    w = synth.to_bf16_bits(g.standard_normal(512).astype(np.float32))
    y1 = oracle.rmsnorm(x, w, 0.0)
    y2 = oracle.rmsnorm(np.float32(7.5) * x, w, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=2e-6, atol=1e-7)


def test_rmsnorm_weight_is_applied():
    # catches: a dropped or misindexed weight (y / w must have RMS ~ 1)
    g = _rng(4)
    x = g.standard_normal(1024).astype(np.float32)
    wf = (g.uniform(0.5, 2.0, 1024) * np.sign(g.standard_normal(1024))).astype(np.float32)
    w = synth.to_bf16_bits(wf)
    y = oracle.rmsnorm(x, w, 1e-6).astype(np.float64) / oracle.bf16_to_f32(w)
    assert math.isclose(np.sqrt(np.mean(y * y)), 1.0, rel_tol=1e-5)
    np.testing.assert_allclose(y, x / np.sqrt(np.mean(x.astype(np.float64) ** 2) + 1e-6), rtol=1e-5)


# ---------------------------------------------------------------- matvec ---

def test_matvec_matches_float64_matmul_nonsquare():
    # catches: a transposed operand (non-square), wrong row stride
    g = _rng(5)
    W = synth.to_bf16_bits(g.standard_normal((37, 53)).astype(np.float32))
    x = g.standard_normal(53).astype(np.float32)
    ref = oracle.bf16_to_f32(W).astype(np.float64) @ x.astype(np.float64)
    np.testing.assert_allclose(oracle.matvec(W, x), ref, rtol=1e-5, atol=1e-5)


# ------------------------------------------------------------------ RoPE ---

def test_rope_identity_at_position_zero():
    g = _rng(6)
    u = g.standard_normal((5, 64)).astype(np.float32)
    assert np.array_equal(oracle.rope(u, 0, 1e6), u)


def test_rope_keeps_pair_norms():
    g = _rng(7)
    u = g.standard_normal((3, 64)).astype(np.float32)
    for pos in (1, 17, 1023, 4096):
        r = oracle.rope(u, pos, 5e5).astype(np.float64)
        n0 = u[:, :32].astype(np.float64) ** 2 + u[:, 32:].astype(np.float64) ** 2
        n1 = r[:, :32] ** 2 + r[:, 32:] ** 2
        np.testing.assert_allclose(n1, n0, rtol=1e-6, atol=1e-9)


def test_rope_relative_position():
    # <R_m q, R_n k> = <R_(m-n) q, k>: catches a frequency mixed up between q and k
    g = _rng(8)
    q = g.standard_normal((1, 64)).astype(np.float32)
    k = g.standard_normal((1, 64)).astype(np.float32)
    for m, n in ((10, 3), (900, 100), (2047, 2000)):
        lhs = float(oracle.rope(q, m, 1e4)[0].astype(np.float64) @ oracle.rope(k, n, 1e4)[0])
        rhs = float(oracle.rope(q, m - n, 1e4)[0].astype(np.float64) @ k[0])
        assert math.isclose(lhs, rhs, rel_tol=1e-5, abs_tol=1e-5)


def test_rope_pair_zero_turns_by_position_radians():
    # theta_0 = 1: pair 0 turns by exactly p radians (cos/sin of p rounded to FP32)
    u = np.zeros((1, 64), dtype=np.float32)
    u[0, 0] = 1.0
    for p in (1, 5, 127, 4096):
        r = oracle.rope(u, p, 1e6)
        assert r[0, 0] == np.float32(math.cos(p)) and r[0, 32] == np.float32(math.sin(p))


@pytest.mark.parametrize("D", [64, 128])
def test_rope_frequencies_and_rotate_half_pairing(D):
    # catches: adjacent pairing (2j, 2j+1), wrong exponent -2j/D, theta ignored
    theta = 1e6
    for j in (0, 1, 7, D // 2 - 1):
        u = np.zeros((1, D), dtype=np.float32)
        u[0, j] = 1.0
        r = oracle.rope(u, 1, theta)[0]
        nz = set(np.flatnonzero(r).tolist())
        assert nz <= {j, j + D // 2}
        ang = math.atan2(float(r[j + D // 2]), float(r[j]))
        assert math.isclose(ang, theta ** (-2.0 * j / D), rel_tol=1e-6, abs_tol=1e-12)


def test_rope_cos_sin_rounding():
    c, s = oracle.rope_cos_sin(1000, 3, 64, 5e5)
    ang = 1000 * 5e5 ** (-6.0 / 64)
    assert c == np.float32(math.cos(ang)) and s == np.float32(math.sin(ang))


# ------------------------------------------------------- SiLU / argmax ---

def test_silu_closed_form():
    assert oracle.silu(0.0) == 0.0
    for z in (-20.0, -3.0, -0.5, 0.25, 1.0, 6.0, 40.0):
        assert math.isclose(float(oracle.silu(z)), z / (1 + math.exp(-z)), rel_tol=1e-6, abs_tol=1e-12)


def test_argmax_first_of_ties_and_numpy():
    v = np.array([0.5, 2.0, -1.0, 2.0, 2.0], dtype=np.float32)
    assert oracle.argmax(v) == 1
    g = _rng(9)
    for _ in range(20):
        v = g.standard_normal(1000).astype(np.float32)
        assert oracle.argmax(v) == int(np.argmax(v))


# ------------------------------------------------------------- attention ---

def _kv(g, n, hkv, D):
    K = oracle.bf16_to_f32(synth.to_bf16_bits(g.standard_normal((n, hkv * D)).astype(np.float32)))
    V = oracle.bf16_to_f32(synth.to_bf16_bits(g.standard_normal((n, hkv * D)).astype(np.float32)))
    return K, V


def test_attention_single_token_is_v0():
    g = _rng(10)
    K, V = _kv(g, 1, 2, 64)
    q = g.standard_normal((8, 64)).astype(np.float32)
    out = oracle.attention(q, K, V, 2, 0.125)
    assert np.array_equal(out, np.repeat(V.reshape(2, 64), 4, axis=0))


def test_attention_constant_scores_give_mean_of_v():
    g = _rng(11)
    for n in (2, 17, 300):
        K, V = _kv(g, n, 2, 64)
        out = oracle.attention(np.zeros((4, 64), np.float32), K, V, 2, 0.125)
        mean = V.astype(np.float64).reshape(n, 2, 64).mean(axis=0)
        np.testing.assert_allclose(out, np.repeat(mean, 2, axis=0), rtol=1e-5, atol=1e-6)


def test_attention_dominant_key():
    g = _rng(12)
    n, t_star = 50, 31
    K, V = _kv(g, n, 1, 64)
    q = g.standard_normal((1, 64)).astype(np.float32)
    K[t_star] = q[0] * 10
    out = oracle.attention(q, K, V, 1, 0.125)
    np.testing.assert_allclose(out[0], V[t_star], atol=1e-5)


def test_attention_two_token_closed_form_fixes_scale():
    # s0 = 0, s1 = ln 3 after scaling by 1/8  ->  o = (V0 + 3 V1) / 4
    # catches: a missing or wrong scale (1/D, none), exponent of the wrong sign
    D = 64
    q = np.zeros((1, D), np.float32)
    q[0, 0] = 1.0
    K = np.zeros((2, D), np.float32)
    K[1, 0] = np.float32(8.0 * math.log(3.0))
    g = _rng(13)
    V = g.standard_normal((2, D)).astype(np.float32)
    out = oracle.attention(q, K, V, 1, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(out[0], (V[0] + 3 * V[1]) / 4, rtol=1e-5, atol=1e-6)


def test_attention_gqa_equals_mha_over_repeated_kv():
    # catches: q head h mapped to kv head h % Hkv instead of h / G
    g = _rng(14)
    hq, hkv, D, n = 8, 2, 64, 40
    K, V = _kv(g, n, hkv, D)
    q = g.standard_normal((hq, D)).astype(np.float32)
    rep = lambda A: np.repeat(A.reshape(n, hkv, D), hq // hkv, axis=1).reshape(n, hq * D)
    a = oracle.attention(q, K, V, hkv, 0.125)
    b = oracle.attention(q, rep(K), rep(V), hq, 0.125)
    assert np.array_equal(a, b)


def test_attention_matches_materialised_float64():
    g = _rng(15)
    for hq, hkv, n in ((4, 2, 1), (14, 2, 128), (32, 8, 333)):
        K, V = _kv(g, n, hkv, 64)
        q = g.standard_normal((hq, 64)).astype(np.float32)
        ref = brute.softmax_attention(q.astype(np.float64), K.reshape(n, hkv, 64).astype(np.float64),
                                      V.reshape(n, hkv, 64).astype(np.float64), 0.125)
        np.testing.assert_allclose(oracle.attention(q, K, V, hkv, 0.125), ref, rtol=1e-4, atol=2e-6)


def test_attention_empty_sequence_gives_zeros():
    out = oracle.attention(np.ones((4, 64), np.float32), np.zeros((0, 128), np.float32),
                           np.zeros((0, 128), np.float32), 2, 0.125)
    assert np.array_equal(out, np.zeros((4, 64), np.float32))


def test_online_softmax_equals_two_pass_float64():
    # the reorganisation the GPU path relies on (block-wise running max / sum)
    g = _rng(16)
    for n, block in ((1, 16), (100, 16), (2048, 128), (777, 7)):
        q = g.standard_normal(64)
        K = g.standard_normal((n, 64)) * 3
        V = g.standard_normal((n, 64))
        two = brute.softmax_attention(q[None], K[:, None], V[:, None], 0.125)[0]
        np.testing.assert_allclose(brute.online_softmax_attention(q, K, V, 0.125, block), two,
                                   rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- paging ---

def test_pool_gather_matches_reshaped_view():
    g = _rng(17)
    geo = oracle.PoolGeometry(kv_heads=2, head_dim=64)
    npages = 20
    pool = synth.to_bf16_bits(g.standard_normal(npages * geo.page_elems).astype(np.float32))
    bt = g.permutation(npages)[:5].astype(np.int32)
    n = 70
    kc, vc = oracle.pool_gather(pool, geo, bt, n)
    K, V = brute.gather(pool, 2, 64, bt, n)
    assert np.array_equal(kc, K.reshape(n, 128).astype(np.float32))
    assert np.array_equal(vc, V.reshape(n, 128).astype(np.float32))


@pytest.mark.parametrize("pos,D", [(0, 64), (15, 64), (16, 64), (31, 64), (77, 64), (0, 128),
                                   (17, 128), (95, 128)])
def test_pool_append_matches_reshaped_view(pos, D):
    g = _rng(18, pos)
    geo = oracle.PoolGeometry(kv_heads=8, head_dim=D)
    npages = 12
    pool = synth.to_bf16_bits(g.standard_normal(npages * geo.page_elems).astype(np.float32))
    bt = g.permutation(npages)[:6].astype(np.int32)
    k = synth.to_bf16_bits(g.standard_normal(8 * D).astype(np.float32))
    v = synth.to_bf16_bits(g.standard_normal(8 * D).astype(np.float32))
    want = pool.copy()
    kv, vv = brute.pool_view(want, 8, D)
    brute.k_of(kv, bt[pos // 16], pos % 16)[...] = k.reshape(8, D // 8, 8)
    vv[bt[pos // 16], 0, :, :, pos % 16] = v.reshape(8, D)
    got = pool.copy()
    oracle.pool_append(got, geo, bt, pos, k, v)
    assert np.array_equal(got, want)
    assert np.count_nonzero(got != pool) <= 2 * 8 * D


@pytest.mark.parametrize("T,D", [(16, 64), (256, 64), (256, 128)])
def test_pool_gather_any_page_size_matches_reshaped_view(T, D):
    g = _rng(20, T, D)
    geo = oracle.PoolGeometry(kv_heads=2, head_dim=D, page_tokens=T)
    npages = 6
    pool = synth.to_bf16_bits(g.standard_normal(npages * geo.page_elems).astype(np.float32))
    bt = g.permutation(npages)[:4].astype(np.int32)
    n = 3 * T + 5
    kc, vc = oracle.pool_gather(pool, geo, bt, n)
    K, V = brute.gather(pool, 2, D, bt, n, page_tokens=T)
    assert np.array_equal(kc, K.reshape(n, 2 * D).astype(np.float32))
    assert np.array_equal(vc, V.reshape(n, 2 * D).astype(np.float32))
    # append at a slot in the middle of a 256-token page
    pos = n - 3
    k = synth.to_bf16_bits(g.standard_normal(2 * D).astype(np.float32))
    v = synth.to_bf16_bits(g.standard_normal(2 * D).astype(np.float32))
    got = pool.copy()
    oracle.pool_append(got, geo, bt, pos, k, v)
    want = pool.copy()
    kv, vv = brute.pool_view(want, 2, D, T)
    brute.k_of(kv, bt[pos // T], pos % T)[...] = k.reshape(2, D // 8, 8)
    vv[bt[pos // T], (pos % T) // 16, :, :, pos % 16] = v.reshape(2, D)
    assert np.array_equal(got, want)


def test_split_pools_are_the_page_blocks():
    g = _rng(21)
    geo = oracle.PoolGeometry(kv_heads=2, head_dim=64, page_tokens=256)
    pool = synth.to_bf16_bits(g.standard_normal(3 * geo.page_elems).astype(np.float32))
    kp, vp = oracle.split_pools(pool, geo)
    kv, vv = brute.pool_view(pool, 2, 64, 256)
    assert np.array_equal(kp, kv.reshape(-1)) and np.array_equal(vp, vv.reshape(-1))
    assert np.array_equal(oracle.whole_pool(kp, vp, geo), pool)


def test_paged_equals_contiguous():
    # identity table over a contiguous copy vs a random permutation of pages
    g = _rng(19)
    geo = oracle.PoolGeometry(kv_heads=2, head_dim=64)
    n, npages = 100, 16
    logical = synth.to_bf16_bits(g.standard_normal(7 * geo.page_elems).astype(np.float32))
    ident = np.zeros(npages * geo.page_elems, np.uint16)
    ident[:logical.size] = logical
    perm = g.permutation(npages)[:7].astype(np.int32)
    shuffled = np.zeros_like(ident)
    for lp, pp in enumerate(perm):
        shuffled[pp * geo.page_elems:(pp + 1) * geo.page_elems] = \
            logical[lp * geo.page_elems:(lp + 1) * geo.page_elems]
    q = g.standard_normal((1, 4, 64)).astype(np.float32)
    a = oracle.paged_attention(ident, geo, q, np.arange(7, dtype=np.int32)[None], [n], 0.125)
    b = oracle.paged_attention(shuffled, geo, q, perm[None], [n], 0.125)
    assert np.array_equal(a, b)


# --------------------------------------------------------- layer / step ---

TINY = synth.tiny_shape(hidden=16, layers=2, heads=4, kv_heads=2, inter=32, vocab=50,
                        head_dim=8, eps=1e-5, theta=1e4, name="brute-tiny")


def _tiny_inputs(seed, positions, shape=TINY):
    wts = synth.model_weights(shape, seed, sigma=0.3, norm_sigma=0.3)
    wl = synth.decode_workload("tiny", shape, seed, positions, num_pages=40)
    tokens = synth.rng(seed, "tokens").integers(0, shape.vocab, size=len(positions))
    return shape, wts, wl, tokens


TINY128 = synth.tiny_shape(hidden=32, layers=2, heads=4, kv_heads=2, inter=64, vocab=50,
                           head_dim=128, eps=1e-5, theta=1e4, name="brute-tiny-d128")


@pytest.mark.parametrize("shape", [TINY, TINY128], ids=["d8", "d128"])
def test_layer_matches_float64_brute_force(shape):
    _, wts, wl, _ = _tiny_inputs(5, [0, 15, 16, 39], shape)
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    hidden = synth.rng(5, "hidden").standard_normal((4, shape.hidden)).astype(np.float32)
    out, kn, vn = oracle.layer_decode_paged(shape, wts["layers"][0], hidden, wl.pool, geo,
                                            wl.block_tables[0], wl.positions)
    for b, p in enumerate(wl.positions):
        K, V = brute.gather(wl.pool, shape.kv_heads, shape.head_dim, wl.block_tables[0, b], int(p))
        ref, k, v = brute.layer(shape, wts["layers"][0], hidden[b].astype(np.float64), K, V, int(p))
        np.testing.assert_allclose(out[b], ref, rtol=1e-5, atol=1e-5)
        # appended K/V: one BF16 ulp at most (FP32 vs float64 pre-rounding values)
        np.testing.assert_allclose(oracle.bf16_to_f32(kn[b]), k.reshape(-1), rtol=2 ** -7, atol=1e-6)
        np.testing.assert_allclose(oracle.bf16_to_f32(vn[b]), v.reshape(-1), rtol=2 ** -7, atol=1e-6)


def test_step_matches_float64_brute_force():
    shape, wts, wl, tokens = _tiny_inputs(6, [3, 20, 39])
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    logits, nxt, _, _ = oracle.decode_step_paged(shape, wts, wl.pool, geo, wl.block_tables,
                                                 wl.positions, tokens)
    ref_logits, ref_tok = brute.decode_step(shape, wts, wl.pool, wl.block_tables, wl.positions, tokens)
    np.testing.assert_allclose(logits, ref_logits, rtol=1e-5, atol=1e-5)
    for b in range(len(tokens)):
        top2 = np.sort(ref_logits[b])[-2:]
        if top2[1] - top2[0] > 1e-4:
            assert nxt[b] == ref_tok[b]


def test_layer_with_zero_weights_is_identity():
    shape = TINY
    z = {k: np.zeros_like(v) for k, v in synth.layer_weights(shape, 1, 0).items()}
    x = np.linspace(-2, 2, shape.hidden).astype(np.float32)
    kvd = shape.kv_heads * shape.head_dim
    kc = np.zeros((4, kvd), np.float32)
    vc = np.zeros((4, kvd), np.float32)
    out, _, _ = oracle.layer_decode(shape, z, x, kc, vc, 3)
    assert np.array_equal(out, x)


def test_swiglu_gate_then_up():
    # gate rows first: with the up half of the packed weight zero the MLP adds nothing,
    # with the gate half zero it adds nothing either (silu(0) = 0)
    shape = TINY
    lw = synth.layer_weights(shape, 2, 0, sigma=0.3)
    lw["w_qkv"] = np.zeros_like(lw["w_qkv"])
    lw["w_o"] = np.zeros_like(lw["w_o"])
    x = np.linspace(-1, 1, shape.hidden).astype(np.float32)
    kvd = shape.kv_heads * shape.head_dim
    I = shape.inter
    for zero_half in (slice(0, I), slice(I, 2 * I)):
        w = dict(lw)
        w["w_gate_up"] = lw["w_gate_up"].copy()
        w["w_gate_up"][zero_half] = 0
        out, _, _ = oracle.layer_decode(shape, w, x, np.zeros((1, kvd), np.float32),
                                        np.zeros((1, kvd), np.float32), 0)
        assert np.array_equal(out, x)
    # with both halves present the MLP contributes, and swapping them changes it
    out, _, _ = oracle.layer_decode(shape, lw, x, np.zeros((1, kvd), np.float32),
                                    np.zeros((1, kvd), np.float32), 0)
    sw = dict(lw)
    sw["w_gate_up"] = np.concatenate([lw["w_gate_up"][I:], lw["w_gate_up"][:I]])
    out_sw, _, _ = oracle.layer_decode(shape, sw, x, np.zeros((1, kvd), np.float32),
                                       np.zeros((1, kvd), np.float32), 0)
    assert not np.array_equal(out, x) and not np.allclose(out, out_sw)


# ------------------------------------------------------------- prefill ---

def _prefill_inputs(seed, start, T):
    shape = TINY
    wts = synth.model_weights(shape, seed, sigma=0.3, norm_sigma=0.3)
    wl = synth.decode_workload("tiny-prefill", shape, seed, [start + T - 1], num_pages=40)
    tokens = synth.rng(seed, "tokens").integers(0, shape.vocab, size=T)
    return shape, wts, wl.pool, wl.block_tables[:, 0], tokens


@pytest.mark.parametrize("start,T", [(0, 21), (7, 25)])
def test_prefill_matches_float64_causal_brute_force(start, T):
    """The oracle's prefill (one decode step per prompt token) against the
    whole prompt computed at once in float64 with a causal mask: last
    token's logits, its argmax, and every K/V row written to the pool."""
    shape, wts, pool, bts, tokens = _prefill_inputs(11 + start, start, T)
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    logits, best, pool_after = oracle.prefill_paged(shape, wts, pool, geo, bts, start, tokens)
    ref_logits, written = brute.prefill(shape, wts, pool, bts, start, tokens)
    np.testing.assert_allclose(logits, ref_logits, rtol=1e-5, atol=1e-5)
    top2 = np.sort(ref_logits)[-2:]
    if top2[1] - top2[0] > 1e-4:
        assert best == int(np.argmax(ref_logits))
    kv_view, vv_view = brute.pool_view(pool_after, shape.kv_heads, shape.head_dim)
    touched = np.zeros(pool.shape, dtype=bool)
    tv, vv_t = brute.pool_view(touched, shape.kv_heads, shape.head_dim)
    for l in range(shape.layers):
        K, V = written[l]
        for t in range(T):
            p = start + t
            page, slot = bts[l][p // 16], p % 16
            got_k = brute.bf16_bits_to_f64(brute.k_of(kv_view, page, slot)).reshape(shape.kv_heads, -1)
            got_v = brute.bf16_bits_to_f64(vv_view[page, 0, :, :, slot])
            # one BF16 ulp at most (FP32 vs float64 values before rounding)
            np.testing.assert_allclose(got_k, K[t], rtol=2 ** -7, atol=1e-6)
            np.testing.assert_allclose(got_v, V[t], rtol=2 ** -7, atol=1e-6)
            brute.k_of(tv, page, slot)[...] = True
            vv_t[page, 0, :, :, slot] = True
    assert np.array_equal(pool_after[~touched], pool[~touched])


def test_prefill_of_one_token_is_a_decode_step():
    shape, wts, pool, bts, tokens = _prefill_inputs(13, 30, 1)
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    logits, best, _ = oracle.prefill_paged(shape, wts, pool, geo, bts, 30, tokens)
    ref, nxt, _, _ = oracle.decode_step_paged(shape, wts, pool, geo, bts[:, None], [30], tokens)
    assert np.array_equal(logits, ref[0]) and best == nxt[0]


def test_layer_with_a_given_cache_row():
    """row_given: attention reads row pos as the caller wrote it.  With the
    values the layer would write itself the result is identical; with
    other values the returned K/V (the layer's own) are unchanged and only
    the output moves."""
    shape = synth.tiny_shape(hidden=64, heads=4, kv_heads=2, inter=128, head_dim=16, name="rowgiven")
    lw = synth.layer_weights(shape, 5, 0, sigma=0.1, norm_sigma=0.2)
    g = np.random.default_rng(6)
    x = g.standard_normal(shape.hidden).astype(np.float32)
    pos, kvd = 6, shape.kv_heads * shape.head_dim
    kc = g.standard_normal((pos + 1, kvd)).astype(np.float32)
    vc = g.standard_normal((pos + 1, kvd)).astype(np.float32)
    y, kb, vb = oracle.layer_decode(shape, lw, x, kc.copy(), vc.copy(), pos)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[pos], vc2[pos] = oracle.bf16_to_f32(kb), oracle.bf16_to_f32(vb)
    y2, kb2, vb2 = oracle.layer_decode(shape, lw, x, kc2, vc2, pos, row_given=True)
    assert np.array_equal(y, y2) and np.array_equal(kb, kb2) and np.array_equal(vb, vb2)
    kc3, vc3 = kc2.copy(), vc2.copy()
    vc3[pos] += 0.5
    y3, kb3, vb3 = oracle.layer_decode(shape, lw, x, kc3, vc3, pos, row_given=True)
    assert np.array_equal(kb, kb3) and np.array_equal(vb, vb3)
    assert not np.array_equal(y, y3)
    assert np.array_equal(vc3[pos], vc2[pos] + 0.5)  # the given row is left as it is
