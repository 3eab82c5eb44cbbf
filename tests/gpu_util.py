"""Helpers of the GPU parity tests: run the HIP path through the C ABI on
seeded inputs and compare with the oracle."""
import sys

import numpy as np
import torch

import oracle
import paged_kv_transformer_amd as pkv


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return pkv.to_device(a)


def host_u16(t):
    return t.cpu().numpy().view(np.uint16)


def device_pool(pool_np, kv_heads, head_dim=64, page_tokens=16):
    """The pool on the GPU: pool_np is one array of whole pages, or a
    (k_pool, v_pool) pair for separate K and V pools.  Returns (pkv Pool,
    a reader of the device pool as whole pages: the separate pools are put
    back together by the oracle's layout definition)."""
    geo = oracle.PoolGeometry(kv_heads, head_dim, page_tokens)
    if isinstance(pool_np, tuple):
        kt, vt = dev(pool_np[0]), dev(pool_np[1])
        P = pkv.kv_pool_create_split(kt, vt, kv_heads, head_dim=head_dim, page_tokens=page_tokens)
        return P, lambda: oracle.whole_pool(host_u16(kt), host_u16(vt), geo)
    t = dev(pool_np)
    P = pkv.kv_pool_create(t, kv_heads, head_dim=head_dim, page_tokens=page_tokens)
    return P, lambda: host_u16(t)


def whole(pool_np, geo):
    """The oracle's input: whole pages (separate pools put together)."""
    return oracle.whole_pool(pool_np[0], pool_np[1], geo) if isinstance(pool_np, tuple) else pool_np


def attention_gpu(pool_np, kv_heads, q_bits, bt, lens, scale, ws=None, page_tokens=16):
    """Run paged_gqa_decode; returns (out [B, Hq, D] float32, device error
    bits).  D is q's last dimension, also the pool's head width."""
    B, Hq, D = q_bits.shape
    pool, _ = device_pool(pool_np, kv_heads, D, page_tokens)
    bt = np.ascontiguousarray(bt, dtype=np.int32)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    if ws is None:
        ws = pkv.alloc_workspace(pkv.attention_workspace_bytes(Hq, kv_heads, B, bt.shape[1], head_dim=D,
                                                               page_tokens=page_tokens))
    pkv.paged_gqa_decode(pool, dev(q_bits), dev(bt), dev(np.asarray(lens, dtype=np.int32)),
                         scale, out, ws)
    err = pkv.device_error(ws)
    return out.cpu().numpy(), err


def attention_oracle(pool_np, kv_heads, q_bits, bt, lens, scale, seqs=None, page_tokens=16):
    geo = oracle.PoolGeometry(kv_heads, q_bits.shape[2], page_tokens)
    return oracle.paged_attention(whole(pool_np, geo), geo, oracle.bf16_to_f32(q_bits), bt, lens, scale, seqs)


def layer_gpu(shape, lw, hidden, pool_np, bt, positions, max_pos=None, page_tokens=16):
    """decoder_layer_decode on one layer; returns (hidden_out, pool_after as
    whole pages, err)."""
    B = len(positions)
    bt = np.ascontiguousarray(bt, dtype=np.int32)
    mp = max_pos or int(max(positions)) + 1
    cfg = pkv.make_config(shape, max_pos=mp, layers=1)
    layer = pkv.upload_layer(lw, head_dim=shape.head_dim)
    c, s = pkv.rope_table(shape.theta, mp, head_dim=shape.head_dim)
    pool, read_pool = device_pool(pool_np, shape.kv_heads, shape.head_dim, page_tokens)
    h = torch.from_numpy(np.ascontiguousarray(hidden, dtype=np.float32)).cuda()
    ws = pkv.alloc_workspace(pkv.workspace_bytes(cfg, B, bt.shape[1], page_tokens))
    pkv.decoder_layer_decode(cfg, layer, c, s, pool, dev(bt), dev(np.asarray(positions, np.int32)), h, ws)
    err = pkv.device_error(ws)
    return h.cpu().numpy(), read_pool(), err


def expected_pool_after(pool_np, geo, bt, positions, k_new, v_new, seqs=None):
    want = pool_np.copy()
    for b in (range(len(positions)) if seqs is None else seqs):
        oracle.pool_append(want, geo, bt[b], int(positions[b]), k_new[b], v_new[b])
    return want


APPEND_REL = 1e-3

# Output bars.  A layer's output: max-abs <= LAYER_TOL * RMS(out), and the
# layer's own contribution (the residual delta out - hidden, which the N(0,1)
# residual would otherwise hide): max-abs <= DELTA_TOL * RMS(out - hidden).
# Logits of the full-size models: max-abs <= LOGIT_ABS, the budget under which
# no argmax whose top-2 gap exceeds 1e-3 can flip (each of two logits off by
# less than 5e-4).  Logits of the small test models, whose weights are drawn
# 2.5 times wider (0.05) and whose norm gains vary 15 times more (0.3) to
# drive larger activations through every path: max-abs <= TINY_LOGIT_REL *
# RMS(logits).
LAYER_TOL = 1e-2
DELTA_TOL = 1e-3
LOGIT_ABS = 4e-4
TINY_LOGIT_REL = 5e-3


def _rms64(a):
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


def assert_layer_out(got, ref, hidden, label):
    """A layer's output against the oracle's (rows already selected)."""
    diff = float(np.abs(np.asarray(got, np.float64) - ref).max())
    delta = diff / max(_rms64(np.asarray(ref, np.float64) - hidden), 1e-30)
    say("%s: max-abs %.3g, RMS(out) %.3g, error/RMS(delta) %.3g" % (label, diff, _rms64(ref), delta))
    assert diff <= LAYER_TOL * _rms64(ref), "%s: max-abs %.3g" % (label, diff)
    assert delta <= DELTA_TOL, "%s: error/RMS(delta) %.3g > %.0e" % (label, delta, DELTA_TOL)
    return diff


def assert_logits(got, ref, label, full_size=False):
    """Logits against the oracle's; returns the max-abs difference."""
    diff = float(np.abs(np.asarray(got, np.float64) - ref).max())
    bar = LOGIT_ABS if full_size else TINY_LOGIT_REL * _rms64(ref)
    say("%s: max|dlogit| %.3g (RMS %.3g, bar %.3g)" % (label, diff, _rms64(ref), bar))
    assert diff <= bar, "%s: max|dlogit| %.3g > %.3g" % (label, diff, bar)
    return diff


def appended_mask(pool_np, geo, rows, positions):
    """Pool elements the appends of `positions` (through table rows `rows`)
    write, found by the oracle's own append of marker values on a zero pool."""
    z = np.zeros(pool_np.shape, np.uint16)
    one = np.full(geo.kv_heads * geo.head_dim, 0x3F80, np.uint16)
    for row, p in zip(rows, positions):
        oracle.pool_append(z, geo, row, int(p), one, one)
    return z != 0


def check_pool_after(got, want, base, rel=APPEND_REL, touched=None):
    """Bytes the step did not append must be untouched.  An appended BF16
    value is the rounding of an FP32 contraction whose last bits differ
    between the two paths (summation order, the two-half BF16 split of the
    activations), so it must lie within one BF16 ulp of the oracle's value or
    within rel * RMS(appended values) of it: near zero an ulp is far smaller
    than the contraction's absolute error.  rel is APPEND_REL for the decode
    step, whose activations keep ~16 bits.  touched: the appended elements
    (default: where the oracle's pool differs from the base)."""
    if touched is None:
        touched = want != base
    assert np.array_equal(got[~touched], base[~touched]), "pool bytes outside the appended slots changed"
    g = oracle.bf16_to_f32(got[touched]).astype(np.float64)
    w = oracle.bf16_to_f32(want[touched]).astype(np.float64)
    ulp = np.abs(w) * 2.0 ** -7 + 1e-38
    rms = float(np.sqrt(np.mean(w * w))) if w.size else 0.0
    bad = np.abs(g - w) > np.maximum(ulp, rel * rms)
    assert not bad.any(), "appended K/V: %d values off by up to %.3g (RMS %.3g)" % (
        int(bad.sum()), float(np.abs(g - w).max()), rms)
    return float(np.abs(g - w).max(initial=0.0)), rms


def check_kv_values(got_bits, want_bits, rel=APPEND_REL, rms=None, what="appended K/V"):
    """BF16 values written by the GPU against the oracle's: each within one
    BF16 ulp of the oracle's value or within rel * RMS (default: the RMS of
    the oracle's values).  Returns (max-abs difference, RMS)."""
    g = oracle.bf16_to_f32(np.asarray(got_bits, np.uint16)).astype(np.float64)
    w = oracle.bf16_to_f32(np.asarray(want_bits, np.uint16)).astype(np.float64)
    if rms is None:
        rms = float(np.sqrt(np.mean(w * w))) if w.size else 0.0
    bad = np.abs(g - w) > np.maximum(np.abs(w) * 2.0 ** -7, rel * rms)
    assert not bad.any(), "%s: %d values off by up to %.3g (RMS %.3g)" % (
        what, int(bad.sum()), float(np.abs(g - w).max()), rms)
    return float(np.abs(g - w).max(initial=0.0)), rms


def teacher_forced_prefill_kv(shape, weights, pool_after, geo, bts, start, tokens, t_list=None):
    """The oracle's K/V of prompt tokens `t_list` at every layer, each token
    run through the layers with the attention reading the GPU's own pool for
    every position up to and including its own (teacher forcing): a later
    layer's K/V then differ from the GPU's only by this token's own
    arithmetic in that layer's projections, not by K/V values (this token's
    or earlier ones') that BF16 rounding put on the other neighbour, which a
    free-running comparison lets pass from layer to layer and token to token
    (a token at position 0 attends to nothing but its own K/V).  Returns
    {(layer, t): (k_bits, v_bits)} and, under key ("x", t), the token's
    final hidden state."""
    T = len(tokens)
    out = {}
    for t in (range(T) if t_list is None else t_list):
        p = start + t
        x = oracle.embed(weights["embed"], int(tokens[t]))
        for l in range(shape.layers):
            kc, vc = oracle.pool_gather(pool_after, geo, bts[l], p + 1)
            x, kb, vb = oracle.layer_decode(shape, weights["layers"][l], x, kc, vc, p, row_given=True)
            out[(l, t)] = (kb, vb)
        out[("x", t)] = x
    return out


def prompt_kv_bits(pool, geo, bt_row, start, T):
    """BF16 bits of the K and V a pool holds at positions start .. start+T-1
    of one layer's table: ([T][kv*D], [T][kv*D])."""
    kc, vc = oracle.pool_gather(pool, geo, bt_row, start + T)
    return oracle.f32_to_bf16(kc[start:]), oracle.f32_to_bf16(vc[start:])


def check_prefill_pool(got, base, geo, bts, start, tokens, shape, weights, t_list=None):
    """Pool after a prefill of the prompt `tokens` at positions start ..
    start + T - 1 through the per-layer tables bts [layers, max_pages].
    Bytes no append writes must be untouched.  Every layer's K/V of the
    tokens in t_list (default: all) must match the oracle's teacher-forced
    values (teacher_forced_prefill_kv) within one BF16 ulp or APPEND_REL of
    the layer's RMS, the decode append's bar.  Returns the per-layer max-abs
    differences."""
    T = len(tokens)
    pos = [start + t for t in range(T)]
    L = shape.layers
    masks = [appended_mask(base, geo, [bts[l]] * T, pos) for l in range(L)]
    every = np.logical_or.reduce(masks)
    assert np.array_equal(got[~every], base[~every]), "pool bytes outside the appended slots changed"
    tl = list(range(T)) if t_list is None else list(t_list)
    ref = teacher_forced_prefill_kv(shape, weights, got, geo, bts, start, tokens, tl)
    out = []
    for l in range(L):
        gk, gv = prompt_kv_bits(got, geo, bts[l], start, T)
        want = np.concatenate([np.concatenate([ref[(l, t)][0], ref[(l, t)][1]]) for t in tl])
        have = np.concatenate([np.concatenate([gk[t], gv[t]]) for t in tl])
        d, _ = check_kv_values(have, want, what="prefill K/V of layer %d" % l)
        out.append(d)
    return out


def step_gpu(shape, weights, pool_np, bts, positions, tokens, want_logits=True, max_pos=None,
             want_pool=True, page_tokens=16):
    """decode_step; returns (logits or None, next_tokens, pool_after (whole
    pages) or None, err)."""
    B = len(positions)
    mp = max_pos or int(max(positions)) + 1
    cfg = pkv.make_config(shape, max_pos=mp)
    model = pkv.upload_model(weights, shape.theta, mp, head_dim=shape.head_dim)
    pool, read_pool = device_pool(pool_np, shape.kv_heads, shape.head_dim, page_tokens)
    bts = np.ascontiguousarray(bts, dtype=np.int32)
    ws = pkv.alloc_workspace(pkv.workspace_bytes(cfg, B, bts.shape[2], page_tokens))
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda") if want_logits else None
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    pkv.decode_step(cfg, model, pool, dev(bts), dev(np.asarray(positions, np.int32)),
                    dev(np.asarray(tokens, np.int32)), logits, nxt, ws)
    err = pkv.device_error(ws)
    pool_after = read_pool() if want_pool else None
    return (None if logits is None else logits.cpu().numpy()), nxt.cpu().numpy(), pool_after, err


def check_argmax_rule(ref_logits, got_tokens, gap=1e-3):
    """Identical argmax wherever the oracle's top-2 gap exceeds `gap`."""
    checked = 0
    for b in range(ref_logits.shape[0]):
        top2 = np.sort(ref_logits[b])[-2:]
        if top2[1] - top2[0] > gap:
            assert int(got_tokens[b]) == int(np.argmax(ref_logits[b])), \
                "sequence %d: argmax %d vs oracle %d (gap %.3g)" % (
                    b, int(got_tokens[b]), int(np.argmax(ref_logits[b])), top2[1] - top2[0])
            checked += 1
    return checked
