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


DEEP_KV_REL = 1e-2


def check_prefill_pool(got, want, base, geo, bts, start, T, layers):
    """Pool after a prefill of T tokens at start .. start + T - 1 through the
    per-layer tables bts [layers, max_pages].  Bytes no append writes must be
    untouched.  Layer 0's K/V come from the exact embedding rows: each within
    one BF16 ulp of the oracle's value or APPEND_REL * RMS (check_pool_after).
    A later layer's K/V are the BF16 rounding of a projection of a hidden
    state that carries the earlier layers' error, including the rounding of
    every earlier prompt token's K/V to BF16 in the pool, which may land on
    the other neighbour in the two paths; that hidden state is held to the
    layer bar (1e-2 of its RMS), so these values must lie within one BF16 ulp
    plus DEEP_KV_REL * RMS of the oracle's.  Returns the per-layer max-abs
    differences."""
    pos = [start + t for t in range(T)]
    masks = [appended_mask(base, geo, [bts[l]] * T, pos) for l in range(layers)]
    every = np.logical_or.reduce(masks)
    assert np.array_equal(got[~every], base[~every]), "pool bytes outside the appended slots changed"
    out = []
    for l, m in enumerate(masks):
        g = oracle.bf16_to_f32(got[m]).astype(np.float64)
        w = oracle.bf16_to_f32(want[m]).astype(np.float64)
        rms = float(np.sqrt(np.mean(w * w))) if w.size else 0.0
        ulp = np.abs(w) * 2.0 ** -7
        bound = np.maximum(ulp, APPEND_REL * rms) if l == 0 else ulp + DEEP_KV_REL * rms
        bad = np.abs(g - w) > bound
        assert not bad.any(), "appended K/V of layer %d: %d values off by up to %.3g (RMS %.3g)" % (
            l, int(bad.sum()), float(np.abs(g - w).max()), rms)
        out.append(float(np.abs(g - w).max(initial=0.0)))
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
