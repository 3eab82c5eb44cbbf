"""The single-launch batch-1 layer (one workgroup per compute unit, the
layer's weights streamed into LDS, the phases passing (value, epoch) words)
against the oracle, through the C ABI: decoder_layer_decode and decode_step
at batch 1 take it whenever pkv_fused_layer_plan says the layer fits.  Bars
as for every layer (gpu_util): output max-abs <= 1e-2 * RMS(out) and <=
1e-3 * RMS(out - hidden), appended K/V within one BF16 ulp or 1e-3 of their
RMS with the rest of the pool untouched, logits <= 4e-4 for the full-size
vocabulary.  Also: the multi-launch path on the same inputs agrees with it
to the same bars, repeated calls and graph replays (each a new epoch) give
bitwise the same result as the first eager call, and bad table entries or
positions set their device-error bits without stalling any phase."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import paged_kv_transformer_amd as pkv
import synth
from gpu_util import (assert_layer_out, assert_logits, check_argmax_rule, check_pool_after, dev,
                      device_pool, expected_pool_after, say, step_gpu)

pytestmark = pytest.mark.gpu

CUS = None


def _cus():
    global CUS
    if CUS is None:
        CUS = torch.cuda.get_device_properties(0).multi_processor_count
    return CUS


class FusedSetting:
    """Run a block with the single-launch layer switched on or off."""

    def __init__(self, on):
        self.on = on

    def __enter__(self):
        self.prev = pkv.set_fused_layer(self.on)

    def __exit__(self, *exc):
        pkv.set_fused_layer(self.prev)


def _run_layer(shape, lw, hidden, pool_np, bt, positions, fused, max_pos=None, reps=1, page_tokens=16):
    """decoder_layer_decode `reps` times on the same inputs (the pool and
    hidden restored before each call); returns (outputs, pool after the
    last call, err bits)."""
    B = len(positions)
    bt = np.ascontiguousarray(bt, dtype=np.int32)
    mp = max_pos or int(max(positions)) + 1
    cfg = pkv.make_config(shape, max_pos=mp, layers=1)
    layer = pkv.upload_layer(lw, head_dim=shape.head_dim)
    c, s = pkv.rope_table(shape.theta, mp, head_dim=shape.head_dim)
    pool, read_pool = device_pool(pool_np, shape.kv_heads, shape.head_dim, page_tokens)
    ws = pkv.alloc_workspace(pkv.workspace_bytes(cfg, B, bt.shape[1], page_tokens))
    outs = []
    with FusedSetting(fused):
        if fused:
            assert pkv.fused_layer_plan(cfg, B, bt.shape[1], page_tokens, _cus()) == 1
        for _ in range(reps):
            h = torch.from_numpy(np.ascontiguousarray(hidden, dtype=np.float32)).cuda()
            pkv.decoder_layer_decode(cfg, layer, c, s, pool, dev(bt), dev(np.asarray(positions, np.int32)), h, ws)
            outs.append(h.cpu().numpy())
        err = pkv.device_error(ws)
    return outs, read_pool(), err


def _oracle_layer(shape, lw, hidden, pool_np, bt, positions, page_tokens=16):
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim, page_tokens)
    whole = oracle.whole_pool(pool_np[0], pool_np[1], geo) if isinstance(pool_np, tuple) else pool_np
    ref, k_new, v_new = oracle.layer_decode_paged(shape, lw, hidden, whole, geo, bt, positions)
    want = expected_pool_after(whole, geo, bt, positions, k_new, v_new)
    return ref, want, whole


def _check(shape, lw, hidden, wl, label, compare_multi=False, pool=None, page_tokens=16):
    bt = wl.block_tables[0]
    pool_np = wl.pool if pool is None else pool
    cfg = pkv.make_config(shape, max_pos=int(max(wl.positions)) + 1, layers=1)
    assert pkv.fused_layer_plan(cfg, 1, bt.shape[1], page_tokens, _cus()) == 1, \
        "%s: expected the single launch" % label
    say("case %s: p=%d, table %d pages" % (label, int(wl.positions[0]), bt.shape[1]))
    (got,), pool_after, err = _run_layer(shape, lw, hidden, pool_np, bt, wl.positions, True, page_tokens=page_tokens)
    assert err == 0, "device error bits %d" % err
    ref, want, base = _oracle_layer(shape, lw, hidden, pool_np, bt, wl.positions, page_tokens)
    assert_layer_out(got, ref, hidden, "%s single launch" % label)
    kv_diff, kv_rms = check_pool_after(pool_after, want, base)
    say("  appended K/V: max-abs %.3g (RMS %.3g)" % (kv_diff, kv_rms))
    if compare_multi:
        (multi,), pool_multi, err = _run_layer(shape, lw, hidden, pool_np, bt, wl.positions, False,
                                               page_tokens=page_tokens)
        assert err == 0
        assert_layer_out(got, multi.astype(np.float64), hidden, "%s single vs multi-launch" % label)
        check_pool_after(pool_after, pool_multi, base)
    return got


def test_plan_takes_the_qwen_layer():
    """The Qwen2.5-0.5B layer at batch 1 runs as one launch on this GPU; the
    Llama-3.2-1B layer (123 MB of weights) and batches above 1 do not."""
    wl = synth.qwen05_layer_b1()
    cfg = pkv.make_config(synth.QWEN05, max_pos=128, layers=1)
    say("compute units: %d, Qwen table %d pages" % (_cus(), wl.max_pages))
    assert pkv.fused_layer_plan(cfg, 1, wl.max_pages, 16, _cus()) == 1
    assert pkv.fused_layer_plan(cfg, 2, wl.max_pages, 16, _cus()) == 0
    llama = pkv.make_config(synth.LLAMA1B, max_pos=1024, layers=1)
    assert pkv.fused_layer_plan(llama, 1, 64, 16, _cus()) == 0


def test_qwen_layer_batch1_single_launch():
    """The Qwen2.5-0.5B-shaped layer at batch 1, 127 cached + 1 new, against
    the oracle and against the multi-launch path."""
    wl = synth.qwen05_layer_b1()
    _check(wl.shape, wl.extra["weights"], wl.extra["hidden"], wl, "qwen0.5b", compare_multi=True)


@pytest.mark.parametrize("p", [0, 1, 15, 16, 17, 100, 255, 256, 383, 520])
def test_qwen_layer_positions(p):
    """Positions at and around tile edges, and tables of 1 to 33 pages (1 to
    5 attention units per kv head, whose records the output projection's
    workgroups merge)."""
    shape = synth.QWEN05
    seed = 2000 + p
    wl = synth.decode_workload("qwen-fused", shape, seed, [p], layers=1, num_pages=64)
    lw = synth.layer_weights(shape, seed, 0)
    hidden = synth.rng(seed, "hidden").standard_normal((1, shape.hidden)).astype(np.float32)
    _check(shape, lw, hidden, wl, "qwen p=%d" % p)


@pytest.mark.parametrize("page_tokens,split,p", [(256, False, 200), (16, True, 200), (256, True, 200),
                                                 (256, False, 511), (256, True, 300)])
def test_page_geometries(page_tokens, split, p):
    """256-token pages (16 tiles under one table entry) and separate K and V
    pools: the attention units' tile copies and the append go through the
    same pool view as every other kernel; at positions 300 and 511 the two
    256-token pages hold 3 and 4 attention units per kv head, whose records
    the O phase merges."""
    shape = synth.QWEN05
    seed = 2150 + page_tokens + int(split) + p
    wl = synth.decode_workload("qwen-fused-geometry", shape, seed, [p], layers=1, page_tokens=page_tokens)
    lw = synth.layer_weights(shape, seed, 0)
    hidden = synth.rng(seed, "hidden").standard_normal((1, shape.hidden)).astype(np.float32)
    pool = wl.pool
    if split:
        geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim, page_tokens)
        pool = oracle.split_pools(wl.pool, geo)
    _check(shape, lw, hidden, wl, "qwen %d-token pages%s, p=%d" % (page_tokens, ", K/V pools" if split else "", p),
           pool=pool, page_tokens=page_tokens)


def test_table_wider_than_the_sequence():
    """A 32-page table for a 21-token sequence: the attention units past the
    sequence leave empty records (m = -inf) that the merge must skip."""
    shape = synth.QWEN05
    seed = 2101
    wl = synth.decode_workload("qwen-wide-table", shape, seed, [20], layers=1, num_pages=64, max_pages=32)
    lw = synth.layer_weights(shape, seed, 0)
    hidden = synth.rng(seed, "hidden").standard_normal((1, shape.hidden)).astype(np.float32)
    _check(shape, lw, hidden, wl, "qwen wide table")


@pytest.mark.parametrize("hidden,heads,kv,inter,hd", [(192, 4, 2, 384, 64), (192, 14, 2, 4096, 64),
                                                      (256, 16, 1, 512, 64), (512, 4, 2, 1024, 128),
                                                      (1024, 8, 2, 2560, 128)])
def test_small_shapes(hidden, heads, kv, inter, hd):
    """Other geometries: group sizes 2, 7, 16; head width 128; intermediate
    sizes whose down projection takes whole or split row groups."""
    shape = synth.tiny_shape(hidden=hidden, heads=heads, kv_heads=kv, inter=inter, head_dim=hd, name="tiny-fused")
    seed = 2200 + hidden + heads + inter
    p = int(synth.rng(seed, "lens").integers(0, 300))
    wl = synth.decode_workload("tiny-fused", shape, seed, [p], layers=1)
    lw = synth.layer_weights(shape, seed, 0, sigma=0.05, norm_sigma=0.3)
    h = synth.rng(seed, "hidden").standard_normal((1, shape.hidden)).astype(np.float32)
    _check(shape, lw, h, wl, "tiny H%d Hq%d Hkv%d I%d D%d" % (hidden, heads, kv, inter, hd), compare_multi=True)


def test_repeated_calls_and_graph_replays():
    """Every call is a new epoch of the exchange words: five eager calls on
    the same inputs and five replays of a captured call give bitwise the
    first call's output (the pool's appended slot is rewritten with the same
    values each time)."""
    wl = synth.qwen05_layer_b1()
    shape, lw, hidden = wl.shape, wl.extra["weights"], wl.extra["hidden"]
    bt = np.ascontiguousarray(wl.block_tables[0], dtype=np.int32)
    outs, _, err = _run_layer(shape, lw, hidden, wl.pool, bt, wl.positions, True, reps=5)
    assert err == 0
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    cfg = pkv.make_config(shape, max_pos=128, layers=1)
    layer = pkv.upload_layer(lw)
    c, s = pkv.rope_table(shape.theta, 128)
    pool, _ = device_pool(wl.pool, shape.kv_heads)
    ws = pkv.alloc_workspace(pkv.workspace_bytes(cfg, 1, bt.shape[1]))
    h = torch.from_numpy(np.ascontiguousarray(hidden, dtype=np.float32)).cuda()
    h0 = h.clone()
    bt_d, pos_d = dev(bt), dev(np.asarray(wl.positions, np.int32))
    stream = torch.cuda.Stream()
    with FusedSetting(True):
        pkv.decoder_layer_decode(cfg, layer, c, s, pool, bt_d, pos_d, h, ws)  # eager call first
        torch.cuda.synchronize()
        h.copy_(h0)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                pkv.decoder_layer_decode(cfg, layer, c, s, pool, bt_d, pos_d, h, ws, stream)
        torch.cuda.synchronize()
        for r in range(5):
            h.copy_(h0)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(h.cpu().numpy(), outs[0]), "replay %d differs" % r
    assert pkv.device_error(ws) == 0


def test_device_errors_do_not_stall():
    """A cached page outside the pool sets PKV_DEVERR_PAGE, a position past
    the RoPE table PKV_DEVERR_ROPE; every phase still receives its inputs
    (no PKV_DEVERR_SYNC) and the call returns."""
    wl = synth.qwen05_layer_b1()
    shape, lw, hidden = wl.shape, wl.extra["weights"], wl.extra["hidden"]
    bt = np.array(wl.block_tables[0], dtype=np.int32)
    bt[0, 2] = wl.num_pages + 5
    _, _, err = _run_layer(shape, lw, hidden, wl.pool, bt, wl.positions, True)
    say("bad page: err bits %d" % err)
    assert err & pkv.DEVERR_PAGE and not err & pkv.DEVERR_SYNC
    bt = np.array(wl.block_tables[0], dtype=np.int32)
    _, _, err = _run_layer(shape, lw, hidden, wl.pool, bt, wl.positions, True, max_pos=100)
    say("position past the RoPE table: err bits %d" % err)
    assert err & pkv.DEVERR_ROPE and not err & pkv.DEVERR_SYNC


def test_step_qwen_batch1_single_launch_layers():
    """decode_step at batch 1 with single-launch layers: a 3-layer model of
    the Qwen2.5-0.5B shape (full 151936-token vocabulary), position 127;
    logits within 4e-4 of the oracle's, the argmax rule, the pool's appends."""
    shape = dataclasses.replace(synth.QWEN05, layers=3)
    seed = 2301
    wl = synth.decode_workload("qwen-fused-step", shape, seed, [127], layers=3)
    weights = synth.model_weights(shape, seed, layers=3)
    tokens = synth.rng(seed, "tokens").integers(0, shape.vocab, size=1).astype(np.int32)
    cfg = pkv.make_config(shape, max_pos=128)
    assert pkv.fused_layer_plan(cfg, 1, wl.max_pages, 16, _cus()) == 1
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    with FusedSetting(True):
        logits, nxt, pool_after, err = step_gpu(shape, weights, wl.pool, wl.block_tables, wl.positions, tokens)
    assert err == 0
    ref_logits, ref_tok, k_all, v_all = oracle.decode_step_paged(shape, weights, wl.pool, geo, wl.block_tables,
                                                                 wl.positions, tokens)
    assert_logits(logits, ref_logits, "qwen 3-layer step, single-launch layers", full_size=True)
    check_argmax_rule(ref_logits, nxt)
    with FusedSetting(False):
        logits_m, nxt_m, _, err = step_gpu(shape, weights, wl.pool, wl.block_tables, wl.positions, tokens,
                                           want_pool=False)
    assert err == 0
    assert_logits(logits, logits_m.astype(np.float64), "single vs multi-launch layers", full_size=True)


def test_one_workspace_across_shapes_and_entry_points():
    """One workspace, sized for the largest call, serves in turn the
    single-launch layer at batch 1, the multi-launch layer at batch 4 over
    tables of up to 4 attention splits, attention alone at batch 6 with
    another head grouping, sampling over 4 rows, then the first two calls
    again: each output is
    bitwise that of the same call on a freshly initialised workspace.  The
    exchange words and launch counters one call leaves behind never pass for
    another's, whatever shape reuses their bytes."""
    shape = synth.QWEN05
    D, Hkv = shape.head_dim, shape.kv_heads
    seed = 2400
    lw = synth.layer_weights(shape, seed, 0)
    layer = pkv.upload_layer(lw, head_dim=D)
    mp = 600
    cfg = pkv.make_config(shape, max_pos=mp, layers=1)
    c, s = pkv.rope_table(shape.theta, mp, head_dim=D)
    wl1 = synth.decode_workload("qwen-shared-ws-b1", shape, seed, [300], layers=1, num_pages=64)
    wl4 = synth.decode_workload("qwen-shared-ws-b4", shape, seed + 1, [450, 37, 511, 260], layers=1,
                                num_pages=256)
    pool1, _ = device_pool(wl1.pool, Hkv, D, 16)
    pool4, _ = device_pool(wl4.pool, Hkv, D, 16)
    bt1, bt4 = dev(np.ascontiguousarray(wl1.block_tables[0])), dev(np.ascontiguousarray(wl4.block_tables[0]))
    pos1, pos4 = dev(np.asarray(wl1.positions, np.int32)), dev(np.asarray(wl4.positions, np.int32))
    h1 = synth.rng(seed, "hidden", 1).standard_normal((1, shape.hidden)).astype(np.float32)
    h4 = synth.rng(seed, "hidden", 4).standard_normal((4, shape.hidden)).astype(np.float32)
    # attention alone: 8 query heads over the batch-4 pool's 2 kv heads (groups of 4)
    Hq_a, Ba = 8, 6
    wla = synth.decode_workload("qwen-shared-ws-attn", shape, seed + 2, [700, 90, 1000, 17, 400, 1023],
                                layers=1, num_pages=wl4.num_pages, max_pages=64, with_pool=False)
    lens_a = dev(np.asarray(wla.positions, np.int32) + 1)
    bta = dev(np.ascontiguousarray(wla.block_tables[0]))
    qa = synth.rng(seed, "q", 6).standard_normal((Ba, Hq_a, D)).astype(np.float32)
    qa_d = torch.from_numpy(qa).to(torch.bfloat16).view(torch.int16).cuda()
    # sampling over 4 rows of 5000 logits (its histograms and candidate
    # lists land where the layers keep other data)
    Bs, Vs = 4, 5000
    lg = torch.from_numpy(synth.rng(seed, "logits").standard_normal((Bs, Vs)).astype(np.float32) * 3).cuda()
    temp = torch.tensor([1.0, 0.7, 1.3, 0.0], dtype=torch.float32, device="cuda")
    topp = torch.tensor([0.9, 0.5, 1.0, 0.9], dtype=torch.float32, device="cuda")
    topk = torch.tensor([0, 50, 7, 0], dtype=torch.int32, device="cuda")
    uu = torch.from_numpy(synth.rng(seed, "sample").random(Bs).astype(np.float32)).cuda()
    need = max(pkv.workspace_bytes(cfg, 1, bt1.shape[1]), pkv.workspace_bytes(cfg, 4, bt4.shape[1]),
               pkv.attention_workspace_bytes(Hq_a, Hkv, Ba, bta.shape[1], head_dim=D),
               pkv.sample_workspace_bytes(Bs, Vs))
    shared = pkv.alloc_workspace(need)

    def layer_call(bt, pos, pool, h, ws):
        t = torch.from_numpy(np.ascontiguousarray(h)).cuda()
        pkv.decoder_layer_decode(cfg, layer, c, s, pool, bt, pos, t, ws)
        return t.cpu().numpy()

    def attn_call(ws):
        out = torch.full((Ba, Hq_a, D), float("nan"), dtype=torch.float32, device="cuda")
        pkv.paged_gqa_decode(pool4, qa_d, bta, lens_a, 0.125, out, ws)
        return out.cpu().numpy()

    def sample_call(ws):
        tok = torch.full((Bs,), -1, dtype=torch.int32, device="cuda")
        pkv.sample_tokens(lg, temp, topp, topk, uu, tok, ws)
        return tok.cpu().numpy()

    calls = [("layer b1 (single launch)", lambda ws: layer_call(bt1, pos1, pool1, h1, ws)),
             ("layer b4", lambda ws: layer_call(bt4, pos4, pool4, h4, ws)),
             ("attention b6 G4", attn_call),
             ("sampling b4", sample_call),
             ("layer b1 again", lambda ws: layer_call(bt1, pos1, pool1, h1, ws)),
             ("layer b4 again", lambda ws: layer_call(bt4, pos4, pool4, h4, ws))]
    with FusedSetting(True):
        assert pkv.fused_layer_plan(cfg, 1, bt1.shape[1], 16, _cus()) == 1
        for label, call in calls:
            say("shared workspace: %s" % label)
            got = call(shared)
            fresh = pkv.alloc_workspace(need)
            want = call(fresh)
            assert pkv.device_error(fresh) == 0
            assert np.array_equal(got, want), "%s on the shared workspace differs" % label
    assert pkv.device_error(shared) == 0


def test_step_qwen_batch1_single_launch_256_token_pages():
    """decode_step at batch 1 with single-launch layers over 256-token pages
    in separate K and V pools: a 2-layer model of the Qwen2.5-0.5B shape at
    position 300 (two pages per layer, three live attention units per kv
    head whose records the O phase merges); logits within 4e-4 of the
    oracle's (the whole pool's), the argmax rule, the appended K/V."""
    shape = dataclasses.replace(synth.QWEN05, layers=2)
    seed = 2321
    PT = 256
    wl = synth.decode_workload("qwen-fused-step-256", shape, seed, [300], layers=2, page_tokens=PT)
    weights = synth.model_weights(shape, seed, layers=2)
    tokens = synth.rng(seed, "tokens").integers(0, shape.vocab, size=1).astype(np.int32)
    cfg = pkv.make_config(shape, max_pos=301)
    assert pkv.fused_layer_plan(cfg, 1, wl.max_pages, PT, _cus()) == 1
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim, PT)
    pools = oracle.split_pools(wl.pool, geo)
    with FusedSetting(True):
        logits, nxt, pool_after, err = step_gpu(shape, weights, pools, wl.block_tables, wl.positions, tokens,
                                                page_tokens=PT)
    assert err == 0
    ref_logits, ref_tok, k_all, v_all = oracle.decode_step_paged(shape, weights, wl.pool, geo, wl.block_tables,
                                                                 wl.positions, tokens)
    assert_logits(logits, ref_logits, "qwen 2-layer step, 256-token pages, K/V pools", full_size=True)
    check_argmax_rule(ref_logits, nxt)
    want = wl.pool
    for l in range(shape.layers):
        want = expected_pool_after(want, geo, wl.block_tables[l], wl.positions, k_all[l], v_all[l])
    kv_diff, kv_rms = check_pool_after(pool_after, want, wl.pool)
    say("  appended K/V of both layers: max-abs %.3g (RMS %.3g)" % (kv_diff, kv_rms))
