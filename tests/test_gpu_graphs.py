"""The entry points under HIP graph capture: each call is captured once and
replayed several times with new inputs written in place between replays
(torch copies on the stream, plus the host synchronisations of
pkv_device_error), and every replay must give bitwise the outputs of an
eager call on a separate, identical set of buffers.  This covers the state
the kernels keep in their workspace between calls (split records, the
sampler's histograms and choices, argmax keys): a replay that found it left
over from an earlier replay would differ from the eager call."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_transformer_amd as pkv
import synth
from gpu_util import dev, host_u16, say

pytestmark = pytest.mark.gpu


def capture(fn):
    """fn(stream) captured into a HIP graph on a side stream (no launch)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("batch", [1, 5, 64])
def test_decode_step_replays_match_eager(batch):
    """Four replays, each one position further with new tokens; batch 1
    takes the single-launch layers (whose exchange words carry a new epoch
    on every replay), batch 64 the tiled projections."""
    shape = synth.tiny_shape(hidden=128, layers=3, heads=4, kv_heads=2, inter=256, vocab=1000)
    seed = 1100 + batch
    p0 = synth.rng(seed, "lens").integers(0, 200, size=batch).astype(np.int32)
    p0[:3] = [0, 14, 15][:batch]
    R = 4
    wl = synth.decode_workload("graph", shape, seed, p0 + R - 1)  # tables hold every replay's token
    weights = synth.model_weights(shape, seed, sigma=0.05, norm_sigma=0.3)
    mp = int(p0.max()) + R
    cfg = pkv.make_config(shape, max_pos=mp)
    if batch == 1:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        assert pkv.fused_layer_plan(cfg, 1, wl.max_pages, 16, cus) == 1
    model = pkv.upload_model(weights, shape.theta, mp)
    bts = dev(wl.block_tables)
    pools, P = [], []
    for _ in range(3):  # graph, eager, warm-up
        t = dev(wl.pool)
        pools.append(t)
        P.append(pkv.kv_pool_create(t, shape.kv_heads))
    nbytes = pkv.workspace_bytes(cfg, batch, wl.max_pages)
    ws = [pkv.alloc_workspace(nbytes) for _ in range(3)]
    logits = [torch.empty((batch, shape.vocab), dtype=torch.float32, device="cuda") for _ in range(3)]
    nxt = [torch.empty(batch, dtype=torch.int32, device="cuda") for _ in range(3)]
    pos_g = dev(p0)
    tok_g = dev(np.zeros(batch, np.int32))
    # load the kernels before the capture (on the warm-up buffers)
    pkv.decode_step(cfg, model, P[2], bts, pos_g, tok_g, logits[2], nxt[2], ws[2])
    torch.cuda.synchronize()
    g = capture(lambda s: pkv.decode_step(cfg, model, P[0], bts, pos_g, tok_g, logits[0], nxt[0], ws[0], s))
    for r in range(R):
        toks = synth.rng(seed, "tokens", r).integers(0, shape.vocab, size=batch).astype(np.int32)
        pos = (p0 + r).astype(np.int32)
        pos_g.copy_(torch.from_numpy(pos).cuda())
        tok_g.copy_(torch.from_numpy(toks).cuda())
        g.replay()
        pkv.decode_step(cfg, model, P[1], bts, dev(pos), dev(toks), logits[1], nxt[1], ws[1])
        assert pkv.device_error(ws[0]) == 0 and pkv.device_error(ws[1]) == 0
        assert torch.equal(logits[0], logits[1]), "replay %d: logits differ from the eager call" % r
        assert torch.equal(nxt[0], nxt[1]), "replay %d: tokens differ from the eager call" % r
        if r == 0:
            geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
            ref, _, _, _ = oracle.decode_step_paged(shape, weights, wl.pool, geo, wl.block_tables, pos, toks)
            rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
            assert np.abs(logits[0].cpu().numpy() - ref).max() <= 1e-2 * rms
    assert np.array_equal(host_u16(pools[0]), host_u16(pools[1]))
    say("decode_step graph B=%d: %d replays bitwise equal to eager" % (batch, R))


def test_paged_attention_replays_match_eager():
    w = synth.attention_workload(batch=8)
    B, Hq = 8, 32
    lens = w["lens"]
    pool_t = dev(w["pool"])
    P = pkv.kv_pool_create(pool_t, 8)
    bt, ln = dev(w["block_table"]), dev(lens)
    q_g = dev(w["q"])
    out = [torch.empty((B, Hq, 64), dtype=torch.float32, device="cuda") for _ in range(2)]
    ws = [pkv.alloc_workspace(pkv.attention_workspace_bytes(Hq, 8, B, bt.shape[1])) for _ in range(2)]
    pkv.paged_gqa_decode(P, q_g, bt, ln, 0.125, out[1], ws[1])
    torch.cuda.synchronize()
    g = capture(lambda s: pkv.paged_gqa_decode(P, q_g, bt, ln, 0.125, out[0], ws[0], s))
    for r in range(4):
        q = synth.bf16_normal(1200 + r, "q", (B, Hq, 64))
        q_g.copy_(torch.from_numpy(q.view(np.int16)).cuda())
        g.replay()
        pkv.paged_gqa_decode(P, dev(q), bt, ln, 0.125, out[1], ws[1])
        assert pkv.device_error(ws[0]) == 0
        assert torch.equal(out[0], out[1]), "replay %d differs from the eager call" % r


def test_sample_tokens_replays_match_eager():
    B, V = 8, 50000
    bufs = []
    for _ in range(2):
        bufs.append({"logits": torch.empty((B, V), dtype=torch.float32, device="cuda"),
                     "temp": torch.empty(B, dtype=torch.float32, device="cuda"),
                     "top_p": torch.empty(B, dtype=torch.float32, device="cuda"),
                     "top_k": torch.empty(B, dtype=torch.int32, device="cuda"),
                     "u": torch.empty(B, dtype=torch.float32, device="cuda"),
                     "tok": torch.empty(B, dtype=torch.int32, device="cuda"),
                     "ws": pkv.alloc_workspace(pkv.sample_workspace_bytes(B, V))})

    def call(b, s=None):
        pkv.sample_tokens(b["logits"], b["temp"], b["top_p"], b["top_k"], b["u"], b["tok"], b["ws"], s)

    def fill(b, r):
        g = synth.rng(1300, "logits", r)
        b["logits"].copy_(torch.from_numpy((g.standard_normal((B, V)) * 3).astype(np.float32)).cuda())
        b["temp"].copy_(torch.from_numpy(g.uniform(0.5, 1.5, B).astype(np.float32)).cuda())
        b["top_p"].copy_(torch.from_numpy(g.uniform(0.5, 1.0, B).astype(np.float32)).cuda())
        b["top_k"].copy_(torch.from_numpy(np.array([0, 1, 5, 50, 0, 1000, 0, 7], np.int32)).cuda())
        b["u"].copy_(torch.from_numpy(g.uniform(0, 1, B).astype(np.float32)).cuda())

    fill(bufs[1], 99)
    call(bufs[1])
    torch.cuda.synchronize()
    g = capture(lambda s: call(bufs[0], s))
    for r in range(5):
        fill(bufs[0], r)
        fill(bufs[1], r)
        g.replay()
        call(bufs[1])
        torch.cuda.synchronize()
        assert torch.equal(bufs[0]["tok"], bufs[1]["tok"]), "replay %d differs from the eager call" % r


def test_prefill_replays_match_eager():
    """A 37-token prompt after 5 cached tokens, replayed with new prompts."""
    shape = synth.tiny_shape(hidden=128, layers=2, heads=4, kv_heads=2, inter=256, vocab=1000)
    start, T = 5, 37
    wl = synth.decode_workload("graph prefill", shape, 1400, [start + T - 1])
    weights = synth.model_weights(shape, 1400, sigma=0.05, norm_sigma=0.3)
    cfg = pkv.make_config(shape, max_pos=start + T)
    model = pkv.upload_model(weights, shape.theta, start + T)
    bts = dev(np.ascontiguousarray(wl.block_tables[:, 0]))
    pools = [dev(wl.pool) for _ in range(3)]
    P = [pkv.kv_pool_create(t, shape.kv_heads) for t in pools]
    ws = [pkv.alloc_workspace(pkv.prefill_workspace_bytes(cfg, T, bts.shape[1])) for _ in range(3)]
    logits = [torch.empty(shape.vocab, dtype=torch.float32, device="cuda") for _ in range(3)]
    nxt = [torch.empty(1, dtype=torch.int32, device="cuda") for _ in range(3)]
    tok_g = dev(np.zeros(T, np.int32))
    pkv.prefill(cfg, model, P[2], bts, start, tok_g, logits[2], nxt[2], ws[2])
    torch.cuda.synchronize()
    g = capture(lambda s: pkv.prefill(cfg, model, P[0], bts, start, tok_g, logits[0], nxt[0], ws[0], s))
    for r in range(3):
        toks = synth.rng(1400, "prompt", r).integers(0, shape.vocab, size=T).astype(np.int32)
        tok_g.copy_(torch.from_numpy(toks).cuda())
        g.replay()
        pkv.prefill(cfg, model, P[1], bts, start, dev(toks), logits[1], nxt[1], ws[1])
        assert pkv.device_error(ws[0]) == 0
        assert torch.equal(logits[0], logits[1]) and torch.equal(nxt[0], nxt[1]), "replay %d differs" % r
        assert np.array_equal(host_u16(pools[0]), host_u16(pools[1]))
