#!/usr/bin/env python3
"""Decode-step benchmark of the gfx950 paged-KV GQA path (one GPU).

Workload: one batched decode step of a Llama-3.2-1B-shaped model (hidden
2048, 32 query / 8 kv heads, head_dim 64, SwiGLU 8192, 16 layers, tied
128256-token embedding / LM head with FP32 logits and argmax) at batch 16,
where the 16 sequences' attention lengths are the paged-attention
workload's draw (lengths uniform in [1, 2048], seed 1002), so that every
layer's attention call is exactly that workload.  Each (layer, sequence)
keeps its pages scattered in one shared BF16 pool of 16-token pages sized
to fit.  Weights N(0, 0.02) and cached K/V N(0, 1), BF16, seeded and
synthetic.  A "step" is one decode_step call (every row of the hot path:
embedding, 16 x [RMSNorm, QKV, RoPE, KV append, paged attention, O-proj +
residual, RMSNorm, SwiGLU, down + residual], final norm, LM head, argmax),
replayed from a HIP graph; inputs are resident in HBM before timing.

Reported (one JSON line): decode tokens/s for the step; the paged
attention call's achieved HBM GB/s against the 8 TB/s peak (its
algorithmic bytes over its average duration: the call's two kernels,
attention and split merge, replayed from a HIP graph over the 16 layers'
tables and timed with HIP events on that stream); the whole step's
algorithmic bytes over the step time; the batch-1 decoder layer (Llama
shape, context 1024) against its weight-streaming roofline; and the CPU
oracle timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
  python bench.py --attention-only   (the attention calls alone, launched
                                      one by one, then a 256 MiB device copy
                                      of known size: the run that rocprofv3
                                      counters are taken on)
  python bench.py --step-counters    (3 eager batch-16 steps, then the same
                                      copy: the step's counter runs)
  python bench.py --qwen-layer-counters
                                     (3 eager passes of the 16-layer batch-1
                                      Qwen chain, then the same copy)
  python bench.py --counter-table FETCH.csv WRITE.csv
                                     (every library kernel's scaled FETCH_SIZE
                                      and WRITE_SIZE per dispatch, markdown)
  python bench.py --traffic-summary FETCH.csv WRITE.csv
                                     (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
                                      counter_collection.csv files of two
                                      --attention-only runs -> the HBM
                                      traffic per attention call, scaled by
                                      what the copy reads, written to
                                      profiles/paged_attention_bench_traffic.json
                                      or --traffic-out PATH)
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s + paged-attn HBM GB/s (% of peak), Llama-1B shape, batch 16"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "paged_attention_bench_traffic.json")
ATTN_SOURCE = os.path.join(ROOT, "paged_kv_transformer_amd", "csrc", "attention.hip")
COPY_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attention_bytes(lens, Hq, Hkv, q_bytes, D=64, page_tokens=16):
    """Algorithmic bytes of one paged attention call: every attended token's
    K and V (BF16), q in, FP32 out, one block-table entry per page."""
    lens = np.asarray(lens, dtype=np.int64)
    B = len(lens)
    return int((lens * Hkv * D * 2 * 2).sum() + B * Hq * D * (q_bytes + 4)
               + ((lens + page_tokens - 1) // page_tokens).sum() * 4)


def decode_layer_bytes(shape, lens):
    """Algorithmic bytes of one decoder layer over a batch: the weights once,
    the attention (FP32 q inside the layer) over lens[b] tokens, the
    appended K/V and the hidden state in and out."""
    B, H = len(lens), shape.hidden
    return (2 * shape.layer_param_count()
            + attention_bytes(lens, shape.heads, shape.kv_heads, 4, shape.head_dim)
            + B * shape.kv_heads * shape.head_dim * 2 * 2 + 2 * B * H * 4)


def step_bytes(shape, lens, logits=True):
    """Algorithmic bytes of one decode step: weights once, each layer's
    attention (FP32 q inside the layer), the appended K/V, the hidden state
    in and out of each layer, the embedding rows, the LM head, the logits."""
    B, H, V = len(lens), shape.hidden, shape.vocab
    layer = decode_layer_bytes(shape, lens)
    return shape.layers * layer + B * H * 2 + 2 * V * H + H * 2 + (B * V * 4 if logits else 0)


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(bytes_per_launch):
    """HBM traffic per attention launch from the committed counter summary,
    or None if it is missing or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("attention_source_sha") != source_sha(ATTN_SOURCE):
        return None
    return {"fetch_bytes": t["fetch_bytes_per_launch"], "write_bytes": t["write_bytes_per_launch"],
            "total_bytes": t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"],
            "ratio_to_algorithmic": (t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"])
            / bytes_per_launch,
            "source": os.path.relpath(TRAFFIC_FILE, ROOT)}


class HostInputs:
    """The workload's host arrays (drawn before the GPU is touched, so the
    oracle's worker processes can be forked from a GPU-free process)."""

    def __init__(self, synth):
        t0 = time.time()
        self.wl = synth.bench_step()
        self.shape = self.wl.shape
        self.weights = synth.model_weights(self.shape, 1002)
        log("inputs drawn in %.1fs (pool %d pages, %.0f MiB)" % (
            time.time() - t0, self.wl.num_pages, self.wl.pool.nbytes / 2 ** 20))


class Setup:
    """Device-resident inputs of the workload."""

    def __init__(self, torch, pkv, synth, host):
        wl, shape = host.wl, host.shape
        self.wl, self.shape = wl, shape
        self.weights = host.weights
        self.max_pos = int(wl.positions.max()) + 1
        self.cfg = pkv.make_config(shape, max_pos=self.max_pos)
        # RoPE tables for 4097 positions: the batch-64 step reuses this model
        self.model = pkv.upload_model(self.weights, shape.theta, max(self.max_pos, 4097))
        self.pool_t = pkv.to_device(wl.pool)
        self.pool = pkv.kv_pool_create(self.pool_t, shape.kv_heads)
        self.bts = pkv.to_device(wl.block_tables)
        self.pos = pkv.to_device(wl.positions)
        self.tokens = pkv.to_device(wl.extra["tokens"])
        B = wl.batch
        self.logits = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
        self.next = torch.empty(B, dtype=torch.int32, device="cuda")
        self.ws = pkv.alloc_workspace(pkv.workspace_bytes(self.cfg, B, wl.max_pages))
        torch.cuda.synchronize()

    def step(self, pkv):
        pkv.decode_step(self.cfg, self.model, self.pool, self.bts, self.pos, self.tokens, self.logits,
                        self.next, self.ws)


class AttentionCalls:
    """paged_gqa_decode over the step's 16 layers' block tables (distinct
    pages per layer), BF16 q, FP32 output."""

    def __init__(self, torch, pkv, synth, S):
        wl, shape = S.wl, S.shape
        B = wl.batch
        self.pkv, self.S = pkv, S
        self.q = pkv.to_device(synth.bf16_normal(1002, "q", (B, shape.heads, shape.head_dim)))
        self.lens = pkv.to_device(wl.lens)
        self.out = torch.empty((B, shape.heads, shape.head_dim), dtype=torch.float32, device="cuda")
        self.ws = pkv.alloc_workspace(pkv.attention_workspace_bytes(shape.heads, shape.kv_heads, B,
                                                                    wl.max_pages))
        self.bts = [S.bts[l].contiguous() for l in range(shape.layers)]
        self.layers = shape.layers

    def launch(self, l, stream):
        self.pkv.paged_gqa_decode(self.S.pool, self.q, self.bts[l], self.lens, 0.125, self.out, self.ws,
                                  stream)


def time_attention(torch, pkv, synth, S, rounds, reps=10):
    """Average duration (ms) of one paged_gqa_decode call: `rounds` passes
    over the 16 layers' tables captured in a HIP graph, replayed `reps`
    times between two HIP events on the replay stream."""
    A = AttentionCalls(torch, pkv, synth, S)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        for l in range(A.layers):
            A.launch(l, cap)
        cap.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(rounds):
                for l in range(A.layers):
                    A.launch(l, cap)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for _ in range(2):
        graph.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    assert pkv.device_error(A.ws) == 0
    return e0.elapsed_time(e1) / (reps * rounds * A.layers), reps * rounds * A.layers


def time_paged_read(torch, pkv, synth, S, rounds, reps=10):
    """Microseconds per pkv_probe_paged_read over the same 16 tables as
    time_attention (the attention call's K/V loads and grid, one launch, no
    arithmetic), replayed from a HIP graph."""
    A = AttentionCalls(torch, pkv, synth, S)
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")

    def run(st):
        for _ in range(rounds):
            for l in range(A.layers):
                pkv.probe_paged_read(S.pool, S.shape.heads, A.bts[l], A.lens, sink, stream=st)

    graph = capture(torch, run)
    graph.replay()
    ms = float(np.median(timed_replays(torch, graph.replay, reps)))
    return ms * 1e3 / (rounds * A.layers)


def cold_attention_us(torch, pkv, synth, S):
    """One paged_gqa_decode call on layer 0's table after a cache flush."""
    A = AttentionCalls(torch, pkv, synth, S)
    return cold_call_us(torch, lambda: A.launch(0, torch.cuda.current_stream()))


def time_layer_b1(torch, pkv, synth, S, reps=10):
    """Batch-1 decoder layer (the step's layer weights, context 1024): the
    16 layers' decoder_layer_decode calls captured in a HIP graph; returns
    (ms per layer, algorithmic bytes per layer)."""
    shape = S.shape
    wl = synth.llama1b_step_b1()
    pool_t = pkv.to_device(wl.pool)
    pool = pkv.kv_pool_create(pool_t, shape.kv_heads)
    bts = [pkv.to_device(wl.block_tables[l]) for l in range(shape.layers)]
    pos = pkv.to_device(wl.positions)
    hidden = torch.randn((1, shape.hidden), dtype=torch.float32, device="cuda")
    ws = pkv.alloc_workspace(pkv.workspace_bytes(S.cfg, 1, wl.max_pages))
    m = S.model

    def run(stream):
        for l in range(shape.layers):
            pkv.decoder_layer_decode(S.cfg, m.layers[l], m.rope_cos, m.rope_sin, pool, bts[l], pos, hidden,
                                     ws, stream)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        run(cap)
        cap.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            run(cap)
    torch.cuda.synchronize()
    for _ in range(2):
        graph.replay()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    assert pkv.device_error(ws) == 0
    n = int(wl.positions[0]) + 1
    layer_bytes = (2 * shape.layer_param_count() + attention_bytes([n - 1], shape.heads, shape.kv_heads, 4)
                   + shape.kv_heads * shape.head_dim * 2 * 2 + 2 * shape.hidden * 4)
    return e0.elapsed_time(e1) / (reps * shape.layers), layer_bytes


MFMA_BF16_PEAK_TFLOPS = 2500.0


def pct(xs):
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 4), "p50": round(float(np.percentile(a, 50)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def timed_replays(torch, run, reps):
    """Each replay between its own pair of events on the current stream: (ms list)."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        run()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def capture(torch, fn, keep=False):
    """fn(stream) run once eagerly, then captured in a HIP graph (keep: the
    graph itself is kept, so its nodes can be counted)."""
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph(keep_graph=True) if keep else torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        fn(cap)
        cap.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            fn(cap)
    if keep:
        graph.instantiate()
    torch.cuda.synchronize()
    return graph


def graph_nodes(graph):
    """Nodes of a graph captured with keep=True (every node here is one
    kernel launch), or None if the runtime cannot say."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        n = ctypes.c_size_t(0)
        rc = hip.hipGraphGetNodes(ctypes.c_void_p(graph.raw_cuda_graph()), None, ctypes.byref(n))
        return int(n.value) if rc == 0 else None
    except (OSError, AttributeError, RuntimeError):
        return None


def layer_bytes(shape, n_attend, q_bytes=4):
    """One decoder layer at batch 1 attending n_attend cached tokens plus the new one."""
    return (2 * shape.layer_param_count() + attention_bytes([n_attend + 1], shape.heads, shape.kv_heads, q_bytes)
            + shape.kv_heads * shape.head_dim * 2 * 2 + 2 * shape.hidden * 4)


def time_layer_qwen05_b1(torch, pkv, synth, reps=100, cold=False, fused=True):
    """The Qwen2.5-0.5B layer at batch 1, position 127, as a chain of 16
    distinct layers (16 weight draws, 16 page sets) in one HIP graph, so the
    layer's 30 MB are not served from the Infinity Cache; per-layer time =
    replay / 16.  fused: the single-launch layer (the library's default for
    this layer), else the multi-launch path.  Returns (list of per-layer ms
    per replay, bytes per layer, with cold=True the microseconds of one layer
    call after a cache flush (else None), kernel launches per layer)."""
    prev = pkv.set_fused_layer(fused)
    try:
        return _time_layer_qwen05_b1(torch, pkv, synth, reps, cold)
    finally:
        pkv.set_fused_layer(prev)


class QwenChain:
    """The Qwen2.5-0.5B layer at batch 1, position 127, as 16 distinct
    layers (weights, page sets) on the device; run(stream) calls
    decoder_layer_decode on each in turn."""
    L = 16

    def __init__(self, torch, pkv, synth):
        shape = self.shape = synth.QWEN05
        L = self.L
        wl = synth.decode_workload("qwen0.5b layer chain", shape, 1001, [127], layers=L)
        self.layers = [pkv.upload_layer(synth.layer_weights(shape, 1001, l)) for l in range(L)]
        self.c, self.sn = pkv.rope_table(shape.theta, 128)
        self.cfg = pkv.make_config(shape, max_pos=128, layers=1)
        self.pool_t = pkv.to_device(wl.pool)
        self.pool = pkv.kv_pool_create(self.pool_t, shape.kv_heads)
        self.bts = [pkv.to_device(wl.block_tables[l]) for l in range(L)]
        self.pos = pkv.to_device(wl.positions)
        self.hidden = torch.from_numpy(
            synth.rng(1001, "hidden").standard_normal((1, shape.hidden), dtype=np.float32)).cuda()
        self.ws = pkv.alloc_workspace(pkv.workspace_bytes(self.cfg, 1, wl.max_pages))
        self.pkv = pkv

    def call(self, l, stream=None):
        self.pkv.decoder_layer_decode(self.cfg, self.layers[l], self.c, self.sn, self.pool, self.bts[l], self.pos,
                                      self.hidden, self.ws, stream)

    def run(self, stream):
        for l in range(self.L):
            self.call(l, stream)


def qwen_layer_counters(torch, pkv, synth, passes=3):
    """Launch sequence for the hardware-counter runs of the batch-1 Qwen
    layer: `passes` eager passes over the 16-layer chain (single launch per
    layer), then the counters' calibration copy."""
    Q = QwenChain(torch, pkv, synth)
    for _ in range(passes):
        Q.run(None)
    torch.cuda.synchronize()
    assert pkv.device_error(Q.ws) == 0
    n = calibration_copies(torch)
    print("qwen-layer-counters: %d eager calls; copy calibration: 3 x %d bytes read + written"
          % (passes * Q.L, n), flush=True)


def _time_layer_qwen05_b1(torch, pkv, synth, reps, cold):
    Q = QwenChain(torch, pkv, synth)
    L = Q.L
    graph = capture(torch, Q.run, keep=True)
    nodes = graph_nodes(graph)
    for _ in range(20):
        graph.replay()
    ms = timed_replays(torch, graph.replay, reps)
    cold_us = None
    if cold:
        cold_us = cold_call_us(torch, lambda: Q.call(0))
    assert pkv.device_error(Q.ws) == 0
    return [m / L for m in ms], layer_bytes(Q.shape, 127), cold_us, (None if nodes is None else nodes / L)


def time_step_cfg(torch, pkv, synth, wl, shape, model, max_pos, reps=10):
    """decode_step of a workload in a HIP graph: (ms list, step bytes)."""
    cfg = pkv.make_config(shape, max_pos=max_pos)
    pool_t = pkv.to_device(wl.pool)
    pool = pkv.kv_pool_create(pool_t, shape.kv_heads)
    bts = pkv.to_device(wl.block_tables)
    pos = pkv.to_device(wl.positions)
    tok = pkv.to_device(wl.extra["tokens"])
    B = wl.batch
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = pkv.alloc_workspace(pkv.workspace_bytes(cfg, B, wl.max_pages))
    graph = capture(torch, lambda st: pkv.decode_step(cfg, model, pool, bts, pos, tok, logits, nxt, ws, st))
    for _ in range(2):
        graph.replay()
    ms = timed_replays(torch, graph.replay, reps)
    assert pkv.device_error(ws) == 0
    del pool_t
    return ms, step_bytes(shape, wl.lens)


def large_batch_steps(torch, pkv, synth, llama_model=None):
    """The batch-1 and batch-64 Llama steps and the batch-128 Qwen step:
    {name: object}."""
    out = {}
    for name, mk, shp, model_fn in (
            ("step_llama1b_b1", synth.llama1b_step_b1, synth.LLAMA1B,
             lambda: llama_model or pkv.upload_model(synth.model_weights(synth.LLAMA1B, 1002),
                                                     synth.LLAMA1B.theta, 4097)),
            ("step_llama1b_b64", synth.llama1b_step_b64, synth.LLAMA1B,
             lambda: llama_model or pkv.upload_model(synth.model_weights(synth.LLAMA1B, 1002),
                                                     synth.LLAMA1B.theta, 4097)),
            ("step_qwen05_b128", synth.qwen05_step_b128, synth.QWEN05,
             lambda: pkv.upload_model(synth.model_weights(synth.QWEN05, 1005), synth.QWEN05.theta, 4097))):
        wlx = mk()
        mp_ = int(wlx.positions.max()) + 1
        model = model_fn()
        xs, xb = time_step_cfg(torch, pkv, synth, wlx, shp, model, mp_)
        xm = float(np.median(xs))
        log("%s: %.3f ms per step (median), batch %d -> %.0f tokens/s, %.0f GB/s" % (
            name, xm, wlx.batch, wlx.batch / (xm * 1e-3), xb / (xm * 1e-3) / 1e9))
        out[name] = {"workload": wlx.name, "batch": int(wlx.batch), "ms_per_step": pct(xs),
                     "tokens_per_s": round(wlx.batch / (xm * 1e-3), 1), "bound": "hbm",
                     "algorithmic_bytes": int(xb), "achieved": round(xb / (xm * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(xb / (xm * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del model, wlx
        torch.cuda.empty_cache()
    return out


def page_geometries(torch, pkv, synth, rounds=4, reps=10, L=16):
    """paged_gqa_decode on the step's attention workload (batch 16, lengths
    U[1,2048], BF16 q) in every pool geometry: pages of 16 or 256 tokens,
    one buffer or separate K and V pools, at head width 64 (Llama-3.2-1B
    heads, 32/8) and 128 (Llama-3-8B heads, 32/8).  Each call reads one of L
    block tables with distinct pages (as the layers of a step do), so no
    call finds its pages in cache; rounds x L calls are captured in a HIP
    graph.  The pool holds seeded N(0,1) BF16 values drawn on the device.
    Returns {"d64": {geometry: object}, "d128": ...}."""
    out = {}
    lens = synth.attention_lens(1002, 16)
    B = len(lens)
    lens_t = pkv.to_device(lens)
    for shape in (synth.LLAMA1B, synth.LLAMA8B):
        D, Hq, Hkv = shape.head_dim, shape.heads, shape.kv_heads
        res = {}
        for PT in (16, 256):
            npages = int(synth.pages_for(lens, PT).sum()) * L
            bt = synth.block_tables(1002, L, lens, npages, max_pages=2048 // PT, page_tokens=PT)
            bts = [pkv.to_device(bt[l]) for l in range(L)]
            pe = synth.page_elems(shape, page_tokens=PT)
            abytes = attention_bytes(lens, Hq, Hkv, 2, D, PT)
            for split in (False, True):
                gen = torch.Generator(device="cuda").manual_seed(1002)
                if split:
                    kt = torch.randn(npages * pe // 2, generator=gen, device="cuda").to(torch.bfloat16)
                    vt = torch.randn(npages * pe // 2, generator=gen, device="cuda").to(torch.bfloat16)
                    pool = pkv.kv_pool_create_split(kt, vt, Hkv, head_dim=D, page_tokens=PT)
                else:
                    pt = torch.randn(npages * pe, generator=gen, device="cuda").to(torch.bfloat16)
                    pool = pkv.kv_pool_create(pt, Hkv, head_dim=D, page_tokens=PT)
                q = torch.randn((B, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
                o = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
                ws = pkv.alloc_workspace(pkv.attention_workspace_bytes(Hq, Hkv, B, bt.shape[2], head_dim=D,
                                                                       page_tokens=PT))

                def run(st):
                    for _ in range(rounds):
                        for l in range(L):
                            pkv.paged_gqa_decode(pool, q, bts[l], lens_t, 1.0 / np.sqrt(D), o, ws, st)

                graph = capture(torch, run)
                for _ in range(2):
                    graph.replay()
                ms = timed_replays(torch, graph.replay, reps)
                assert pkv.device_error(ws) == 0
                us = float(np.median(ms)) * 1e3 / (rounds * L)
                gbs = abytes / (us * 1e3)
                name = "pt%d_%s" % (PT, "split" if split else "whole")
                log("attention d%d %s: %.2f us per call, %.0f GB/s" % (D, name, us, gbs))
                res[name] = {"us_per_call": round(us, 3), "algorithmic_bytes": int(abytes),
                             "achieved": round(gbs, 1), "unit": "GB/s",
                             "frac": round(gbs / HBM_PEAK_GBS, 4)}
                del graph, pool, q, o, ws
                if split:
                    del kt, vt
                else:
                    del pt
                torch.cuda.empty_cache()
        out["d%d" % D] = res
    out["workload"] = ("paged_gqa_decode, 32/8 heads, batch 16, lengths U[1,2048] (seed 1002), "
                       "%d tables of distinct pages per graph pass; d64 Llama-3.2-1B heads, d128 "
                       "Llama-3-8B heads; pt16/pt256: page tokens; whole: K and V blocks in one "
                       "buffer, split: separate K and V pools" % L)
    out["peak"] = HBM_PEAK_GBS
    return out


def time_layer_llama8b(torch, pkv, synth, reps=10, L=4):
    """decoder_layer_decode of Llama-3-8B-shaped layers (hidden 4096, 32/8
    heads of width 128, SwiGLU 14336) at batch 16, attention lengths
    U[1,2048]: L distinct layers (weights and page sets) chained in one HIP
    graph, so the 436 MB of each layer's weights come from HBM.  Returns an
    object for the JSON line."""
    shape = synth.LLAMA8B
    lens = synth.attention_lens(1002, 16)
    positions = (lens - 1).astype(np.int32)
    wl = synth.decode_workload("8b layers", shape, 1010, positions, layers=L, with_pool=False)
    layers = [pkv.upload_layer(synth.layer_weights(shape, 1010, l), head_dim=128) for l in range(L)]
    mp = int(positions.max()) + 1
    c, sn = pkv.rope_table(shape.theta, mp, head_dim=128)
    cfg = pkv.make_config(shape, max_pos=mp, layers=1)
    gen = torch.Generator(device="cuda").manual_seed(1010)
    pool_t = torch.randn(wl.num_pages * synth.page_elems(shape), generator=gen,
                         device="cuda").to(torch.bfloat16)
    pool = pkv.kv_pool_create(pool_t, shape.kv_heads, head_dim=128)
    bts = [pkv.to_device(wl.block_tables[l]) for l in range(L)]
    pos = pkv.to_device(positions)
    B = len(positions)
    hidden = torch.randn((B, shape.hidden), generator=gen, device="cuda")
    ws = pkv.alloc_workspace(pkv.workspace_bytes(cfg, B, wl.max_pages))

    def run(stream):
        for l in range(L):
            pkv.decoder_layer_decode(cfg, layers[l], c, sn, pool, bts[l], pos, hidden, ws, stream)

    graph = capture(torch, run)
    for _ in range(2):
        graph.replay()
    ms = timed_replays(torch, graph.replay, reps)
    assert pkv.device_error(ws) == 0
    us = [m * 1e3 / L for m in ms]
    nbytes = decode_layer_bytes(shape, lens)
    gbs = nbytes / (float(np.median(us)) * 1e3)
    log("llama-8b-shape layer, batch 16: %.1f us per layer (median), %.1f MB -> %.0f GB/s" % (
        float(np.median(us)), nbytes / 1e6, gbs))
    del graph, layers, pool_t
    torch.cuda.empty_cache()
    return {"workload": "decoder_layer_decode, llama-3-8b-shape layer (head width 128), batch 16, "
                        "attention lengths U[1,2048] (seed 1002), %d distinct layers chained in one "
                        "HIP graph (per-layer = replay / %d)" % (L, L),
            "bound": "hbm", "algorithmic_bytes": int(nbytes), "us_per_layer": pct(us),
            "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def ceilings(torch, pkv, nbytes=1 << 30, reps=10):
    """Read ceilings of this GPU from the library's streaming-read probe (no
    arithmetic, non-temporal 16-byte loads): one launch over 1 GiB (best of
    several workgroup counts), and 32 launches of 32 MiB over distinct
    chunks of the same buffer in one HIP graph (a launch the size of the
    attention call, nothing cache-resident); a torch device copy (read +
    write) for context."""
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    best_wg, best_ms = None, None
    for wg in (512, 1024, 2048, 4096):
        pkv.probe_read(buf, sink, wg)
        ms = min(timed_replays(torch, lambda: pkv.probe_read(buf, sink, wg), reps))
        if best_ms is None or ms < best_ms:
            best_wg, best_ms = wg, ms
    chunk = 32 << 20
    parts = [buf[i * chunk:(i + 1) * chunk] for i in range(nbytes // chunk)]
    graph = capture(torch, lambda st: [pkv.probe_read(c, sink, best_wg, stream=st) for c in parts])
    graph.replay()
    per = min(timed_replays(torch, graph.replay, reps)) / len(parts)
    y = torch.empty_like(buf)
    y.copy_(buf)
    cp = min(timed_replays(torch, lambda: y.copy_(buf), reps))
    del buf, y, graph
    torch.cuda.empty_cache()
    return {"stream_read_gbs": round(nbytes / (best_ms * 1e-3) / 1e9, 1), "stream_read_workgroups": best_wg,
            "read_32mib_launch_us": round(per * 1e3, 3),
            "read_32mib_launch_gbs": round(chunk / (per * 1e-3) / 1e9, 1),
            "copy_gbs": round(2 * nbytes / (cp * 1e-3) / 1e9, 1),
            "note": "pkv_probe_read (one launch streaming 1 GiB; and 32 launches of 32 MiB over distinct "
                    "chunks in one HIP graph), best of %d; copy: torch, bytes read + written" % reps}


def launch_floor(torch, pkv, n=64, reps=10):
    """Microseconds per empty kernel (pkv_probe_empty) replayed n at a time
    from a HIP graph, for 1, 256 and 1024 one-wave workgroups."""
    out = {}
    for wg in (1, 256, 1024):
        graph = capture(torch, lambda st: pkv.probe_empty(n, wg, stream=st))
        graph.replay()
        ms = float(np.median(timed_replays(torch, graph.replay, reps)))
        out["wg%d" % wg] = round(ms * 1e3 / n, 3)
        del graph
    return out


def cold_call_us(torch, fn, reps=10, flush_bytes=1 << 30):
    """One call after a 1 GiB device write (outside the event interval)
    that evicts the Infinity Cache and L2: median microseconds."""
    flush = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    fn()
    times = []
    for i in range(reps):
        flush.fill_(i & 0xff)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    del flush
    torch.cuda.empty_cache()
    return round(float(np.median(times)), 3)


def time_sampling(torch, pkv, synth, S, rounds=8, reps=10):
    """sample_tokens on the step's own logits [B][V] (temperature 1, top-p
    0.9, no top-k, seeded draws), captured rounds times in a HIP graph;
    returns (us per call, algorithmic bytes per call)."""
    B, V = S.logits.shape
    r = synth.rng(1002, "sample")
    T = torch.ones(B, dtype=torch.float32, device="cuda")
    p = torch.full((B,), 0.9, dtype=torch.float32, device="cuda")
    k = torch.zeros(B, dtype=torch.int32, device="cuda")
    u = torch.from_numpy(r.random(size=B).astype(np.float32)).cuda()
    out = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = pkv.alloc_workspace(pkv.sample_workspace_bytes(B, V))
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        pkv.sample_tokens(S.logits, T, p, k, u, out, ws, cap)
        cap.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            for _ in range(rounds):
                pkv.sample_tokens(S.logits, T, p, k, u, out, ws, cap)
    torch.cuda.synchronize()
    graph.replay()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    # the logits once, the per-sequence parameters and the tokens
    return e0.elapsed_time(e1) * 1e3 / (reps * rounds), B * V * 4 + B * 4 * 5


def prefill_flops(shape, start, T):
    """Algorithmic FLOPs of one prefill: every prompt token through every
    layer's projections (2 per weight), causal attention (QK and PV, 2 each
    per head dim and attended key), and the LM head for the last token."""
    proj = 2 * (shape.layer_param_count() - 2 * shape.hidden) * T
    keys = sum(start + t + 1 for t in range(T))
    attn = 4 * shape.heads * shape.head_dim * keys
    return shape.layers * (proj + attn) + 2 * shape.vocab * shape.hidden


def time_prefill(torch, pkv, synth, S, T=512, reps=5):
    """One prompt of T tokens of a fresh sequence (positions 0..T-1), the
    step's model weights, captured in a HIP graph; returns (ms, flops)."""
    shape = S.shape
    wl = synth.decode_workload("prefill", shape, 1007, [T - 1])
    pool_t = pkv.to_device(wl.pool)
    pool = pkv.kv_pool_create(pool_t, shape.kv_heads)
    bts = pkv.to_device(np.ascontiguousarray(wl.block_tables[:, 0]))
    tokens = pkv.to_device(synth.rng(1007, "prompt").integers(0, shape.vocab, size=T).astype(np.int32))
    if T > S.max_pos:
        raise SystemExit("prefill of %d tokens exceeds the model's %d rotary positions" % (T, S.max_pos))
    cfg, model = S.cfg, S.model
    ws = pkv.alloc_workspace(pkv.prefill_workspace_bytes(cfg, T, bts.shape[1]))
    logits = torch.empty(shape.vocab, dtype=torch.float32, device="cuda")
    nxt = torch.empty(1, dtype=torch.int32, device="cuda")

    def run(stream):
        pkv.prefill(cfg, model, pool, bts, 0, tokens, logits, nxt, ws, stream)

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        run(cap)
        cap.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            run(cap)
    torch.cuda.synchronize()
    graph.replay()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    assert pkv.device_error(ws) == 0
    return e0.elapsed_time(e1) / reps, prefill_flops(shape, 0, T)


class PrefillSetup:
    """The step's model weights (same seed) without the decode workload."""

    def __init__(self, pkv, synth, T):
        self.shape = synth.LLAMA1B
        self.max_pos = T
        self.cfg = pkv.make_config(self.shape, max_pos=T)
        self.model = pkv.upload_model(synth.model_weights(self.shape, 1002), self.shape.theta, T)


def prefill_only(torch, pkv, synth, T):
    ms, flops = time_prefill(torch, pkv, synth, PrefillSetup(pkv, synth, T), T)
    tf = flops / (ms * 1e-3) / 1e12
    print(json.dumps({"prefill_tokens": T, "ms": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1),
                      "algorithmic_tflops": round(tf, 2), "frac_of_bf16_peak": round(tf / MFMA_BF16_PEAK_TFLOPS, 5)}))


_CPU_STATE = None


def _oracle_seq(b):
    """The oracle's full step for sequence b of the bench workload (worker)."""
    import oracle
    shape, weights, wl = _CPU_STATE[:3]
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    _, nxt, _, _ = oracle.decode_step_paged(shape, weights, wl.pool, geo, wl.block_tables,
                                            wl.positions, wl.extra["tokens"], seqs=[b])
    return int(nxt[b])


def _pin_core0():
    os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})


def _timed(fn, reps=1):
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def oracle_config_inputs(synth, shape_l):
    """Inputs of the per-workload oracle timings, drawn in this process
    before any worker is forked (torch's generator is not used after a
    fork)."""
    t0 = time.time()
    inp = {"qwen_layer": synth.qwen05_layer_b1(), "attention": synth.attention_workload()}
    inp["llama_b1"] = synth.decode_workload("llama b1 sample", shape_l, 1004, [1023])
    inp["llama_b64"] = synth.decode_workload("llama b64 sample", shape_l, 1004,
                                             list(synth.llama1b_b64_positions()[:2]))
    inp["qwen_weights"] = synth.model_weights(synth.QWEN05, 1005)
    inp["qwen_b128"] = synth.decode_workload("qwen b128 sample", synth.QWEN05, 1005, [4096, 4096])
    log("oracle timing inputs drawn in %.1fs" % (time.time() - t0))
    return inp


def _oracle_configs(_arg=None):
    """The oracle timed on each workload of the set (worker, one core):
    seconds per call or step and what was timed."""
    import oracle
    import synth
    shape_l, weights_l, inp = _CPU_STATE[0], _CPU_STATE[1], _CPU_STATE[3]
    out = {}
    wl = inp["qwen_layer"]
    geo = oracle.PoolGeometry(wl.shape.kv_heads, wl.shape.head_dim)
    t = _timed(lambda: oracle.layer_decode_paged(wl.shape, wl.extra["weights"], wl.extra["hidden"], wl.pool, geo,
                                                 wl.block_tables[0], wl.positions), reps=5)
    out["layer_qwen05_b1"] = {"seconds": round(t, 4), "tokens_per_s": round(1 / t, 2),
                              "sample": "the whole layer (median of 5)"}
    log("  oracle: qwen layer %.3fs" % t)
    w = inp["attention"]
    geo = oracle.PoolGeometry(8, 64)
    q = oracle.bf16_to_f32(w["q"])
    t = _timed(lambda: oracle.paged_attention(w["pool"], geo, q, w["block_table"], w["lens"], w["scale"]))
    out["paged_attention_b16"] = {"seconds": round(t, 4), "calls_per_s": round(1 / t, 3),
                                  "sample": "the whole call (16 sequences)"}
    log("  oracle: attention call %.3fs" % t)
    geo = oracle.PoolGeometry(shape_l.kv_heads, shape_l.head_dim)
    for name, key in (("step_llama1b_b1", "llama_b1"), ("step_llama1b_b64", "llama_b64")):
        wl = inp[key]
        n = len(wl.positions)
        toks = np.zeros(n, np.int32)
        t = _timed(lambda: oracle.decode_step_paged(shape_l, weights_l, wl.pool, geo, wl.block_tables,
                                                    wl.positions, toks))
        out[name] = {"seconds_per_sequence": round(t / n, 3), "tokens_per_s": round(n / t, 4),
                     "sample": "%d sequence(s) at positions %s through all 16 layers, LM head and argmax%s" % (
                         n, [int(p) for p in wl.positions],
                         "" if n == 1 else " (of the 64: per-sequence time scales linearly)")}
        log("  oracle: %s %.2fs" % (name, t))
    shape_q = synth.QWEN05
    wl = inp["qwen_b128"]
    geo = oracle.PoolGeometry(shape_q.kv_heads, shape_q.head_dim)
    toks = np.zeros(2, np.int32)
    t = _timed(lambda: oracle.decode_step_paged(shape_q, inp["qwen_weights"], wl.pool, geo, wl.block_tables,
                                                wl.positions, toks))
    out["step_qwen05_b128"] = {"seconds_per_sequence": round(t / 2, 3), "tokens_per_s": round(2 / t, 4),
                               "sample": "2 sequences at 4096 cached tokens through all 24 layers, LM head and "
                                         "argmax (of the 128: per-sequence time scales linearly)"}
    log("  oracle: step_qwen05_b128 %.2fs" % t)
    return out


def host_description():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model}


def cpu_baseline(host, single_seqs, synth_mod):
    """The oracle on this host's cores, in forked worker processes: one
    process pinned to one core over `single_seqs` sequences, then one process
    per core (at most 16) over every sequence of the batch.  Returns
    (single seconds, tokens), (all-cores seconds, processes, tokens), and
    the oracle's time on every workload of the set (one core)."""
    import multiprocessing as mp
    import oracle
    global _CPU_STATE
    oracle._load()  # build / load the C oracle once, before forking
    inp = oracle_config_inputs(synth_mod, host.shape)
    _CPU_STATE = (host.shape, host.weights, host.wl, inp)
    ctx = mp.get_context("fork")
    with ctx.Pool(1, initializer=_pin_core0) as pool:
        t0 = time.perf_counter()
        single = pool.map(_oracle_seq, single_seqs, chunksize=1)
        d1 = time.perf_counter() - t0
        per_config = pool.map(_oracle_configs, [None])[0]
    B = host.wl.batch
    n = max(1, min(16, len(os.sched_getaffinity(0)), B))
    with ctx.Pool(n) as pool:
        t0 = time.perf_counter()
        allt = pool.map(_oracle_seq, range(B), chunksize=1)
        dn = time.perf_counter() - t0
    return (d1, single), (dn, n, allt), per_config


def calibration_copies(torch):
    """Three device copies of COPY_BYTES (the hardware counters' scale:
    what FETCH_SIZE and WRITE_SIZE read for a known number of bytes)."""
    n = COPY_BYTES
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    return n


def attention_only(torch, pkv, synth, rounds):
    """Launch sequence for the hardware-counter runs: the attention calls
    over the 16 layers' tables, one by one, then a device copy of known
    size (the counters' calibration)."""
    S = Setup(torch, pkv, synth, HostInputs(synth))
    A = AttentionCalls(torch, pkv, synth, S)
    stream = torch.cuda.current_stream()
    for _ in range(rounds):
        for l in range(A.layers):
            A.launch(l, stream)
    torch.cuda.synchronize()
    assert pkv.device_error(A.ws) == 0
    n = calibration_copies(torch)
    abytes = attention_bytes(S.wl.lens, S.shape.heads, S.shape.kv_heads, 2)
    print("attention-only: %d calls, %d algorithmic bytes per call; copy calibration: 3 x %d bytes "
          "read + written" % (rounds * A.layers, abytes, n), flush=True)


def step_counters(torch, pkv, synth, steps=3):
    """Launch sequence for the hardware-counter runs of the step: `steps`
    eager decode steps of the batch-16 workload (each kernel its own
    dispatch), then the counters' calibration copy."""
    S = Setup(torch, pkv, synth, HostInputs(synth))
    for _ in range(steps):
        S.step(pkv)
    torch.cuda.synchronize()
    assert pkv.device_error(S.ws) == 0
    n = calibration_copies(torch)
    print("step-counters: %d eager steps; copy calibration: 3 x %d bytes read + written" % (steps, n),
          flush=True)


def decode_only(torch, pkv, synth, args):
    """The batch-16 step, the attention call and the two batch-1 layers,
    each from a HIP graph (a quick line for tuning and profiling)."""
    S = Setup(torch, pkv, synth, HostInputs(synth))
    graph = capture(torch, lambda st: pkv.decode_step(S.cfg, S.model, S.pool, S.bts, S.pos, S.tokens, S.logits,
                                                      S.next, S.ws, st))
    for _ in range(20):
        graph.replay()
    step = float(np.median(timed_replays(torch, graph.replay, 100)))
    attn_ms, _ = time_attention(torch, pkv, synth, S, args.attn_rounds)
    l_ms, _ = time_layer_b1(torch, pkv, synth, S)
    lq_ms, _, _, lq_n = time_layer_qwen05_b1(torch, pkv, synth)
    lm_ms, _, _, _ = time_layer_qwen05_b1(torch, pkv, synth, fused=False)
    samp_us, _ = time_sampling(torch, pkv, synth, S)
    wl1 = synth.llama1b_step_b1()
    s1, _ = time_step_cfg(torch, pkv, synth, wl1, synth.LLAMA1B, S.model, int(wl1.positions.max()) + 1)
    out = {"step_b16_ms": round(step, 4), "attention_us": round(attn_ms * 1e3, 3), "sampling_us": round(samp_us, 2),
           "layer_llama1b_b1_us": round(l_ms * 1e3, 3), "layer_qwen05_b1_us": round(float(np.median(lq_ms)) * 1e3, 3),
           "qwen_launches_per_layer": lq_n, "layer_qwen05_b1_multi_launch_us": round(float(np.median(lm_ms)) * 1e3, 3),
           "step_llama1b_b1_ms": round(float(np.median(s1)), 4)}
    assert pkv.device_error(S.ws) == 0
    print(json.dumps(out), flush=True)


def counter_table(fetch_csv, write_csv):
    """Every library kernel's FETCH_SIZE and WRITE_SIZE per dispatch, each
    scaled by what the counter reads for the calibration copy, as a
    markdown table (MB per dispatch)."""
    rows = {}
    for cname, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = _counter_values(path)
        copy = [max(v) for (k, c), v in vals.items() if c == cname and "copyBuffer" in k]
        assert copy, "no device copy in %s" % path
        scale = COPY_BYTES / (max(copy) * 1024.0)
        for (k, c), v in vals.items():
            if c != cname or "pkv::" not in k:
                continue
            short = k.replace("pkv::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            r = rows.setdefault(short, {})
            r["n"] = len(v)
            r[cname] = sum(v) / len(v) * 1024.0 * scale / 1e6
    print("| kernel | dispatches | fetch MB / dispatch | write MB / dispatch |")
    print("|---|---:|---:|---:|")
    for k, r in sorted(rows.items(), key=lambda kv: -kv[1].get("FETCH_SIZE", 0.0) * kv[1]["n"]):
        print("| %s | %d | %.3f | %.3f |" % (k, r["n"], r.get("FETCH_SIZE", 0.0), r.get("WRITE_SIZE", 0.0)))


def _counter_values(path):
    """Counter values per (kernel name, counter) from a rocprofv3
    counter_collection.csv (one row per dispatch and counter)."""
    import csv
    vals = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            key = (row.get("Kernel_Name", ""), row.get("Counter_Name", ""))
            vals.setdefault(key, []).append(float(row["Counter_Value"]))
    return vals


def traffic_summary(fetch_csv, write_csv, out_path=TRAFFIC_FILE):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the attention
    kernels, scaled by what the same counters read for the 256 MiB copy,
    summed per paged_gqa_decode call -> TRAFFIC_FILE."""
    out = {"attention_source_sha": source_sha(ATTN_SOURCE), "copy_bytes": COPY_BYTES}
    for cname, path, key in (("FETCH_SIZE", fetch_csv, "fetch"), ("WRITE_SIZE", write_csv, "write")):
        vals = _counter_values(path)
        # the calibration copy is the largest device copy of the run
        copy = [max(v) for (k, c), v in vals.items() if c == cname and "copyBuffer" in k]
        assert copy, "no device copy in %s" % path
        copy_kib = max(copy)
        scale = COPY_BYTES / (copy_kib * 1024.0)
        per_call = 0.0
        kernels = {}
        for (k, c), v in vals.items():
            if c != cname:
                continue
            short = k.replace("pkv::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            if short.startswith("paged_attention_kernel") or short.startswith("attention_merge_kernel"):
                m = sum(v) / len(v)
                kernels[short] = {"mean_kib_per_dispatch": round(m, 1), "dispatches": len(v),
                                  "bytes_scaled": round(m * 1024.0 * scale)}
                per_call += m * 1024.0 * scale
        out[key + "_copy_kib"] = round(copy_kib, 1)
        out[key + "_scale"] = round(scale, 4)
        out[key + "_kernels"] = kernels
        out[key + "_bytes_per_launch"] = int(round(per_call))
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--attn-rounds", type=int, default=4)
    ap.add_argument("--cpu-seqs", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch the step directly, no HIP graph")
    ap.add_argument("--attention-only", action="store_true")
    ap.add_argument("--step-counters", action="store_true",
                    help="3 eager batch-16 steps and the calibration copy (for counter runs)")
    ap.add_argument("--counter-table", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="per-kernel scaled FETCH_SIZE / WRITE_SIZE of a counter run")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--traffic-out", default=TRAFFIC_FILE)
    ap.add_argument("--no-layer-b1", action="store_true")
    ap.add_argument("--large-batch-only", action="store_true",
                    help="time the batch-64 and batch-128 steps alone (for profiling)")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="skip the qwen0.5b layer chain, the batch-64/128 steps and the copy ceilings")
    ap.add_argument("--prefill-tokens", type=int, default=512, help="0 skips the prefill timing")
    ap.add_argument("--variants-only", action="store_true",
                    help="time the page-geometry variants and the head-width-128 layer alone")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time the prefill alone (the step's model, no decode workload)")
    ap.add_argument("--qwen-layer-counters", action="store_true",
                    help="3 eager passes of the batch-1 Qwen layer chain and the calibration copy (counter runs)")
    ap.add_argument("--qwen-layer-only", action="store_true",
                    help="time the qwen2.5-0.5b-shape batch-1 layer chain alone (for profiling)")
    ap.add_argument("--decode-only", action="store_true",
                    help="time the batch-16 step, the attention call and the batch-1 layers alone")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary, out_path=args.traffic_out)
        return
    if args.counter_table:
        counter_table(*args.counter_table)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only (the path runs on a single MI355X); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_transformer_amd as pkv
    import synth

    if (args.attention_only or args.prefill_only or args.large_batch_only or args.variants_only
            or args.step_counters or args.qwen_layer_only or args.decode_only or args.qwen_layer_counters):
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(2)
        torch.cuda.set_device(0)
        if args.attention_only:
            attention_only(torch, pkv, synth, args.attn_rounds)
        elif args.step_counters:
            step_counters(torch, pkv, synth)
        elif args.qwen_layer_counters:
            qwen_layer_counters(torch, pkv, synth)
        elif args.prefill_only:
            prefill_only(torch, pkv, synth, args.prefill_tokens)
        elif args.decode_only:
            decode_only(torch, pkv, synth, args)
        elif args.qwen_layer_only:
            lq_ms, lq_bytes, _, lq_n = time_layer_qwen05_b1(torch, pkv, synth)
            lm_ms, _, _, lm_n = time_layer_qwen05_b1(torch, pkv, synth, fused=False)
            lq_us = float(np.median(lq_ms)) * 1e3
            print(json.dumps({"layer_qwen05_b1_us": round(lq_us, 3), "algorithmic_bytes": int(lq_bytes),
                              "achieved_gbs": round(lq_bytes / (lq_us * 1e3), 1), "launches_per_layer": lq_n,
                              "multi_launch_us": round(float(np.median(lm_ms)) * 1e3, 3),
                              "multi_launch_launches_per_layer": lm_n}),
                  flush=True)
            n = calibration_copies(torch)
            print("copy calibration: 3 x %d bytes read + written" % n, flush=True)
        elif args.variants_only:
            print(json.dumps({"page_geometry": page_geometries(torch, pkv, synth),
                              "layer_llama8b": time_layer_llama8b(torch, pkv, synth)}))
        else:
            print(json.dumps(large_batch_steps(torch, pkv, synth)))
        return

    host = HostInputs(synth)
    cpu = None
    if not args.no_cpu_baseline:
        # the oracle first, in processes forked before this one touches the GPU
        single_seqs = list(range(min(args.cpu_seqs, host.wl.batch)))
        cpu = cpu_baseline(host, single_seqs, synth)
        log("oracle: %d sequences on 1 core in %.1fs; %d sequences on %d processes in %.1fs; per workload %s" % (
            len(single_seqs), cpu[0][0], host.wl.batch, cpu[1][1], cpu[1][0], cpu[2]))
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    S = Setup(torch, pkv, synth, host)
    shape, wl = S.shape, S.wl
    B = wl.batch

    # reference tokens from one eager step
    S.step(pkv)
    torch.cuda.synchronize()
    assert pkv.device_error(S.ws) == 0
    ref_next = S.next.clone()

    if args.eager:
        run = lambda: S.step(pkv)
    else:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                S.step(pkv)
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        run = graph.replay

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    log("step: %.3f ms (events), %.3f ms (wall)" % (ms, wall * 1e3 / args.steps))
    # percentiles over 100 single replays, after 20 more warm-up replays
    for _ in range(20):
        run()
    step_pct = pct(timed_replays(torch, run, max(args.steps, 100)))
    assert pkv.device_error(S.ws) == 0
    assert torch.equal(S.next, ref_next), "replayed steps changed the next tokens"

    # paged attention call: achieved HBM rate against the peak
    attn_ms, calls = time_attention(torch, pkv, synth, S, args.attn_rounds)
    abytes = attention_bytes(wl.lens, shape.heads, shape.kv_heads, 2)
    achieved = abytes / (attn_ms * 1e-3) / 1e9
    log("attention: %.2f us per call (graph, %d calls), %.1f MB -> %.0f GB/s" % (
        attn_ms * 1e3, calls, abytes / 1e6, achieved))
    floor = launch_floor(torch, pkv)
    pr_us = time_paged_read(torch, pkv, synth, S, args.attn_rounds)
    attn_cold = cold_attention_us(torch, pkv, synth, S)
    log("launch floor (us per empty launch, by workgroups): %s; paged-read probe %.2f us per call; "
        "cold single attention call %.2f us" % (floor, pr_us, attn_cold))
    sbytes = step_bytes(shape, wl.lens)
    step_gbs = sbytes / (ms * 1e-3) / 1e9
    layer_b1 = None
    if not args.no_layer_b1:
        l_ms, l_bytes = time_layer_b1(torch, pkv, synth, S)
        l_gbs = l_bytes / (l_ms * 1e-3) / 1e9
        log("batch-1 layer: %.2f us, %.1f MB -> %.0f GB/s" % (l_ms * 1e3, l_bytes / 1e6, l_gbs))
        layer_b1 = {"workload": "decoder_layer_decode, llama-3.2-1b-shape layer, batch 1, context 1024, "
                                "16 layers' weights in turn (HIP graph)",
                    "bound": "hbm", "algorithmic_bytes": int(l_bytes), "us_per_layer": round(l_ms * 1e3, 3),
                    "achieved": round(l_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(l_gbs / HBM_PEAK_GBS, 4)}

    s_us, s_bytes = time_sampling(torch, pkv, synth, S)
    log("sampling: %.2f us per call (graph), %.1f MB -> %.0f GB/s" % (s_us, s_bytes / 1e6, s_bytes / (s_us * 1e3)))
    sampling = {"workload": "sample_tokens on the step's logits, %d x %d FP32, temperature 1, top-p 0.9, "
                            "HIP graph" % tuple(S.logits.shape),
                "us": round(s_us, 3), "bound": "hbm", "algorithmic_bytes": s_bytes,
                "achieved": round(s_bytes / (s_us * 1e3), 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(s_bytes / (s_us * 1e3) / HBM_PEAK_GBS, 5)}

    extra = {}
    if not args.no_extra_configs:
        lq_ms, lq_bytes, lq_cold, lq_n = time_layer_qwen05_b1(torch, pkv, synth, cold=True)
        lm_ms, _, _, lm_n = time_layer_qwen05_b1(torch, pkv, synth, fused=False)
        lq_us = float(np.median(lq_ms)) * 1e3
        log("qwen0.5b layer chain, multi-launch path: %.2f us per layer, %s launches per layer" % (
            float(np.median(lm_ms)) * 1e3, lm_n))
        lq_gbs = lq_bytes / (lq_us * 1e3)
        lq_floor = None if lq_n is None else round(lq_n * floor["wg256"], 3)
        log("qwen0.5b layer chain: %.2f us per layer (median), %.2f MB -> %.0f GB/s; %s launches per layer, "
            "floor %s us; cold single layer %.2f us" % (lq_us, lq_bytes / 1e6, lq_gbs, lq_n, lq_floor, lq_cold))
        extra["layer_qwen05_b1"] = {
            "workload": "decoder_layer_decode, qwen2.5-0.5b-shape layer, batch 1, position 127, "
                        "16 distinct layers chained in one HIP graph (per-layer = replay / 16)",
            "bound": "hbm", "algorithmic_bytes": int(lq_bytes), "us_per_layer": pct([m * 1e3 for m in lq_ms]),
            "achieved": round(lq_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(lq_gbs / HBM_PEAK_GBS, 4), "gate_frac": 0.6,
            "launches_per_layer": lq_n, "launch_floor_us": lq_floor,
            "data_time_at_stream_ceiling_us": None,
            "cold_single_call_us": lq_cold,
            "multi_launch": {"us_per_layer": pct([m * 1e3 for m in lm_ms]), "launches_per_layer": lm_n},
            "note": "the single-launch layer (one workgroup per compute unit); multi_launch: the same "
                    "chain through the six-kernel path (pkv_set_fused_layer(0)); launch_floor_us = launches "
                    "per layer x one empty launch of 256 workgroups in a graph; cold_single_call_us: one "
                    "layer call after a 1 GiB device write"}
        extra.update(large_batch_steps(torch, pkv, synth, S.model))
        extra["page_geometry"] = page_geometries(torch, pkv, synth)
        extra["layer_llama8b"] = time_layer_llama8b(torch, pkv, synth)
        ceil = ceilings(torch, pkv)
        log("ceilings: %s" % ceil)
        extra["ceiling"] = ceil
        extra["launch_floor_us"] = floor
        if extra["layer_qwen05_b1"]["launches_per_layer"] is not None:
            extra["layer_qwen05_b1"]["data_time_at_stream_ceiling_us"] = round(
                lq_bytes / (ceil["stream_read_gbs"] * 1e3), 3)

    prefill = None
    if args.prefill_tokens > 0:
        p_ms, p_flops = time_prefill(torch, pkv, synth, S, args.prefill_tokens)
        p_tf = p_flops / (p_ms * 1e-3) / 1e12
        log("prefill: %d tokens in %.3f ms (%.0f tokens/s), %.2f TFLOP/s" % (
            args.prefill_tokens, p_ms, args.prefill_tokens / (p_ms * 1e-3), p_tf))
        prefill = {"workload": "prefill of one %d-token prompt from position 0, llama-3.2-1b-shape, "
                               "HIP graph" % args.prefill_tokens,
                   "tokens_per_s": round(args.prefill_tokens / (p_ms * 1e-3), 1), "ms": round(p_ms, 3),
                   "bound": "mfma", "algorithmic_flops": int(p_flops), "achieved": round(p_tf, 2),
                   "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                   "frac": round(p_tf / MFMA_BF16_PEAK_TFLOPS, 5)}

    result = {
        "metric": METRIC,
        "value": round(B / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) BF16 weights, N(0,1) BF16 KV pool, random page tables)",
        "config": {
            "workload": "llama-3.2-1b-shape 16-layer decode step, batch 16, attention lengths "
                        "U[1,2048] (seed 1002 draw), 16-token pages scattered in one shared BF16 pool",
            "batch": B, "layers": shape.layers, "hidden": shape.hidden, "heads": shape.heads,
            "kv_heads": shape.kv_heads, "head_dim": shape.head_dim, "intermediate": shape.inter,
            "vocab": shape.vocab, "context_lens": [int(x) for x in wl.lens],
            "pool_pages": int(wl.num_pages), "page_tokens": 16, "hip_graph": not args.eager,
        },
        "roofline": {
            "kernel": "paged_gqa_decode (paged_attention_kernel + attention_merge_kernel) on each "
                      "layer's tables",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": load_traffic(abytes),
            "algorithmic_bytes_per_launch": abytes,
            "avg_launch_us": round(attn_ms * 1e3, 3),
            "launches": int(calls),
            "attainable": {
                "paged_read_probe_us": round(pr_us, 3),
                "paged_read_probe_gbs": round(abytes / (pr_us * 1e3), 1),
                "two_launch_floor_us": round(2 * floor["wg256"], 3),
                "frac_of_paged_read_probe": round(pr_us / (attn_ms * 1e3), 4),
                "cold_single_call_us": attn_cold,
                "note": "paged_read_probe: pkv_probe_paged_read, the call's K/V loads and grid in one launch "
                        "without arithmetic, over the same 16 tables in a HIP graph; two_launch_floor: two empty "
                        "launches of 256 workgroups; cold_single_call: one call after a 1 GiB device write",
            },
        },
        "step_roofline": {
            "bound": "hbm", "algorithmic_bytes": int(sbytes), "achieved": round(step_gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4),
        },
        "step_ms_percentiles": step_pct,
        "layer_b1_roofline": layer_b1,
        "prefill": prefill,
        "sampling": sampling,
        **extra,
        "cpu_baseline": None,
    }

    if cpu is not None:
        (d1, single), (dn, n, allt), per_config = cpu
        seqs = list(range(len(single)))
        got = S.next.cpu().numpy()
        log("oracle tokens %s vs GPU %s" % (allt, got.tolist()))
        result["cpu_baseline"] = {
            "value": round(len(seqs) / d1, 4), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": "the full 16-layer step (embedding, layers, LM head, argmax) for sequences %s "
                      "of the batch, single-threaded FP32 C oracle in one process pinned to one core; "
                      "%.1f s" % (seqs, d1),
            "all_cores": {"value": round(len(allt) / dn, 4), "unit": "tokens/s", "cores": n,
                          "sample": "all %d sequences of the step, one oracle process per core, %.1f s"
                                    % (len(allt), dn)},
            "oracle_matches_gpu_tokens": int(sum(int(a == b) for a, b in zip(allt, got.tolist()))),
            "per_workload_one_core": per_config,
            "host": host_description(),
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
