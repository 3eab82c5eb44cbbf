"""Write the stored oracle outputs of the full-size decode and prefill
workloads (tests/golden/*.npz).

This script calls nothing but the CPU oracle (``oracle``) and the seeded
input generators (``synth``); it never loads the HIP library.  The GPU tests
compare the HIP path with what it writes, for every sequence of:

  step_llama1b_b16   the benchmark's decode step: Llama-3.2-1B shape,
                     16 layers, batch 16, attention lengths U[1,2048] (seed 1002)
  step_llama1b_b64   Llama-3.2-1B shape, batch 64, contexts U[64,2048] (seed 1004)
  step_qwen05_b128   Qwen2.5-0.5B shape, 24 layers, batch 128, 4096 cached
                     tokens each (seed 1005)
  prefill_llama1b_t512  the benchmark's prefill: one 512-token prompt from
                     position 0 through the Llama-3.2-1B-shape model (weights
                     seed 1002, prompt and pool seed 1007)
  layer_llama8b_b16  one Llama-3-8B-shaped decoder layer (head width 128),
                     batch 16, contexts U[1,1024] (seed 1010)

What is stored per sequence (a decode step or layer) or for the prompt (prefill):
  * a layer: its whole output row and the new token's appended K and V (as
    for a step, one layer);
  * the oracle's argmax and the gap between its two largest logits;
  * the RMS of all logits, and the logits at a fixed sample of indices: the
    16 largest (descending, lower index first among equals) followed by 256
    evenly strided vocabulary indices (0, V // 256, 2 V // 256, ...);
  * for every layer, the new token's appended K and V (BF16 bits) at 64
    evenly strided positions of the [kv heads * head dim] vector, and the RMS
    of the whole appended K and V vectors.  For the prefill, layer 0's K and
    V of every prompt token (its inputs are exact embedding rows).

The decode steps run one oracle process per core over the sequences
(processes forked after the inputs are drawn).  The prefill is the oracle's
token-by-token definition (each token a decode step at its position whose
K/V are appended before the next token runs); since token t at layer l needs
only token t at layer l - 1 and tokens < t at layer l, the layers are split
over processes that pass each token's hidden state down a pipeline, every
process keeping its layers' contiguous caches.  A CPU test checks that this
pipeline gives exactly ``oracle.prefill_paged``'s results on a small model.

Usage:  python tests/golden/make_golden.py [--only NAME ...] [--procs N]
"""
import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

TOP = 16
STRIDED = 256
KV_SAMPLES = 64


def logit_sample_index(logits):
    """Top-16 indices (descending, lower index first among equals), then
    256 evenly strided indices."""
    V = logits.size
    order = np.lexsort((np.arange(V), -logits.astype(np.float64)))
    return np.concatenate([order[:TOP], np.arange(STRIDED, dtype=np.int64) * (V // STRIDED)]).astype(np.int32)


def kv_sample_index(kvd):
    return (np.arange(KV_SAMPLES, dtype=np.int64) * (kvd // KV_SAMPLES)).astype(np.int32)


def top2_gap(logits):
    t = np.sort(logits.astype(np.float64))[-2:]
    return float(t[1] - t[0])


def rms(a):
    a = np.asarray(a, dtype=np.float64)
    return float(np.sqrt(np.mean(a * a))) if a.size else 0.0


# ------------------------------------------------------------ decode ---

_STATE = None


def _one_sequence(b):
    shape, weights, wl = _STATE
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    logits, nxt, k_new, v_new = oracle.decode_step_paged(shape, weights, wl.pool, geo, wl.block_tables,
                                                         wl.positions, wl.extra["tokens"], seqs=[b])
    lg = logits[b]
    idx = logit_sample_index(lg)
    kvi = kv_sample_index(shape.kv_heads * shape.head_dim)
    kb = k_new[:, b, :]
    vb = v_new[:, b, :]
    return {
        "token": int(nxt[b]), "gap": top2_gap(lg), "logit_rms": rms(lg), "logit_idx": idx,
        "logit_val": lg[idx].astype(np.float32), "k": kb[:, kvi], "v": vb[:, kvi],
        "k_rms": np.array([rms(oracle.bf16_to_f32(kb[l])) for l in range(shape.layers)], np.float32),
        "v_rms": np.array([rms(oracle.bf16_to_f32(vb[l])) for l in range(shape.layers)], np.float32),
    }


def step_golden(wl, weights, procs, seqs=None):
    """Oracle outputs of a decode-step workload for `seqs` (default: all)."""
    import multiprocessing as mp
    global _STATE
    oracle._load()
    _STATE = (wl.shape, weights, wl)
    seqs = list(range(wl.batch)) if seqs is None else list(seqs)
    with mp.get_context("fork").Pool(procs) as pool:
        res = pool.map(_one_sequence, seqs, chunksize=1)
    out = {"seqs": np.asarray(seqs, np.int32),
           "kv_idx": kv_sample_index(wl.shape.kv_heads * wl.shape.head_dim)}
    for key in ("token", "gap", "logit_rms"):
        out[key] = np.asarray([r[key] for r in res], np.int32 if key == "token" else np.float64)
    for key in ("logit_idx", "logit_val", "k", "v", "k_rms", "v_rms"):
        out[key] = np.stack([r[key] for r in res])
    return out


def layer8b_inputs():
    """One Llama-3-8B-shaped layer (hidden 4096, 32/8 heads of width 128,
    SwiGLU 14336) at batch 16, positions U[0,1024) (seed 1010): (shape,
    workload, layer weights, hidden [16][4096])."""
    shape = synth.LLAMA8B
    batch, seed = 16, 1010
    positions = synth.rng(seed, "lens").integers(0, 1024, size=batch).astype(np.int32)
    wl = synth.decode_workload("d128 8b layer", shape, seed, positions, layers=1)
    lw = synth.layer_weights(shape, seed, 0)
    hidden = synth.rng(seed, "hidden").standard_normal((batch, shape.hidden)).astype(np.float32)
    return shape, wl, lw, hidden


_LSTATE = None


def _one_layer_sequence(b):
    shape, wl, lw, hidden = _LSTATE
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    out, k_new, v_new = oracle.layer_decode_paged(shape, lw, hidden, wl.pool, geo, wl.block_tables[0],
                                                  wl.positions, [b])
    kvi = kv_sample_index(shape.kv_heads * shape.head_dim)
    return {"out": out[b].astype(np.float32), "k": k_new[b][kvi], "v": v_new[b][kvi],
            "k_rms": np.float32(rms(oracle.bf16_to_f32(k_new[b]))),
            "v_rms": np.float32(rms(oracle.bf16_to_f32(v_new[b])))}


def layer_golden(shape, wl, lw, hidden, procs):
    """Oracle outputs of one decoder layer for every sequence."""
    import multiprocessing as mp
    global _LSTATE
    oracle._load()
    _LSTATE = (shape, wl, lw, hidden)
    with mp.get_context("fork").Pool(procs) as pool:
        res = pool.map(_one_layer_sequence, list(range(wl.batch)), chunksize=1)
    out = {"seqs": np.arange(wl.batch, dtype=np.int32), "kv_idx": kv_sample_index(shape.kv_heads * shape.head_dim),
           "positions": np.asarray(wl.positions, np.int32)}
    for key in ("out", "k", "v", "k_rms", "v_rms"):
        out[key] = np.stack([r[key] for r in res])
    return out


# ----------------------------------------------------------- prefill ---

def _prefill_stage(shape, weights, layers, pool, geo, bts, start, tokens, q_in, q_out, kv_out):
    """One pipeline stage: `layers` of the prompt's tokens in order.  Each
    layer's contiguous cache starts with the pool's tokens 0 .. start - 1
    and gains one BF16 row per prompt token (what the pool would hold)."""
    T = len(tokens)
    kvd = shape.kv_heads * shape.head_dim
    caches = {}
    for l in layers:
        kc = np.zeros((start + T, kvd), np.float32)
        vc = np.zeros((start + T, kvd), np.float32)
        if start > 0:
            kc[:start], vc[:start] = oracle.pool_gather(pool, geo, bts[l], start)
        caches[l] = (kc, vc)
    for t in range(T):
        p = start + t
        x = oracle.embed(weights["embed"], int(tokens[t])) if q_in is None else q_in.get()
        kv = []
        for l in layers:
            kc, vc = caches[l]
            x, kb, vb = oracle.layer_decode(shape, weights["layers"][l], x, kc, vc, p)
            kv.append((l, kb, vb))
        q_out.put(x)
        kv_out.put((t, kv))


def _stage_proc(args):
    _prefill_stage(*args)


def prefill_pipeline(shape, weights, pool, geo, bts, start, tokens, procs):
    """The oracle's prefill of one prompt, its layers split over `procs`
    processes.  Returns (last-token logits, argmax, k [L][T][kvd], v
    [L][T][kvd] BF16 bits of every prompt token's appended K/V)."""
    import multiprocessing as mp
    oracle._load()
    ctx = mp.get_context("fork")
    L, T = shape.layers, len(tokens)
    n = max(1, min(procs, L))
    groups = [list(range(i * L // n, (i + 1) * L // n)) for i in range(n)]
    qs = [ctx.Queue() for _ in range(n)]
    kvq = ctx.Queue()
    ps = []
    for i, g in enumerate(groups):
        q_in = None if i == 0 else qs[i - 1]
        p = ctx.Process(target=_stage_proc,
                        args=((shape, weights, g, pool, geo, bts, start, tokens, q_in, qs[i], kvq),))
        p.start()
        ps.append(p)
    kvd = shape.kv_heads * shape.head_dim
    k = np.zeros((L, T, kvd), np.uint16)
    v = np.zeros((L, T, kvd), np.uint16)
    x_last = None
    for t in range(T):
        x = qs[-1].get()
        if t == T - 1:
            x_last = x
    for _ in range(T * n):
        t, kv = kvq.get()
        for l, kb, vb in kv:
            k[l, t], v[l, t] = kb, vb
    for p in ps:
        p.join()
        if p.exitcode != 0:
            raise RuntimeError("prefill stage failed (exit code %s)" % p.exitcode)
    logits, best = oracle.lm_head(weights["embed"], weights["final_norm"], shape.eps, x_last)
    return logits, best, k, v


def prefill_golden(shape, weights, pool, bts, start, tokens, procs):
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    logits, best, k, v = prefill_pipeline(shape, weights, pool, geo, bts, start, tokens, procs)
    idx = logit_sample_index(logits)
    kvi = kv_sample_index(shape.kv_heads * shape.head_dim)
    return {"token": np.int32(best), "gap": top2_gap(logits), "logit_rms": rms(logits), "logit_idx": idx,
            "logit_val": logits[idx].astype(np.float32), "kv_idx": kvi, "k0": k[0][:, kvi], "v0": v[0][:, kvi],
            "k0_rms": np.array([rms(oracle.bf16_to_f32(k[0, t])) for t in range(len(tokens))], np.float32),
            "v0_rms": np.array([rms(oracle.bf16_to_f32(v[0, t])) for t in range(len(tokens))], np.float32),
            "start": np.int32(start), "tokens": np.asarray(tokens, np.int32)}


# ------------------------------------------------------------ workloads ---

def prefill_inputs(T=512):
    """The benchmark's prefill: Llama-3.2-1B shape, weights seed 1002, a
    fresh sequence's table and pool (seed 1007), prompt seed 1007."""
    shape = synth.LLAMA1B
    weights = synth.model_weights(shape, 1002)
    wl = synth.decode_workload("prefill", shape, 1007, [T - 1])
    tokens = synth.rng(1007, "prompt").integers(0, shape.vocab, size=T).astype(np.int32)
    return shape, weights, wl.pool, np.ascontiguousarray(wl.block_tables[:, 0]), tokens


STEPS = {
    "step_llama1b_b16": (lambda: synth.bench_step(), 1002),
    "step_llama1b_b64": (lambda: synth.llama1b_step_b64(), 1004),
    "step_qwen05_b128": (lambda: synth.qwen05_step_b128(), 1005),
}


def path_of(name):
    return os.path.join(HERE, name + ".npz")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--only", nargs="*", default=None)
    ap.add_argument("--procs", type=int, default=max(1, (os.cpu_count() or 2) - 1))
    args = ap.parse_args()
    names = list(STEPS) + ["prefill_llama1b_t512", "layer_llama8b_b16"]
    for name in names:
        if args.only and name not in args.only:
            continue
        t0 = time.time()
        if name in STEPS:
            mk, wseed = STEPS[name]
            wl = mk()
            weights = synth.model_weights(wl.shape, wseed)
            out = step_golden(wl, weights, args.procs)
            del wl
        elif name == "layer_llama8b_b16":
            shape, wl, lw, hidden = layer8b_inputs()
            out = layer_golden(shape, wl, lw, hidden, args.procs)
        else:
            shape, weights, pool, bts, tokens = prefill_inputs()
            out = prefill_golden(shape, weights, pool, bts, 0, tokens, args.procs)
        np.savez_compressed(path_of(name), **out)
        print("%s: %.0f s -> %s" % (name, time.time() - t0, path_of(name)), flush=True)


if __name__ == "__main__":
    main()
