"""The stored oracle outputs (tests/golden/*.npz) and the script that writes
them, checked on the CPU against the oracle itself:
  * the pipelined prefill of make_golden.py (layers split over processes)
    gives exactly oracle.prefill_paged's logits, argmax and appended K/V;
  * sequences of the stored benchmark step recomputed by the oracle give
    exactly the stored values;
  * every stored file holds every sequence of its workload, and the
    prefill's stored prompt is the benchmark's;
  * a sequence of the stored Llama-3-8B-shaped layer recomputed by the
    oracle gives exactly the stored output and K/V samples."""
import numpy as np
import pytest

import oracle
import synth
from golden import make_golden


def test_pipelined_prefill_equals_the_oracle_definition():
    shape = synth.tiny_shape(hidden=128, layers=5, heads=4, kv_heads=2, inter=256, vocab=1000)
    w = synth.model_weights(shape, 3, sigma=0.05, norm_sigma=0.3)
    start, T = 7, 30
    wl = synth.decode_workload("p", shape, 3, [start + T - 1])
    bts = np.ascontiguousarray(wl.block_tables[:, 0])
    tokens = synth.rng(3, "prompt").integers(0, shape.vocab, size=T).astype(np.int32)
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    lg, best, k, v = make_golden.prefill_pipeline(shape, w, wl.pool, geo, bts, start, tokens, 3)
    ref, rtok, rpool = oracle.prefill_paged(shape, w, wl.pool, geo, bts, start, tokens)
    assert np.array_equal(lg, ref) and best == rtok
    for l in range(shape.layers):
        kc, vc = oracle.pool_gather(rpool, geo, bts[l], start + T)
        assert np.array_equal(oracle.f32_to_bf16(kc[start:]), k[l])
        assert np.array_equal(oracle.f32_to_bf16(vc[start:]), v[l])


@pytest.mark.parametrize("name,batch", [("step_llama1b_b16", 16), ("step_llama1b_b64", 64),
                                        ("step_qwen05_b128", 128)])
def test_stored_step_holds_every_sequence(name, batch):
    g = np.load(make_golden.path_of(name), allow_pickle=False)
    assert list(g["seqs"]) == list(range(batch))
    assert g["logit_idx"].shape == (batch, make_golden.TOP + make_golden.STRIDED)
    assert np.all(np.diff(g["logit_val"][:, :make_golden.TOP], axis=1) <= 0)
    assert np.array_equal(g["logit_val"][:, 0] > -np.inf, np.ones(batch, bool))


def test_stored_benchmark_step_is_the_oracle_output():
    """Sequences 0 and 15 of the benchmark step recomputed from scratch."""
    g = np.load(make_golden.path_of("step_llama1b_b16"), allow_pickle=False)
    wl = synth.bench_step()
    weights = synth.model_weights(wl.shape, 1002)
    make_golden._STATE = (wl.shape, weights, wl)
    for b in (0, 15):
        r = make_golden._one_sequence(b)
        assert r["token"] == g["token"][b]
        assert np.array_equal(r["logit_idx"], g["logit_idx"][b])
        assert np.array_equal(r["logit_val"], g["logit_val"][b])
        assert np.array_equal(r["k"], g["k"][b]) and np.array_equal(r["v"], g["v"][b])


def test_stored_prefill_prompt_is_the_benchmark_prompt():
    g = np.load(make_golden.path_of("prefill_llama1b_t512"), allow_pickle=False)
    tokens = synth.rng(1007, "prompt").integers(0, synth.LLAMA1B.vocab, size=512).astype(np.int32)
    assert np.array_equal(g["tokens"], tokens) and int(g["start"]) == 0
    assert g["k0"].shape == (512, make_golden.KV_SAMPLES)


def test_stored_llama8b_layer_is_the_oracle_output():
    g = np.load(make_golden.path_of("layer_llama8b_b16"), allow_pickle=False)
    shape, wl, lw, hidden = make_golden.layer8b_inputs()
    assert list(g["seqs"]) == list(range(16)) and np.array_equal(g["positions"], wl.positions)
    assert g["out"].shape == (16, shape.hidden) and g["k"].shape == (16, make_golden.KV_SAMPLES)
    make_golden._LSTATE = (shape, wl, lw, hidden)
    r = make_golden._one_layer_sequence(5)
    for key in ("out", "k", "v", "k_rms", "v_rms"):
        assert np.array_equal(r[key], g[key][5]), key
