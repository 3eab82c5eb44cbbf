"""GPU parity of decoder_layer_decode and decode_step against the oracle,
through the C ABI.  Bars: layer outputs max-abs <= 1e-2 * RMS(out), and
the stricter bar on the layer's own contribution, max-abs <= 1e-3 *
RMS(out - hidden) (the residual delta; without it the N(0,1) residual would
hide a twenty-fold regression); each appended K/V value within one BF16 ulp
of the oracle's or within 1e-3 of the appended values' RMS, and the rest of
the pool untouched; logits max-abs <= 4e-4 for the full-size model (the
budget under which no argmax with a top-2 gap above 1e-3 can flip) and
<= 5e-3 * RMS(logits) for the small test models, whose weights are drawn
2.5 times wider and whose norm gains vary 15 times more than the full-size
models' to drive larger activations; the argmax identical wherever the
oracle's top-2 logit gap exceeds 1e-3.  The full-size batch-16, batch-64
and batch-128 steps are compared, every sequence, with stored oracle
outputs in test_gpu_golden.py."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import (DELTA_TOL, LAYER_TOL, LOGIT_ABS, TINY_LOGIT_REL, check_argmax_rule, check_pool_after, expected_pool_after, layer_gpu, say,
                      step_gpu)

pytestmark = pytest.mark.gpu



def _rms(a):
    return float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))


def _check_layer(shape, lw, hidden, wl, seqs=None):
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    bt = wl.block_tables[0]
    got, pool_after, err = layer_gpu(shape, lw, hidden, wl.pool, bt, wl.positions)
    assert err == 0
    ref, k_new, v_new = oracle.layer_decode_paged(shape, lw, hidden, wl.pool, geo, bt, wl.positions, seqs)
    rows = list(range(len(wl.positions))) if seqs is None else list(seqs)
    diff = np.abs(got[rows] - ref[rows]).max()
    delta_err = diff / max(_rms(ref[rows] - hidden[rows]), 1e-30)
    say("layer %s B=%d: max-abs %.3g, RMS(out) %.3g, error/RMS(delta) %.3g"
        % (shape.name, len(wl.positions), diff, _rms(ref[rows]), delta_err))
    assert diff <= LAYER_TOL * _rms(ref[rows])
    assert delta_err <= DELTA_TOL
    want = expected_pool_after(wl.pool, geo, bt, wl.positions, k_new, v_new, seqs)
    if seqs is None:
        kv_diff, kv_rms = check_pool_after(pool_after, want, wl.pool)
        say("  appended K/V: max-abs %.3g (RMS %.3g)" % (kv_diff, kv_rms))
    return diff


def test_layer_qwen_shape_batch1():
    """One Qwen2.5-0.5B-shaped layer, batch 1, 127 cached + 1 new, 64-page pool."""
    wl = synth.qwen05_layer_b1()
    _check_layer(wl.shape, wl.extra["weights"], wl.extra["hidden"], wl)


@pytest.mark.parametrize("batch,hkv,heads", [(1, 2, 4), (3, 2, 14), (9, 2, 4), (16, 2, 14), (17, 1, 16),
                                             (40, 4, 8), (70, 2, 4), (130, 2, 4)])
def test_layer_tiny_shapes(batch, hkv, heads):
    shape = synth.tiny_shape(hidden=192, heads=heads, kv_heads=hkv, inter=384, name="tiny-layer")
    seed = 100 + batch
    g = synth.rng(seed, "lens")
    positions = g.integers(0, 300, size=batch).astype(np.int32)
    positions[0] = 0
    if batch > 2:
        positions[1] = 15
        positions[2] = 16
    wl = synth.decode_workload("tiny", shape, seed, positions, layers=1)
    lw = synth.layer_weights(shape, seed, 0, sigma=0.05, norm_sigma=0.3)
    hidden = synth.rng(seed, "hidden").standard_normal((batch, shape.hidden)).astype(np.float32)
    _check_layer(shape, lw, hidden, wl)


@pytest.mark.parametrize("batch,inter", [(1, 4096), (5, 4352), (16, 8192), (33, 4352), (64, 4352)])
def test_layer_split_k_down_projection(batch, inter):
    """Down projections with K >= 4096 split K over workgroups and add the
    splits in a second kernel; 4352 (136 K steps) gives 17 splits, more than
    one round of the reduce kernel's 16-split loads; batch 33 also takes the
    two-column-tile path, batch 64 the tiled large-batch path."""
    shape = synth.tiny_shape(hidden=192, heads=4, kv_heads=2, inter=inter, name="tiny-split")
    seed = 300 + batch
    positions = synth.rng(seed, "lens").integers(0, 100, size=batch).astype(np.int32)
    wl = synth.decode_workload("tiny-split", shape, seed, positions, layers=1)
    lw = synth.layer_weights(shape, seed, 0, sigma=0.05, norm_sigma=0.3)
    hidden = synth.rng(seed, "hidden").standard_normal((batch, shape.hidden)).astype(np.float32)
    _check_layer(shape, lw, hidden, wl)


@pytest.mark.parametrize("head_dim", [64, 128])
def test_layer_tiled_split_qkv(head_dim):
    """Batch 70 takes the tiled projections; with hidden 512 the QKV
    projection has too few row tiles to fill the chip, so it splits K into
    partial sums finished (RoPE, q halves, K/V append) by a second kernel."""
    shape = synth.tiny_shape(hidden=512, heads=4, kv_heads=2, inter=512, head_dim=head_dim,
                             name="tiny-split-qkv")
    batch, seed = 70, 350 + head_dim
    positions = synth.rng(seed, "lens").integers(0, 300, size=batch).astype(np.int32)
    positions[:3] = [0, 15, 16]
    wl = synth.decode_workload("tiny-split-qkv", shape, seed, positions, layers=1)
    lw = synth.layer_weights(shape, seed, 0, sigma=0.05, norm_sigma=0.3)
    hidden = synth.rng(seed, "hidden").standard_normal((batch, shape.hidden)).astype(np.float32)
    _check_layer(shape, lw, hidden, wl)


def _check_step(shape, weights, wl, tokens, seqs=None, want_logits=True, logit_abs=None):
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    logits, nxt, pool_after, err = step_gpu(shape, weights, wl.pool, wl.block_tables, wl.positions,
                                            tokens, want_logits, want_pool=False)
    assert err == 0
    ref_logits, ref_tok, _, _ = oracle.decode_step_paged(shape, weights, wl.pool, geo, wl.block_tables,
                                                         wl.positions, tokens, seqs)
    rows = list(range(len(tokens))) if seqs is None else list(seqs)
    checked = check_argmax_rule(ref_logits[rows], nxt[rows])
    msg = "step %s B=%d rows=%s: argmax checked %d/%d" % (shape.name, len(tokens), rows, checked, len(rows))
    if logits is not None:
        per_row = np.abs(logits[rows] - ref_logits[rows]).max(axis=1)
        diff = float(per_row.max())
        worst = np.argsort(per_row)[::-1][:4]
        msg += ", max|dlogit| %.3g (RMS %.3g), worst rows %s" % (
            diff, _rms(ref_logits[rows]), ["%d@p%d:%.3g" % (rows[i], int(wl.positions[rows[i]]), per_row[i])
                                          for i in worst])
        bar = logit_abs if logit_abs is not None else TINY_LOGIT_REL * _rms(ref_logits[rows])
        say(msg)
        assert diff <= bar, "max|dlogit| %.3g > %.3g" % (diff, bar)
    else:
        say(msg)
    return nxt


def test_step_tiny_model():
    shape = synth.tiny_shape(hidden=128, layers=3, heads=4, kv_heads=2, inter=256, vocab=1000)
    positions = np.array([0, 5, 16, 47, 200], dtype=np.int32)
    weights = synth.model_weights(shape, 7, sigma=0.05, norm_sigma=0.3)
    wl = synth.decode_workload("tiny-step", shape, 7, positions)
    tokens = synth.rng(7, "tokens").integers(0, shape.vocab, size=5)
    nxt = _check_step(shape, weights, wl, tokens)
    # the same step without logits gives the same tokens
    _, nxt2, _, _ = step_gpu(shape, weights, wl.pool, wl.block_tables, wl.positions, tokens,
                             want_logits=False)
    assert np.array_equal(nxt, nxt2)


@pytest.mark.parametrize("batch", [64, 100])
def test_step_tiny_model_large_batch(batch):
    """Batches of 64 and more take the tiled projections and the tiled LM
    head (logits and per-tile argmax keys): every sequence against the
    oracle, and the same tokens without logits."""
    shape = synth.tiny_shape(hidden=128, layers=3, heads=4, kv_heads=2, inter=256, vocab=1000)
    seed = 70 + batch
    positions = synth.rng(seed, "lens").integers(0, 300, size=batch).astype(np.int32)
    positions[:3] = [0, 15, 16]
    weights = synth.model_weights(shape, seed, sigma=0.05, norm_sigma=0.3)
    wl = synth.decode_workload("tiny-step", shape, seed, positions)
    tokens = synth.rng(seed, "tokens").integers(0, shape.vocab, size=batch)
    nxt = _check_step(shape, weights, wl, tokens)
    _, nxt2, _, _ = step_gpu(shape, weights, wl.pool, wl.block_tables, wl.positions, tokens,
                             want_logits=False)
    assert np.array_equal(nxt, nxt2)


def test_step_llama_shape_batch1():
    """16-layer Llama-3.2-1B-shaped step, batch 1, context 1024."""
    wl = synth.llama1b_step_b1()
    weights = synth.model_weights(wl.shape, 1003)
    _check_step(wl.shape, weights, wl, wl.extra["tokens"], logit_abs=LOGIT_ABS)
