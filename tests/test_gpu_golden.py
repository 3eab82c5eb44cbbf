"""GPU parity at full size against stored oracle outputs.

tests/golden/make_golden.py (CPU only: the oracle and the input generators)
wrote, for every sequence of three full-size decode steps and for the
benchmark's 512-token prefill, the oracle's argmax, top-2 logit gap, logit
RMS, logits at fixed sample indices, and the appended K/V at fixed sample
positions.  Here the HIP path runs the same seeded inputs through the C ABI
and every sequence is compared:
  * logits at the sample indices (the 16 largest and 256 strided ones):
    max-abs <= LOGIT_ABS = 4e-4, the budget under which no argmax whose top-2
    gap exceeds 1e-3 can flip (two logits each off by less than 5e-4); for
    the prefill, whose two sides also compute and round every prompt
    token's K/V, 2.5e-3 free-running and 4e-4 against the oracle fed the
    GPU's own K/V;
  * the argmax equals the oracle's wherever the oracle's top-2 gap exceeds
    1e-3; elsewhere it is one of the oracle's top logits within 1e-3 of the
    largest;
  * each layer's appended K and V at the sample positions: within one BF16
    ulp of the oracle's value or 1e-3 of the RMS of that layer's appended
    vector;
  * prefill: layer 0's K/V of all 512 prompt tokens the same way, and every
    layer's K/V of sampled tokens against the oracle fed the GPU's own K/V
    of the earlier positions (teacher forcing), at the same bar.
The three steps are the benchmark's (Llama-3.2-1B shape, batch 16, lengths
U[1,2048]), batch 64 with contexts U[64,2048] (the tiled projections), and
the 24-layer Qwen2.5-0.5B shape at batch 128 with 4096 cached tokens each;
and one Llama-3-8B-shaped layer (head width 128) at batch 16, every output
row against the stored oracle output."""
import os

import numpy as np
import pytest
import torch

import oracle
import paged_kv_transformer_amd as pkv
import synth
from golden import make_golden
from gpu_util import assert_layer_out, check_kv_values, dev, layer_gpu, say, teacher_forced_prefill_kv

pytestmark = pytest.mark.gpu

LOGIT_ABS = 4e-4
# The prefill's free-running logits: every one of the 512 prompt tokens'
# K/V at each of the 16 layers is computed and rounded to BF16 by both sides,
# and a value that rounds to the other BF16 neighbour (its FP32 sums differ
# in the last bits) changes every later token's attention; measured
# 1.2e-3 at the last token, against 4e-4 or less once the oracle reads the
# GPU's own K/V (teacher forcing, asserted below).
PREFILL_LOGIT_ABS = 2.5e-3
GAP = 1e-3


def _load(name):
    path = make_golden.path_of(name)
    if not os.path.exists(path):
        pytest.fail("stored oracle outputs missing: run python tests/golden/make_golden.py --only %s" % name)
    return dict(np.load(path, allow_pickle=False))


_SLOT_OFFSETS = {}


def slot_offsets(geo, slot):
    """Element offsets, inside a page, of one token's K ([kv*D]) and V
    ([kv*D]) at `slot`: found by the oracle's own append of distinct marker
    values into an empty page."""
    key = (geo.kv_heads, geo.head_dim, geo.page_tokens, slot)
    if key not in _SLOT_OFFSETS:
        kvd = geo.kv_heads * geo.head_dim
        page = np.zeros(geo.page_elems, np.uint16)
        oracle.pool_append(page, geo, np.zeros(1, np.int32), slot, np.arange(1, kvd + 1, dtype=np.uint16),
                           np.arange(kvd + 1, 2 * kvd + 1, dtype=np.uint16))
        where = np.full(2 * kvd + 1, -1, np.int64)
        nz = np.nonzero(page)[0]
        where[page[nz]] = nz
        assert (where[1:] >= 0).all()
        _SLOT_OFFSETS[key] = (where[1:kvd + 1], where[kvd + 1:])
    return _SLOT_OFFSETS[key]


def appended_index(geo, bt_row, pos, sample):
    """Flat pool element indices of the K and V that position `pos` of a
    sequence (table row bt_row) holds, at the sampled [kv*D] positions."""
    ko, vo = slot_offsets(geo, pos % geo.page_tokens)
    page = int(bt_row[pos // geo.page_tokens])
    base = page * geo.page_elems
    return base + ko[sample], base + vo[sample]


def check_logits(gold, logits_rows, tokens, label, bar=LOGIT_ABS):
    """logits_rows[i] / tokens[i]: the GPU's row for stored sequence i."""
    idx = gold["logit_idx"]
    got = np.take_along_axis(logits_rows, idx.astype(np.int64), axis=1)
    diff = np.abs(got.astype(np.float64) - gold["logit_val"].astype(np.float64))
    worst = float(diff.max())
    flips = 0
    for i in range(len(tokens)):
        if gold["gap"][i] > GAP:
            assert int(tokens[i]) == int(gold["token"][i]), "%s row %d: argmax %d vs oracle %d (gap %.3g)" % (
                label, i, int(tokens[i]), int(gold["token"][i]), gold["gap"][i])
        else:
            top = gold["logit_val"][i, 0]
            near = {int(j) for j, v in zip(idx[i, :make_golden.TOP], gold["logit_val"][i, :make_golden.TOP])
                    if top - v <= GAP}
            assert int(tokens[i]) in near, "%s row %d: token %d not among the oracle's near-top %s" % (
                label, i, int(tokens[i]), sorted(near))
            flips += int(tokens[i]) != int(gold["token"][i])
    say("%s: %d rows, max|dlogit| %.3g at the samples (RMS %.3g), argmax checked %d, near-ties %d (%d differ)" % (
        label, len(tokens), worst, float(np.mean(gold["logit_rms"])), int((gold["gap"] > GAP).sum()),
        int((gold["gap"] <= GAP).sum()), flips))
    assert worst <= bar, "%s: max|dlogit| %.3g > %.1e" % (label, worst, bar)
    return worst


STEP_SEEDS = {"step_llama1b_b16": 1002, "step_llama1b_b64": 1004, "step_qwen05_b128": 1005}


@pytest.mark.parametrize("name", list(STEP_SEEDS))
def test_step_every_sequence_against_stored_oracle(name):
    gold = _load(name)
    wl = make_golden.STEPS[name][0]()
    shape = wl.shape
    weights = synth.model_weights(shape, STEP_SEEDS[name])
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    B = wl.batch
    assert list(gold["seqs"]) == list(range(B))
    mp = int(wl.positions.max()) + 1
    cfg = pkv.make_config(shape, max_pos=mp)
    model = pkv.upload_model(weights, shape.theta, mp, head_dim=shape.head_dim)
    pool_t = dev(wl.pool)
    del weights
    pool = pkv.kv_pool_create(pool_t, shape.kv_heads, head_dim=shape.head_dim)
    bts = np.ascontiguousarray(wl.block_tables, dtype=np.int32)
    ws = pkv.alloc_workspace(pkv.workspace_bytes(cfg, B, bts.shape[2]))
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    say("%s: running the GPU step" % name)
    pkv.decode_step(cfg, model, pool, dev(bts), dev(wl.positions), dev(wl.extra["tokens"]), logits, nxt, ws)
    assert pkv.device_error(ws) == 0
    check_logits(gold, logits.cpu().numpy(), nxt.cpu().numpy(), name)

    # appended K/V of every (layer, sequence) at the sampled positions
    sample = gold["kv_idx"].astype(np.int64)
    kidx, vidx = [], []
    for l in range(shape.layers):
        for b in range(B):
            ki, vi = appended_index(geo, bts[l, b], int(wl.positions[b]), sample)
            kidx.append(ki)
            vidx.append(vi)
    flat = pool_t.view(-1)
    gk = flat[torch.from_numpy(np.concatenate(kidx)).cuda()].cpu().numpy().view(np.uint16)
    gv = flat[torch.from_numpy(np.concatenate(vidx)).cuda()].cpu().numpy().view(np.uint16)
    gk = gk.reshape(shape.layers, B, -1)
    gv = gv.reshape(shape.layers, B, -1)
    worst = 0.0
    for l in range(shape.layers):
        for b in range(B):
            d1, _ = check_kv_values(gk[l, b], gold["k"][b, l], rms=float(gold["k_rms"][b, l]),
                                    what="%s K layer %d seq %d" % (name, l, b))
            d2, _ = check_kv_values(gv[l, b], gold["v"][b, l], rms=float(gold["v_rms"][b, l]),
                                    what="%s V layer %d seq %d" % (name, l, b))
            worst = max(worst, d1, d2)
    say("%s: appended K/V of %d layers x %d sequences, max-abs %.3g at the samples" % (
        name, shape.layers, B, worst))


def test_layer_llama8b_every_sequence_against_stored_oracle():
    """One Llama-3-8B-shaped layer (head width 128), batch 16, contexts
    U[1,1024]: every sequence's output row against the stored oracle output
    (max-abs <= 1e-2 RMS(out) and <= 1e-3 RMS(out - hidden)) and its appended
    K/V at the sample positions (one BF16 ulp or 1e-3 of the vector's RMS)."""
    gold = _load("layer_llama8b_b16")
    shape, wl, lw, hidden = make_golden.layer8b_inputs()
    assert np.array_equal(gold["positions"], wl.positions)
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    bt = wl.block_tables[0]
    got, pool_after, err = layer_gpu(shape, lw, hidden, wl.pool, bt, wl.positions)
    assert err == 0
    assert_layer_out(got, gold["out"], hidden, "layer %s B=%d (stored oracle)" % (shape.name, wl.batch))
    sample = gold["kv_idx"].astype(np.int64)
    worst = 0.0
    for b in range(wl.batch):
        ki, vi = appended_index(geo, bt[b], int(wl.positions[b]), sample)
        worst = max(worst, check_kv_values(pool_after[ki], gold["k"][b], rms=float(gold["k_rms"][b]),
                                           what="8b layer K seq %d" % b)[0])
        worst = max(worst, check_kv_values(pool_after[vi], gold["v"][b], rms=float(gold["v_rms"][b]),
                                           what="8b layer V seq %d" % b)[0])
    say("8b layer: appended K/V of %d sequences, max-abs %.3g at the samples" % (wl.batch, worst))


def test_prefill_512_against_stored_oracle():
    """The benchmark's prefill (Llama-3.2-1B shape, 512 tokens from position
    0): the last token's logits and argmax against the stored oracle, layer
    0's K/V of every token, and every layer's K/V of sampled tokens against
    the teacher-forced oracle."""
    from test_gpu_prefill import prefill_gpu
    gold = _load("prefill_llama1b_t512")
    shape, weights, pool, bts, tokens = make_golden.prefill_inputs()
    assert np.array_equal(tokens, gold["tokens"])
    T = len(tokens)
    geo = oracle.PoolGeometry(shape.kv_heads, shape.head_dim)
    logits, nxt, pool_after, err = prefill_gpu(shape, weights, pool, bts, 0, tokens)
    assert err == 0
    one = {k: (v[None] if k in ("logit_idx", "logit_val") else np.atleast_1d(v)) for k, v in gold.items()}
    check_logits(one, logits[None], np.array([nxt]), "prefill 512 (free-running oracle)",
                 bar=PREFILL_LOGIT_ABS)
    sample = gold["kv_idx"].astype(np.int64)
    gk, gv = [], []
    for t in range(T):
        ki, vi = appended_index(geo, bts[0], t, sample)
        gk.append(pool_after[ki])
        gv.append(pool_after[vi])
    w0 = 0.0
    for t in range(T):
        w0 = max(w0, check_kv_values(gk[t], gold["k0"][t], rms=float(gold["k0_rms"][t]),
                                     what="prefill layer-0 K token %d" % t)[0])
        w0 = max(w0, check_kv_values(gv[t], gold["v0"][t], rms=float(gold["v0_rms"][t]),
                                     what="prefill layer-0 V token %d" % t)[0])
    t_list = [1, 15, 16, 255, 256, 511]
    ref = teacher_forced_prefill_kv(shape, weights, pool_after, geo, bts, 0, tokens, t_list)
    deep = []
    for l in range(shape.layers):
        have, want = [], []
        for t in t_list:
            kc, vc = oracle.pool_gather(pool_after, geo, bts[l], t + 1)
            have += [oracle.f32_to_bf16(kc[t]), oracle.f32_to_bf16(vc[t])]
            want += [ref[(l, t)][0], ref[(l, t)][1]]
        deep.append(check_kv_values(np.concatenate(have), np.concatenate(want),
                                    what="prefill K/V of layer %d (teacher-forced)" % l)[0])
    say("prefill 512: layer-0 K/V of %d tokens max-abs %.3g; teacher-forced K/V of tokens %s per layer %s" % (
        T, w0, t_list, ["%.3g" % d for d in deep]))
    # the last token's logits from the teacher-forced oracle: the budget of
    # a decode step holds once both sides attend over the same K/V
    tf, _ = oracle.lm_head(weights["embed"], weights["final_norm"], shape.eps, ref[("x", T - 1)])
    diff = float(np.abs(logits.astype(np.float64) - tf).max())
    say("prefill 512: last logits against the teacher-forced oracle max-abs %.3g (RMS %.3g)" % (
        diff, float(np.sqrt(np.mean(tf.astype(np.float64) ** 2)))))
    assert diff <= LOGIT_ABS
