"""GPU parity of sample_tokens (temperature, top-p, then top-k, inverse CDF
in vocabulary order) through the C ABI against the oracle's float64
sampler.  The result is an integer decided by floating point: the GPU's
token must be one the oracle accepts within oracle.SAMPLE_EPS of its
decisions (the nucleus boundary, the step of the CDF the draw falls on),
and equal to the oracle's token wherever that is unambiguous.  Repeated
calls must agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_transformer_amd as pkv
import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


def _draw_params(seed, B):
    r = synth.rng(seed, "sample")
    T = r.choice([0.0, 0.5, 0.7, 1.0, 1.3], size=B).astype(np.float32)
    p = r.choice([0.0, 0.3, 0.9, 0.95, 1.0], size=B).astype(np.float32)
    k = r.choice([0, 0, 1, 5, 50, 1000], size=B).astype(np.int32)
    u = r.random(size=B).astype(np.float32)
    return T, p, k, u


def _run(logits, T, p, k, u, ws=None):
    B, V = logits.shape
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    if ws is None:
        ws = pkv.alloc_workspace(pkv.sample_workspace_bytes(B, V))
    out = torch.full((B,), -1, dtype=torch.int32, device="cuda")
    pkv.sample_tokens(dev(logits), dev(T), dev(p), dev(k), dev(u), out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(logits, T, p, k, u, got, label):
    exact = 0
    for b in range(logits.shape[0]):
        tok, acc = oracle.sample_token(logits[b], float(T[b]), float(p[b]), int(k[b]), float(u[b]))
        assert int(got[b]) in acc, "%s seq %d (T %.2f p %.2f k %d u %.4f): GPU %d, oracle %d %s" % (
            label, b, T[b], p[b], k[b], u[b], got[b], tok, sorted(acc)[:8])
        if len(acc) == 1:
            exact += 1
    say("%s: %d sequences, %d unambiguous, all within the oracle's set" % (label, len(got), exact))


@pytest.mark.parametrize("V", [1000, 4097, 50001])
def test_sample_mixed_settings(V):
    B = 40
    logits = (synth.rng(V, "logits").normal(size=(B, V)) * 2.5).astype(np.float32)
    T, p, k, u = _draw_params(V, B)
    _check(logits, T, p, k, u, _run(logits, T, p, k, u), "V=%d" % V)


def test_sample_ties_and_minus_inf():
    """Logits on a coarse grid (many equal values, so the nucleus often ends
    inside a group of ties; the grid holds both +0 and -0, equal logits that
    form one group) and a quarter of the vocabulary at -inf."""
    B, V = 24, 3001
    r = synth.rng(7, "logits")
    logits = (np.round(r.normal(size=(B, V)) * 2.0) / 2.0).astype(np.float32)
    logits[r.random(size=(B, V)) < 0.25] = -np.inf
    T, p, k, u = _draw_params(8, B)
    _check(logits, T, p, k, u, _run(logits, T, p, k, u), "ties")


def test_sample_wide_first_level_bucket():
    """Logits within a narrow band (and one row of equal logits), so most of
    the vocabulary shares the first level's chosen bucket: the candidate
    list is longer than the part each thread holds in registers (8192
    entries), and the ties of the threshold key run through many chunks."""
    B, V = 6, 50001
    r = synth.rng(21, "logits")
    logits = (1.0 + np.round(r.normal(size=(B, V)) * 64.0) / 65536.0).astype(np.float32)
    logits[0] = 0.75
    T = np.array([1.0, 1.0, 0.7, 1.0, 1.3, 1.0], np.float32)
    p = np.array([0.5, 0.9, 0.3, 1.0, 0.95, 0.6], np.float32)
    k = np.array([0, 0, 0, 20000, 0, 9000], np.int32)
    u = r.random(size=B).astype(np.float32)
    _check(logits, T, p, k, u, _run(logits, T, p, k, u), "wide bucket")


def test_sample_grid_of_draws_one_sequence():
    """One distribution, 512 draws on a grid of u: every token the oracle's."""
    V, N = 2000, 512
    base = (synth.rng(11, "logits").normal(size=V) * 1.5).astype(np.float32)
    logits = np.repeat(base[None], N, axis=0)
    T = np.full(N, 0.8, np.float32)
    p = np.full(N, 0.9, np.float32)
    k = np.full(N, 0, np.int32)
    u = ((np.arange(N) + 0.5) / N).astype(np.float32)
    _check(logits, T, p, k, u, _run(logits, T, p, k, u), "grid")


def test_sample_large_batch_and_repeat_is_bitwise():
    B, V = 300, 5000
    logits = (synth.rng(300, "logits").normal(size=(B, V)) * 3.0).astype(np.float32)
    T, p, k, u = _draw_params(300, B)
    ws = pkv.alloc_workspace(pkv.sample_workspace_bytes(B, V))
    a = _run(logits, T, p, k, u, ws)
    b = _run(logits, T, p, k, u, ws)
    assert np.array_equal(a, b)
    _check(logits, T, p, k, u, a, "batch 300")


def test_sample_llama_vocab_batch16():
    """The bench's shape: 16 sequences of 128256 logits (N(0, 2.5): nuclei of
    thousands of tokens), mixed settings, plus top-p 0.9 at T 1 for all."""
    B, V = 16, 128256
    logits = (synth.rng(1002, "logits").normal(size=(B, V)) * 2.5).astype(np.float32)
    T, p, k, u = _draw_params(1002, B)
    _check(logits, T, p, k, u, _run(logits, T, p, k, u), "llama mixed")
    T = np.ones(B, np.float32)
    p = np.full(B, 0.9, np.float32)
    k = np.zeros(B, np.int32)
    _check(logits, T, p, k, u, _run(logits, T, p, k, u), "llama top-p 0.9")
