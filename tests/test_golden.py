"""Facts the source pages print, checked against the shapes and pool
geometry this repository uses (CPU only).  Fixtures: tests/golden/*.json,
each with its source."""
import json
import os

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_default_pool_holds_exactly_two_full_context_requests():
    g = _load("pool_geometry.json")
    page_bytes = 2 * g["llama_3_2_1b_kv_heads"] * g["page_tokens"] * g["llama_3_2_1b_head_dim"] * g["kv_dtype_bytes"]
    assert page_bytes == synth.page_elems(synth.LLAMA1B) * 2 == 32 * 1024
    pages = g["pool_default_mib"] * 2 ** 20 // page_bytes
    assert pages == 4096
    # admission budget of a request that may fill the context: prompt + new - 1 tokens,
    # rounded up to pages, in every layer
    budget = -(-(g["context_tokens"] - 1) // g["page_tokens"]) * g["layers"]
    assert budget == 2048 and pages // budget == 2


def test_qwen_shape_matches_checkpoint_sizes():
    g = _load("qwen_sizes.json")
    s = synth.QWEN05
    bias = (s.heads + 2 * s.kv_heads) * s.head_dim if g["qkv_bias_in_checkpoint"] else 0
    params = s.layers * (s.layer_param_count() + bias) + s.vocab * s.hidden + s.hidden
    assert abs(params * 2 / 2 ** 20 - g["safetensors_mib_approx"]) < 1.0
    fp32_bin = (params + s.vocab * s.hidden) * 4 / 2 ** 30
    assert abs(fp32_bin - g["fp32_bin_gib_approx"]) < 0.1
