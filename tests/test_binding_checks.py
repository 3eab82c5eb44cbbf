"""The Python binding refuses tensors too small for what a call reads or
writes, before anything reaches the device (the C ABI takes plain pointers
and cannot check sizes).  CPU tensors: a call with the right sizes gets as
far as the device check ("must be on the GPU"), a short one stops at the
size check."""
import types

import pytest
import torch

import paged_kv_transformer_amd as pkv


def _pool(kv_heads=2, head_dim=64):
    p = pkv.Pool()
    p.num_kv_heads, p.head_dim, p.page_tokens = kv_heads, head_dim, 16
    return p


def _cfg(**kw):
    c = pkv.Config(256, 2, 4, 2, 64, 512, 1000, 64, 1e4, 1e-5)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def bf(*shape):
    return torch.zeros(shape, dtype=torch.int16)


def ws():
    return torch.zeros(256, dtype=torch.uint8)


def _packed(rows, cols, layout=pkv.PACK_ROWS):
    """Elements of a packed matrix (whole 16-row groups)."""
    return pkv.packed_weight_bytes(rows, cols, layout) // 2


def _layer(cfg, shrink=None):
    H, I, D = cfg.hidden_size, cfg.intermediate_size, cfg.head_dim
    qkv = (cfg.num_attention_heads + 2 * cfg.num_key_value_heads) * D
    n = {"attn_norm": H, "mlp_norm": H, "w_qkv": qkv * H, "w_o": H * cfg.num_attention_heads * D,
         "w_gate_up": 2 * I * H, "w_down": H * I}
    if shrink:
        n[shrink] -= 1
    return types.SimpleNamespace(tensors={k: bf(v) for k, v in n.items()}, c=pkv.LayerWeights())


def _gpu_only(fn):
    with pytest.raises(ValueError, match="GPU"):
        fn()


def _too_small(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_paged_gqa_decode_sizes():
    P, B, Hq = _pool(), 3, 8
    call = lambda q=bf(B, Hq, 64), bt=i32(B, 4), lens=i32(B), out=f32(B, Hq, 64): pkv.paged_gqa_decode(
        P, q, bt, lens, 0.125, out, ws())
    _gpu_only(call)
    _too_small(lambda: call(q=bf(B, Hq, 128)), "q must be")   # head width of another pool
    _too_small(lambda: call(out=f32(B, Hq, 63)), "out holds")
    _too_small(lambda: call(bt=i32(B - 1, 4)), "block_table")
    _too_small(lambda: call(lens=i32(B - 1)), "context_lens")


def test_kv_append_sizes():
    P, B = _pool(kv_heads=2, head_dim=128), 4
    call = lambda k=bf(B, 256), v=bf(B, 256), bt=i32(B, 2): pkv.kv_append(P, bt, i32(B), k, v)
    _gpu_only(call)
    _too_small(lambda: call(k=bf(B, 255)), "k_new")
    _too_small(lambda: call(v=bf(B - 1, 256)), "v_new")
    _too_small(lambda: call(bt=i32(B - 1, 2)), "block_table")


def test_decoder_layer_decode_sizes():
    cfg, B = _cfg(), 5
    rope = f32(cfg.max_position_embeddings, 32)
    call = lambda hidden=f32(B, 256), layer=_layer(cfg), rc=rope: pkv.decoder_layer_decode(
        cfg, layer, rc, rope, _pool(), i32(B, 4), i32(B), hidden, ws())
    _gpu_only(call)
    _too_small(lambda: call(hidden=f32(B, 255)), "hidden")
    _too_small(lambda: call(rc=f32(cfg.max_position_embeddings - 1, 32)), "rope_cos")
    for k in ("w_qkv", "w_o", "w_gate_up", "w_down", "attn_norm"):
        _too_small(lambda: call(layer=_layer(cfg, shrink=k)), k)


def test_decode_step_sizes():
    cfg, B = _cfg(), 4
    rope = f32(cfg.max_position_embeddings, 32)

    full = _packed(cfg.vocab_size, cfg.hidden_size)

    def model(layers=2, embed=bf(full)):
        return types.SimpleNamespace(layers=[_layer(cfg) for _ in range(layers)], embed=embed,
                                     final_norm=bf(cfg.hidden_size), rope_cos=rope, rope_sin=rope, c=pkv.ModelWeights())

    call = lambda bts=i32(2, B, 4), logits=f32(B, cfg.vocab_size), m=None: pkv.decode_step(
        cfg, m or model(), _pool(), bts, i32(B), i32(B), logits, i32(B), ws())
    _gpu_only(call)
    _gpu_only(lambda: call(logits=None))
    _too_small(lambda: call(bts=i32(2, B + 1, 4)), "block_tables")   # layer-major needs exactly B rows
    _too_small(lambda: call(bts=i32(1, B, 4)), "block_tables")
    _too_small(lambda: call(logits=f32(B, cfg.vocab_size - 1)), "logits")
    _too_small(lambda: call(m=model(layers=1)), "layers")
    _too_small(lambda: call(m=model(embed=bf(full - 1))), "embed")


def test_prefill_and_sampling_sizes():
    cfg = _cfg()
    rope = f32(cfg.max_position_embeddings, 32)
    m = types.SimpleNamespace(layers=[_layer(cfg) for _ in range(2)], embed=bf(_packed(cfg.vocab_size, 256)),
                              final_norm=bf(256), rope_cos=rope, rope_sin=rope, c=pkv.ModelWeights())
    call = lambda bts=i32(2, 4), logits=f32(cfg.vocab_size): pkv.prefill(
        cfg, m, _pool(), bts, 0, i32(10), logits, i32(1), ws())
    _gpu_only(call)
    _too_small(lambda: call(bts=i32(1, 4)), "block_tables")
    _too_small(lambda: call(logits=f32(cfg.vocab_size - 1)), "logits")

    B, V = 3, 100
    s = lambda logits=f32(B, V), tok=i32(B), k=i32(B): pkv.sample_tokens(logits, f32(B), f32(B), k, f32(B), tok, ws())
    _gpu_only(s)
    _too_small(lambda: s(tok=i32(B - 1)), "tokens")
    _too_small(lambda: s(k=i32(B - 1)), "top_k")
    _too_small(lambda: s(logits=f32(B * V)), "logits must be")
