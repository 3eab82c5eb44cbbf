"""The C-ABI library on the host (no GPU needed): it loads, exports every
function include/pkv.h declares, and rejects bad arguments with the stated
negative errno before any HIP call."""
import ctypes
import errno
import os
import re

import pytest

import paged_kv_transformer_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

if not os.path.exists(pkv.LIB_PATH):
    pytest.skip("libpkv.so is not built", allow_module_level=True)

L = pkv.lib()
FAKE = 1 << 20          # an aligned non-null address: validation never dereferences it
EINVAL, ENOTSUP, ENOSPC = -errno.EINVAL, -errno.ENOTSUP, -errno.ENOSPC


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function():
    names = declared_functions()
    for must in ("kv_pool_create", "kv_append", "paged_gqa_decode", "decoder_layer_decode",
                 "decode_step", "pkv_workspace_bytes", "pkv_device_error"):
        assert must in names
    for n in names:
        assert hasattr(L, n), n


def _pool(hkv=8, pages=64):
    p = pkv.Pool()
    assert L.kv_pool_create(FAKE, pages * 2 * hkv * 16 * 64 * 2, hkv, 64, 16, ctypes.byref(p)) == 0
    return p


def test_kv_pool_create_geometry_and_errors():
    p = pkv.Pool()
    assert L.kv_pool_create(FAKE, 128 << 20, 8, 64, 16, ctypes.byref(p)) == 0
    assert p.page_bytes == 32768 and p.num_pages == 4096
    assert L.kv_pool_create(FAKE, 8 * 8192 + 100, 2, 64, 16, ctypes.byref(p)) == 0
    assert p.page_bytes == 8192 and p.num_pages == 8
    assert L.kv_pool_create(None, 1 << 20, 8, 64, 16, ctypes.byref(p)) == EINVAL
    assert L.kv_pool_create(FAKE + 8, 1 << 20, 8, 64, 16, ctypes.byref(p)) == EINVAL
    assert L.kv_pool_create(FAKE, 1 << 20, 0, 64, 16, ctypes.byref(p)) == EINVAL
    assert L.kv_pool_create(FAKE, 128 << 20, 8, 128, 16, ctypes.byref(p)) == 0
    assert p.page_bytes == 65536 and p.num_pages == 2048 and p.head_dim == 128
    assert L.kv_pool_create(FAKE, 1 << 20, 8, 96, 16, ctypes.byref(p)) == ENOTSUP
    assert L.kv_pool_create(FAKE, 1 << 20, 8, 256, 16, ctypes.byref(p)) == ENOTSUP
    assert L.kv_pool_create(FAKE, 1 << 20, 8, 64, 128, ctypes.byref(p)) == ENOTSUP
    assert L.kv_pool_create(FAKE, 1000, 8, 64, 16, ctypes.byref(p)) == ENOSPC
    assert L.kv_pool_create(FAKE, 1 << 20, 8, 64, 16, None) == EINVAL


def test_page_sizes_and_split_pools():
    p = pkv.Pool()
    # 256-token pages: 16 times the bytes of a 16-token page
    assert L.kv_pool_create(FAKE, 128 << 20, 8, 64, 256, ctypes.byref(p)) == 0
    assert p.page_bytes == 16 * 32768 and p.num_pages == 256 and p.page_tokens == 256
    assert not p.v_base
    assert L.kv_pool_create(FAKE, 128 << 20, 8, 64, 32, ctypes.byref(p)) == ENOTSUP
    # separate K and V pools: each page of each pool holds one block
    V = FAKE + (1 << 30)
    assert L.kv_pool_create_split(FAKE, V, 64 << 20, 8, 64, 16, ctypes.byref(p)) == 0
    assert p.page_bytes == 16384 and p.num_pages == 4096 and p.v_base == V
    assert L.kv_pool_create_split(FAKE, V, 64 << 20, 8, 128, 256, ctypes.byref(p)) == 0
    assert p.page_bytes == 8 * 256 * 128 * 2 and p.num_pages == 128
    assert L.kv_pool_create_split(FAKE, None, 64 << 20, 8, 64, 16, ctypes.byref(p)) == EINVAL
    assert L.kv_pool_create_split(FAKE, FAKE, 64 << 20, 8, 64, 16, ctypes.byref(p)) == EINVAL
    assert L.kv_pool_create_split(FAKE, FAKE + (32 << 20), 64 << 20, 8, 64, 16,
                                  ctypes.byref(p)) == EINVAL              # overlapping
    assert L.kv_pool_create_split(FAKE, V + 8, 64 << 20, 8, 64, 16, ctypes.byref(p)) == EINVAL
    # a table of 8 pages of 256 tokens needs the splits of 128 pages of 16
    assert (L.pkv_attention_workspace_bytes(32, 8, 64, 16, 8, 256)
            == L.pkv_attention_workspace_bytes(32, 8, 64, 16, 128, 16))
    assert L.pkv_attention_workspace_bytes(32, 8, 64, 16, 8, 64) == 0
    cfg = _cfg()
    assert (L.pkv_workspace_bytes(ctypes.byref(cfg), 16, 8, 256)
            == L.pkv_workspace_bytes(ctypes.byref(cfg), 16, 128, 16))


def test_paged_gqa_decode_validation():
    p = _pool()
    ws_need = L.pkv_attention_workspace_bytes(32, 8, 64, 16, 128, 16)
    assert ws_need > 0
    args = lambda **kw: [ctypes.byref(kw.get("pool", p)), kw.get("q", FAKE), kw.get("hq", 32),
                         kw.get("bt", FAKE), kw.get("mp", 128), kw.get("lens", FAKE), kw.get("b", 16),
                         kw.get("scale", 0.125), kw.get("out", FAKE), kw.get("ws", FAKE),
                         kw.get("wsb", ws_need), None]
    assert L.paged_gqa_decode(*args(q=None)) == EINVAL
    assert L.paged_gqa_decode(*args(hq=30)) == EINVAL          # 30 % 8 != 0
    assert L.paged_gqa_decode(*args(hq=8 * 17)) == ENOTSUP     # group of 17
    assert L.paged_gqa_decode(*args(b=-1)) == EINVAL
    assert L.paged_gqa_decode(*args(mp=0)) == EINVAL
    assert L.paged_gqa_decode(*args(b=65536)) == ENOTSUP       # grid y limit
    assert L.paged_gqa_decode(*args(mp=8 * 65535 + 1)) == ENOTSUP  # more than 65535 splits
    assert L.paged_gqa_decode(*args(wsb=ws_need - 1)) == ENOSPC
    assert L.paged_gqa_decode(*args(ws=FAKE + 4)) == EINVAL
    assert L.paged_gqa_decode(*args(scale=float("nan"))) == EINVAL
    assert L.paged_gqa_decode(*args(b=0)) == 0                 # empty batch: nothing to do
    bad = pkv.Pool.from_buffer_copy(p)
    bad.page_tokens = 32
    assert L.paged_gqa_decode(*args(pool=bad)) == ENOTSUP


def test_paged_gqa_decode_noalloc_validation():
    """The allocation-free variant validates like paged_gqa_decode, needs
    an error word, and refuses calls whose split records exceed its fixed
    scratch array, all before any HIP call."""
    p = _pool(pages=4096)
    args = lambda **kw: [ctypes.byref(kw.get("pool", p)), kw.get("q", FAKE), kw.get("hq", 32),
                         kw.get("bt", FAKE), kw.get("mp", 128), kw.get("lens", FAKE), kw.get("b", 16),
                         kw.get("scale", 0.125), kw.get("out", FAKE), kw.get("err", FAKE), None]
    f = L.paged_gqa_decode_noalloc
    assert f(*args(q=None)) == EINVAL
    assert f(*args(err=None)) == EINVAL
    assert f(*args(err=FAKE + 2)) == EINVAL
    assert f(*args(hq=30)) == EINVAL
    assert f(*args(hq=8 * 17)) == ENOTSUP
    assert f(*args(b=65536)) == ENOTSUP
    assert f(*args(scale=float("inf"))) == EINVAL
    assert f(*args(b=0)) == 0
    # 64 sequences x 8 kv heads over 2048-token tables: 8 splits of
    # 4224-byte records = 17.3 MB > PKV_NOALLOC_SCRATCH_BYTES (16 MiB)
    assert pkv.NOALLOC_SCRATCH_BYTES == 16 << 20
    assert f(*args(b=64)) == ENOSPC
    assert f(*args(b=64, mp=8192)) == ENOSPC


def _cfg(**kw):
    c = pkv.Config(2048, 16, 32, 8, 64, 8192, 128256, 4096, 5e5, 1e-5)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_layer_and_step_validation():
    p = _pool()
    lw = pkv.LayerWeights(*([FAKE] * 6))
    cfg = _cfg()
    need = L.pkv_workspace_bytes(ctypes.byref(cfg), 16, 128, 16)
    assert need > 0

    def layer(c=cfg, w=lw, pool=p, b=16, wsb=need, ws=FAKE, hidden=FAKE):
        return L.decoder_layer_decode(ctypes.byref(c), ctypes.byref(w), FAKE, FAKE, ctypes.byref(pool),
                                      FAKE, 128, FAKE, b, hidden, ws, wsb, None)

    assert layer(c=_cfg(head_dim=96)) == ENOTSUP
    assert layer(c=_cfg(head_dim=128)) == EINVAL               # the pool's heads are 64 wide
    assert layer(c=_cfg(hidden_size=2000)) == ENOTSUP
    assert layer(c=_cfg(intermediate_size=100)) == ENOTSUP
    assert layer(c=_cfg(intermediate_size=65536 + 64)) == ENOTSUP   # past the 32-bit byte ranges
    assert layer(c=_cfg(hidden_size=65536 + 64)) == ENOTSUP
    assert layer(c=_cfg(hidden_size=16384, intermediate_size=65536)) == ENOTSUP  # gate/up over 2 GiB
    assert layer(c=_cfg(vocab_size=600000)) == ENOTSUP         # tied embedding over 2 GiB
    assert layer(c=_cfg(num_key_value_heads=3)) == EINVAL
    assert layer(c=_cfg(rms_norm_eps=float("nan"))) == EINVAL
    assert layer(pool=_pool(hkv=2)) == EINVAL                  # pool heads != config heads
    assert layer(w=pkv.LayerWeights(FAKE, None, FAKE, FAKE, FAKE, FAKE)) == EINVAL
    assert layer(wsb=need - 1) == ENOSPC
    assert layer(hidden=None) == EINVAL
    assert layer(b=-3) == EINVAL
    assert layer(b=0) == 0

    layers = (pkv.LayerWeights * 16)(*([lw] * 16))
    mw = pkv.ModelWeights(FAKE, FAKE, ctypes.cast(layers, ctypes.POINTER(pkv.LayerWeights)), FAKE, FAKE)

    def step(c=cfg, m=mw, nxt=FAKE, wsb=need, b=16):
        return L.decode_step(ctypes.byref(c), ctypes.byref(m), ctypes.byref(p), FAKE, 128, FAKE, FAKE, b,
                             None, nxt, FAKE, wsb, None)

    assert step(nxt=None) == EINVAL
    assert step(c=_cfg(vocab_size=0)) == EINVAL
    assert step(wsb=need - 256) == ENOSPC
    layers[5] = pkv.LayerWeights(FAKE, FAKE, FAKE, FAKE, None, FAKE)
    assert step() == EINVAL
    assert step(b=0) == EINVAL                                 # layer 5 is still incomplete


def test_rope_table_and_workspace_validation():
    assert L.pkv_rope_table(1e4, 96, 10, FAKE, FAKE, None) == ENOTSUP
    assert L.pkv_rope_table(1e4, 32, 10, FAKE, FAKE, None) == ENOTSUP
    assert L.pkv_rope_table(1e4, 64, 0, FAKE, FAKE, None) == EINVAL
    assert L.pkv_rope_table(-1.0, 64, 10, FAKE, FAKE, None) == EINVAL
    assert L.pkv_rope_table(1e4, 64, 10, None, FAKE, None) == EINVAL
    assert L.pkv_workspace_init(None, 256, None) == EINVAL
    assert L.pkv_workspace_init(FAKE + 1, 256, None) == EINVAL
    assert L.pkv_device_error(None, None) == EINVAL
    assert L.pkv_attention_workspace_bytes(32, 8, 96, 16, 128, 16) == 0
    # the split records hold a head's FP32 partial output: twice as wide at D 128
    w64 = L.pkv_attention_workspace_bytes(32, 8, 64, 16, 128, 16)
    w128 = L.pkv_attention_workspace_bytes(32, 8, 128, 16, 128, 16)
    assert w64 > 0 and w128 > w64
    assert L.pkv_workspace_bytes(None, 1, 1, 16) == 0


def test_head_dim_128_config_and_packing_sizes():
    cfg = _cfg(head_dim=128)
    assert L.pkv_workspace_bytes(ctypes.byref(cfg), 16, 64, 16) > L.pkv_workspace_bytes(ctypes.byref(_cfg()), 16, 64, 16)
    assert L.pkv_workspace_bytes(ctypes.byref(_cfg(head_dim=96)), 16, 64, 16) == 0
    assert L.pkv_packed_weight_bytes(3 * 128, 64, pkv.PACK_QKV128) == 3 * 128 * 64 * 2
    assert L.pkv_packed_weight_bytes(3 * 64, 64, pkv.PACK_QKV128) == 0      # not whole 128-wide heads
    assert L.pkv_packed_weight_bytes(3 * 64, 64, pkv.PACK_QKV) == 3 * 64 * 64 * 2
    assert L.pkv_packed_weight_bytes(64, 64, 4) == 0


def test_workspace_sizes_grow_with_batch_and_pages():
    cfg = _cfg()
    a = L.pkv_workspace_bytes(ctypes.byref(cfg), 1, 64, 16)
    b = L.pkv_workspace_bytes(ctypes.byref(cfg), 64, 64, 16)
    c = L.pkv_workspace_bytes(ctypes.byref(cfg), 64, 128, 16)
    assert 0 < a < b < c
    assert all(x % 256 == 0 for x in (a, b, c))


def test_measurement_probes_reject_bad_arguments():
    """The probes validate like every other entry point, before any HIP
    call: buffer, alignment, byte count and workgroup count; the paged-read
    probe takes the attention call's own checks."""
    assert L.pkv_probe_read(None, 1024, 4, FAKE, None) == EINVAL
    assert L.pkv_probe_read(FAKE + 4, 1024, 4, FAKE, None) == EINVAL     # not 16-byte aligned
    assert L.pkv_probe_read(FAKE, 1000, 4, FAKE, None) == EINVAL         # not whole 16-byte chunks
    assert L.pkv_probe_read(FAKE, 0, 4, FAKE, None) == EINVAL
    assert L.pkv_probe_read(FAKE, 1024, 0, FAKE, None) == EINVAL
    assert L.pkv_probe_read(FAKE, 1024, 4, None, None) == EINVAL
    assert L.pkv_probe_empty(-1, 1, None) == EINVAL
    assert L.pkv_probe_empty(1, 0, None) == EINVAL
    pool = _pool()
    assert L.pkv_probe_paged_read(ctypes.byref(pool), 30, FAKE, 8, FAKE, 4, FAKE, None) == EINVAL  # 30 % 8
    assert L.pkv_probe_paged_read(ctypes.byref(pool), 32, None, 8, FAKE, 4, FAKE, None) == EINVAL
    assert L.pkv_probe_paged_read(ctypes.byref(pool), 32, FAKE, 0, FAKE, 4, FAKE, None) == EINVAL
    assert L.pkv_probe_paged_read(ctypes.byref(pool), 32, FAKE, 8, FAKE, 0, FAKE, None) == 0  # nothing to do


def test_fused_layer_plan_host():
    """The single-launch batch-1 layer's plan (host only): the
    Qwen2.5-0.5B-shaped layer fits 256 compute units at 128-token tables and
    up to 33 pages; batches above 1, the Llama-3.2-1B-shaped layer (123 MB of
    weights), and too few compute units for its weights take the multi-launch
    path; bad arguments are errors.  pkv_set_fused_layer returns the previous
    setting."""
    import synth
    qwen = pkv.make_config(synth.QWEN05, max_pos=4096, layers=1)
    assert pkv.fused_layer_plan(qwen, 1, 8, 16, 256) == 1
    assert pkv.fused_layer_plan(qwen, 1, 33, 16, 256) == 1
    assert pkv.fused_layer_plan(qwen, 1, 1, 256, 256) == 1   # one 256-token page
    assert pkv.fused_layer_plan(qwen, 2, 8, 16, 256) == 0
    assert pkv.fused_layer_plan(qwen, 1, 8, 16, 64) == 0      # 30 MB of weights on 64 CUs
    llama = pkv.make_config(synth.LLAMA1B, max_pos=4096, layers=1)
    assert pkv.fused_layer_plan(llama, 1, 64, 16, 256) == 0
    lib = pkv.lib()
    assert lib.pkv_fused_layer_plan(None, 1, 8, 16, 256) == -errno.EINVAL
    assert lib.pkv_fused_layer_plan(ctypes.byref(qwen), 1, 0, 16, 256) == -errno.EINVAL
    assert lib.pkv_fused_layer_plan(ctypes.byref(qwen), 1, 8, 32, 256) == -errno.ENOTSUP
    assert lib.pkv_fused_layer_plan(ctypes.byref(qwen), 1, 8, 16, 0) == -errno.EINVAL
    prev = pkv.set_fused_layer(False)
    try:
        assert pkv.set_fused_layer(False) == 0
    finally:
        pkv.set_fused_layer(prev)
