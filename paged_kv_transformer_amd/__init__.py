"""Paged-KV GQA decode on MI355X (gfx950): ctypes binding of libpkv.so.

The binding only marshals arguments into the C ABI of ``include/pkv.h``:
torch supplies device memory and the stream, every step of the computation
runs in the library's HIP kernels.  There is no fallback: if ``libpkv.so``
is missing the first call raises.

Entry points (same names as the C ABI): ``kv_pool_create``,
``kv_pool_create_split``, ``kv_append``,
``paged_gqa_decode``, ``decoder_layer_decode``, ``decode_step``, plus
``workspace_bytes``, ``attention_workspace_bytes``, ``workspace_init``,
``rope_table``, ``pack_weight``, ``device_error``, ``set_fused_layer`` and
``fused_layer_plan``.
"""
import ctypes
import errno
import os

import torch

# The library this binding loads: the in-tree build, or another build of the
# same sources named by PKV_LIBRARY (the host-sanitized libpkv_san.so).
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PAGE_TOKENS = 16
HEAD_DIM = 64
DEVERR_PAGE, DEVERR_LENGTH, DEVERR_ROPE, DEVERR_TOKEN, DEVERR_SYNC = 1, 2, 4, 8, 16
PACK_ROWS, PACK_QKV, PACK_GATE_UP, PACK_QKV128 = 0, 1, 2, 3


class PkvError(RuntimeError):
    def __init__(self, fn, rc):
        self.rc = rc
        name = errno.errorcode.get(-rc, str(rc))
        super().__init__("%s failed: -%s (%d)" % (fn, name, rc))


class Config(ctypes.Structure):
    _fields_ = [("hidden_size", ctypes.c_int32), ("num_hidden_layers", ctypes.c_int32),
                ("num_attention_heads", ctypes.c_int32), ("num_key_value_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("intermediate_size", ctypes.c_int32),
                ("vocab_size", ctypes.c_int32), ("max_position_embeddings", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_norm_eps", ctypes.c_float)]


class Pool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("bytes", ctypes.c_int64), ("page_bytes", ctypes.c_int64),
                ("num_pages", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("v_base", ctypes.c_void_p)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in
                ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")]


class ModelWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LayerWeights)),
                ("rope_cos", ctypes.c_void_p), ("rope_sin", ctypes.c_void_p)]


LAYER_KEYS = ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")

_lib = None


def lib():
    """The loaded library with argument types set (raw calls return rc)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("the HIP library is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        PP = ctypes.POINTER(Pool)
        sigs = {
            "kv_pool_create": (ctypes.c_int, [P, I64, I32, I32, I32, PP]),
            "kv_pool_create_split": (ctypes.c_int, [P, P, I64, I32, I32, I32, PP]),
            "kv_append": (ctypes.c_int, [PP, P, I32, P, P, P, I32, P, P]),
            "paged_gqa_decode": (ctypes.c_int, [PP, P, I32, P, I32, P, I32, F, P, P, SZ, P]),
            "paged_gqa_decode_noalloc": (ctypes.c_int, [PP, P, I32, P, I32, P, I32, F, P, P, P]),
            "decoder_layer_decode": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(LayerWeights),
                                                    P, P, PP, P, I32, P, I32, P, P, SZ, P]),
            "decode_step": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(ModelWeights), PP, P,
                                           I32, P, P, I32, P, P, P, SZ, P]),
            "prefill": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(ModelWeights), PP, P, I32, I32,
                                       P, I32, P, P, P, SZ, P]),
            "pkv_prefill_workspace_bytes": (SZ, [ctypes.POINTER(Config), I32, I32]),
            "sample_tokens": (ctypes.c_int, [P, I32, I32, P, P, P, P, P, P, SZ, P]),
            "pkv_sample_workspace_bytes": (SZ, [I32, I32]),
            "pkv_workspace_bytes": (SZ, [ctypes.POINTER(Config), I32, I32, I32]),
            "pkv_attention_workspace_bytes": (SZ, [I32, I32, I32, I32, I32, I32]),
            "pkv_workspace_init": (ctypes.c_int, [P, SZ, P]),
            "pkv_rope_table": (ctypes.c_int, [F, I32, I32, P, P, P]),
            "pkv_packed_weight_bytes": (SZ, [I32, I32, I32]),
            "pkv_pack_weight": (ctypes.c_int, [P, I32, I32, I32, P, P]),
            "pkv_device_error": (ctypes.c_int, [P, P]),
            "pkv_probe_read": (ctypes.c_int, [P, I64, I32, P, P]),
            "pkv_probe_paged_read": (ctypes.c_int, [PP, I32, P, I32, P, I32, P, P]),
            "pkv_probe_empty": (ctypes.c_int, [I32, I32, P]),
            "pkv_set_fused_layer": (ctypes.c_int, [I32]),
            "pkv_fused_layer_plan": (ctypes.c_int, [ctypes.POINTER(Config), I32, I32, I32, I32]),
            "pkv_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn, rc):
    if rc < 0:
        raise PkvError(fn, rc)
    return rc


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


_BF16_DTYPES = (torch.bfloat16, torch.int16, torch.uint16)


def _dev(t, dtypes, what):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % what)
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU" % what)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (what, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    return t.data_ptr()


# The library takes plain pointers and cannot see how large a buffer is: the
# wrappers check every tensor against the elements the call reads or writes
# before anything reaches the device (a short buffer would otherwise be
# read or written past its end).

def _at_least(t, n, what):
    if t.numel() < n:
        raise ValueError("%s holds %d elements; the call uses %d" % (what, t.numel(), n))


def _table(t, rows, what):
    """A block table [rows or more, max_pages]."""
    if t.dim() != 2 or t.shape[0] < rows or t.shape[1] < 1:
        raise ValueError("%s must be [>= %d, max_pages], got %s" % (what, rows, tuple(t.shape)))


def _bytes_at_least(t, nbytes, what):
    if t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes; the call reads %d" % (what, t.numel() * t.element_size(), nbytes))


def _check_layer(cfg, layer, what="layer"):
    H, I, D = cfg.hidden_size, cfg.intermediate_size, cfg.head_dim
    QKV = (cfg.num_attention_heads + 2 * cfg.num_key_value_heads) * D
    need = {"attn_norm": 2 * H, "mlp_norm": 2 * H,
            "w_qkv": packed_weight_bytes(QKV, H, qkv_pack_kind(D) if D in (64, 128) else PACK_QKV),
            "w_o": packed_weight_bytes(H, cfg.num_attention_heads * D, PACK_ROWS),
            "w_gate_up": packed_weight_bytes(2 * I, H, PACK_GATE_UP),
            "w_down": packed_weight_bytes(H, I, PACK_ROWS)}
    for k, n in need.items():
        _bytes_at_least(layer.tensors[k], n, "%s.%s" % (what, k))


def _check_rope(cfg, rope_cos, rope_sin):
    n = cfg.max_position_embeddings * (cfg.head_dim // 2)
    _at_least(rope_cos, n, "rope_cos")
    _at_least(rope_sin, n, "rope_sin")


def _check_model(cfg, model):
    if len(model.layers) < cfg.num_hidden_layers:
        raise ValueError("the model has %d layers, the config %d" % (len(model.layers), cfg.num_hidden_layers))
    _bytes_at_least(model.embed, packed_weight_bytes(cfg.vocab_size, cfg.hidden_size, PACK_ROWS), "embed")
    _at_least(model.final_norm, cfg.hidden_size, "final_norm")
    _check_rope(cfg, model.rope_cos, model.rope_sin)
    for l in range(cfg.num_hidden_layers):
        _check_layer(cfg, model.layers[l], "layer %d" % l)


def make_config(shape, max_pos=None, layers=None):
    """Config from any object with the llmc header fields' meaning
    (hidden, layers, heads, kv_heads, head_dim, inter, vocab, max_pos,
    theta, eps)."""
    return Config(shape.hidden, shape.layers if layers is None else layers, shape.heads,
                  shape.kv_heads, shape.head_dim, shape.inter, shape.vocab,
                  shape.max_pos if max_pos is None else max_pos, shape.theta, shape.eps)


# ------------------------------------------------------------------ pool ---

def kv_pool_create(pool_tensor, num_kv_heads, head_dim=HEAD_DIM, page_tokens=PAGE_TOKENS):
    """Describe a device tensor (any dtype) as a page pool; returns a Pool."""
    if pool_tensor.device.type != "cuda" or not pool_tensor.is_contiguous():
        raise ValueError("pool must be a contiguous GPU tensor")
    out = Pool()
    nbytes = pool_tensor.numel() * pool_tensor.element_size()
    _check("kv_pool_create", lib().kv_pool_create(pool_tensor.data_ptr(), nbytes, num_kv_heads,
                                                  head_dim, page_tokens, ctypes.byref(out)))
    out._tensor = pool_tensor
    return out


def kv_pool_create_split(k_tensor, v_tensor, num_kv_heads, head_dim=HEAD_DIM,
                         page_tokens=PAGE_TOKENS):
    """Two device tensors of equal size as separate K and V pools."""
    for t in (k_tensor, v_tensor):
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("pools must be contiguous GPU tensors")
    nbytes = k_tensor.numel() * k_tensor.element_size()
    if v_tensor.numel() * v_tensor.element_size() != nbytes:
        raise ValueError("the K and V pools must have the same size")
    out = Pool()
    _check("kv_pool_create_split", lib().kv_pool_create_split(
        k_tensor.data_ptr(), v_tensor.data_ptr(), nbytes, num_kv_heads, head_dim, page_tokens,
        ctypes.byref(out)))
    out._tensor = (k_tensor, v_tensor)
    return out


def kv_append(pool, block_table, positions, k_new, v_new, stream=None, dev_error=None):
    """dev_error: None, or a device tensor (a workspace from
    alloc_workspace, read with device_error) whose first 32-bit word takes
    the PKV_DEVERR_* bits of sequences that could not be written."""
    B = positions.numel()
    _table(block_table, B, "block_table")
    _at_least(k_new, B * pool.num_kv_heads * pool.head_dim, "k_new")
    _at_least(v_new, B * pool.num_kv_heads * pool.head_dim, "v_new")
    bt = _dev(block_table, (torch.int32,), "block_table")
    err = None
    if dev_error is not None:
        _bytes_at_least(dev_error, 4, "dev_error")
        err = _dev(dev_error, (torch.uint8, torch.int32), "dev_error")
    _check("kv_append", lib().kv_append(
        ctypes.byref(pool), bt, block_table.shape[-1], _dev(positions, (torch.int32,), "positions"),
        _dev(k_new, _BF16_DTYPES, "k_new"), _dev(v_new, _BF16_DTYPES, "v_new"), B, err, _stream(stream)))


# ------------------------------------------------------------- workspace ---

def attention_workspace_bytes(num_q_heads, num_kv_heads, batch, max_pages, head_dim=HEAD_DIM,
                              page_tokens=PAGE_TOKENS):
    return lib().pkv_attention_workspace_bytes(num_q_heads, num_kv_heads, head_dim, batch, max_pages,
                                               page_tokens)


def workspace_bytes(cfg, batch, max_pages, page_tokens=PAGE_TOKENS):
    return lib().pkv_workspace_bytes(ctypes.byref(cfg), batch, max_pages, page_tokens)


def alloc_workspace(nbytes, device="cuda", stream=None):
    """A zero-initialised workspace tensor of at least nbytes (uint8)."""
    ws = torch.empty(max(256, (nbytes + 255) // 256 * 256), dtype=torch.uint8, device=device)
    workspace_init(ws, stream)
    return ws


def workspace_init(ws, stream=None):
    _check("pkv_workspace_init", lib().pkv_workspace_init(
        _dev(ws, (torch.uint8,), "workspace"), ws.numel(), _stream(stream)))


def set_fused_layer(enable):
    """Switch the single-launch batch-1 layer on or off; returns the
    previous setting."""
    return lib().pkv_set_fused_layer(1 if enable else 0)


def fused_layer_plan(cfg, batch, max_pages, page_tokens=PAGE_TOKENS, compute_units=256):
    """1 if such calls run each layer as one launch, else 0."""
    return _check("pkv_fused_layer_plan", lib().pkv_fused_layer_plan(
        ctypes.byref(cfg), batch, max_pages, page_tokens, compute_units))


def device_error(ws, stream=None):
    return _check("pkv_device_error", lib().pkv_device_error(
        _dev(ws, (torch.uint8,), "workspace"), _stream(stream)))


def probe_read(buf, sink, workgroups=1024, nbytes=None, stream=None):
    """Stream nbytes (default: all) of the device tensor buf once (a
    measurement kernel: no arithmetic, no stores)."""
    n = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check("pkv_probe_read", lib().pkv_probe_read(buf.data_ptr(), n, workgroups,
                                                  _dev(sink, (torch.float32,), "sink"), _stream(stream)))


def probe_paged_read(pool, num_q_heads, block_table, context_lens, sink, stream=None):
    """The K/V loads of one paged_gqa_decode call, without its arithmetic."""
    B = context_lens.numel()
    _table(block_table, B, "block_table")
    _check("pkv_probe_paged_read", lib().pkv_probe_paged_read(
        ctypes.byref(pool), num_q_heads, _dev(block_table, (torch.int32,), "block_table"),
        block_table.shape[-1], _dev(context_lens, (torch.int32,), "context_lens"), B,
        _dev(sink, (torch.float32,), "sink"), _stream(stream)))


def probe_empty(launches, workgroups=1, stream=None):
    """`launches` empty kernels (the cost of a launch)."""
    _check("pkv_probe_empty", lib().pkv_probe_empty(launches, workgroups, _stream(stream)))


def rope_table(theta, max_pos, head_dim=HEAD_DIM, device="cuda", stream=None):
    """(cos, sin) FP32 [max_pos, head_dim/2] computed by the library's kernel."""
    c = torch.empty((max_pos, head_dim // 2), dtype=torch.float32, device=device)
    s = torch.empty_like(c)
    _check("pkv_rope_table", lib().pkv_rope_table(theta, head_dim, max_pos, c.data_ptr(),
                                                  s.data_ptr(), _stream(stream)))
    return c, s


# ---------------------------------------------------------------- packing ---

def packed_weight_bytes(rows, cols, layout):
    return lib().pkv_packed_weight_bytes(rows, cols, layout)


def pack_weight(src, layout, stream=None):
    """Packed copy (int16 device tensor) of a row-major BF16 [rows, cols]
    device matrix, in the projections' tiled layout."""
    if src.dim() != 2:
        raise ValueError("src must be a [rows, cols] matrix, got %s" % (tuple(src.shape),))
    rows, cols = src.shape
    nbytes = packed_weight_bytes(rows, cols, layout)
    if nbytes == 0:
        raise ValueError("cannot pack a [%d, %d] matrix with layout %d" % (rows, cols, layout))
    dst = torch.empty(nbytes // 2, dtype=torch.int16, device=src.device)
    _check("pkv_pack_weight", lib().pkv_pack_weight(_dev(src, _BF16_DTYPES, "src"), rows, cols, layout,
                                                    dst.data_ptr(), _stream(stream)))
    return dst


# ------------------------------------------------------------- attention ---

def paged_gqa_decode(pool, q, block_table, context_lens, scale, out, workspace, stream=None):
    """q [B, Hq, D] BF16, block_table [B, max_pages] int32, context_lens [B]
    int32, out [B, Hq, D] FP32 (written); D is the pool's head width."""
    if q.dim() != 3 or q.shape[2] != pool.head_dim:
        raise ValueError("q must be [B, Hq, %d], got %s" % (pool.head_dim, tuple(q.shape)))
    B, Hq = q.shape[0], q.shape[1]
    _table(block_table, B, "block_table")
    _at_least(context_lens, B, "context_lens")
    _at_least(out, B * Hq * pool.head_dim, "out")
    _check("paged_gqa_decode", lib().paged_gqa_decode(
        ctypes.byref(pool), _dev(q, _BF16_DTYPES, "q"), Hq,
        _dev(block_table, (torch.int32,), "block_table"), block_table.shape[-1],
        _dev(context_lens, (torch.int32,), "context_lens"), B, scale,
        _dev(out, (torch.float32,), "out"), _dev(workspace, (torch.uint8,), "workspace"),
        workspace.numel(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20


def paged_gqa_decode_noalloc(pool, q, block_table, context_lens, scale, out, dev_error, stream=None):
    """paged_gqa_decode without a workspace: the library's own per-GPU
    scratch array holds the split records (calls that overlap on one GPU
    race on it); dev_error is a device tensor of at least 4 bytes whose first
    32-bit word takes the PKV_DEVERR_* bits (a workspace from
    alloc_workspace, read and cleared with device_error, will do)."""
    if q.dim() != 3 or q.shape[2] != pool.head_dim:
        raise ValueError("q must be [B, Hq, %d], got %s" % (pool.head_dim, tuple(q.shape)))
    B, Hq = q.shape[0], q.shape[1]
    _table(block_table, B, "block_table")
    _at_least(context_lens, B, "context_lens")
    _at_least(out, B * Hq * pool.head_dim, "out")
    _bytes_at_least(dev_error, 4, "dev_error")
    _check("paged_gqa_decode_noalloc", lib().paged_gqa_decode_noalloc(
        ctypes.byref(pool), _dev(q, _BF16_DTYPES, "q"), Hq,
        _dev(block_table, (torch.int32,), "block_table"), block_table.shape[-1],
        _dev(context_lens, (torch.int32,), "context_lens"), B, scale,
        _dev(out, (torch.float32,), "out"), _dev(dev_error, (torch.uint8, torch.int32), "dev_error"),
        _stream(stream)))


# ---------------------------------------------------------------- layers ---

class DeviceLayer:
    """One layer's device weights (matrices already packed) and the C
    struct pointing at them."""

    def __init__(self, tensors):
        self.tensors = {k: tensors[k] for k in LAYER_KEYS}
        for k, t in self.tensors.items():
            _dev(t, _BF16_DTYPES, k)
        self.c = LayerWeights(*[self.tensors[k].data_ptr() for k in LAYER_KEYS])


class DeviceModel:
    """Whole-model device weights (packed embedding, final_norm, layers,
    RoPE tables)."""

    def __init__(self, embed, final_norm, layers, rope_cos, rope_sin):
        self.embed, self.final_norm = embed, final_norm
        self.layers = [l if isinstance(l, DeviceLayer) else DeviceLayer(l) for l in layers]
        self.rope_cos, self.rope_sin = rope_cos, rope_sin
        self._arr = (LayerWeights * len(self.layers))(*[l.c for l in self.layers])
        self.c = ModelWeights(_dev(embed, _BF16_DTYPES, "embed"), _dev(final_norm, _BF16_DTYPES, "final_norm"),
                              ctypes.cast(self._arr, ctypes.POINTER(LayerWeights)),
                              _dev(rope_cos, (torch.float32,), "rope_cos"),
                              _dev(rope_sin, (torch.float32,), "rope_sin"))


def decoder_layer_decode(cfg, layer, rope_cos, rope_sin, pool, block_table, positions, hidden,
                         workspace, stream=None):
    """hidden [B, H] FP32 is updated in place; block_table [B, max_pages]."""
    B = positions.numel()
    _table(block_table, B, "block_table")
    _at_least(hidden, B * cfg.hidden_size, "hidden")
    _check_rope(cfg, rope_cos, rope_sin)
    _check_layer(cfg, layer)
    _check("decoder_layer_decode", lib().decoder_layer_decode(
        ctypes.byref(cfg), ctypes.byref(layer.c), _dev(rope_cos, (torch.float32,), "rope_cos"),
        _dev(rope_sin, (torch.float32,), "rope_sin"), ctypes.byref(pool),
        _dev(block_table, (torch.int32,), "block_table"), block_table.shape[-1],
        _dev(positions, (torch.int32,), "positions"), B, _dev(hidden, (torch.float32,), "hidden"),
        _dev(workspace, (torch.uint8,), "workspace"), workspace.numel(), _stream(stream)))


def decode_step(cfg, model, pool, block_tables, positions, token_ids, logits, next_tokens,
                workspace, stream=None):
    """block_tables [L, B, max_pages]; logits [B, V] FP32 or None."""
    B = positions.numel()
    L = cfg.num_hidden_layers
    if block_tables.dim() != 3 or block_tables.shape[0] < L or block_tables.shape[1] != B:
        raise ValueError("block_tables must be [>= %d, %d, max_pages], got %s" % (L, B, tuple(block_tables.shape)))
    _at_least(token_ids, B, "token_ids")
    _at_least(next_tokens, B, "next_tokens")
    if logits is not None:
        _at_least(logits, B * cfg.vocab_size, "logits")
    _check_model(cfg, model)
    _check("decode_step", lib().decode_step(
        ctypes.byref(cfg), ctypes.byref(model.c), ctypes.byref(pool),
        _dev(block_tables, (torch.int32,), "block_tables"), block_tables.shape[-1],
        _dev(positions, (torch.int32,), "positions"), _dev(token_ids, (torch.int32,), "token_ids"), B,
        None if logits is None else _dev(logits, (torch.float32,), "logits"),
        _dev(next_tokens, (torch.int32,), "next_tokens"), _dev(workspace, (torch.uint8,), "workspace"),
        workspace.numel(), _stream(stream)))


def prefill_workspace_bytes(cfg, num_tokens, max_pages):
    return lib().pkv_prefill_workspace_bytes(ctypes.byref(cfg), num_tokens, max_pages)


def prefill(cfg, model, pool, block_tables, start_pos, token_ids, logits, next_token, workspace,
            stream=None):
    """Prefill of one sequence: block_tables [L, max_pages] (its table per
    layer), token_ids [T] at positions start_pos ..; logits [V] FP32 or None
    (the last token's), next_token [1] int32."""
    L = cfg.num_hidden_layers
    _table(block_tables, L, "block_tables")
    _at_least(next_token, 1, "next_token")
    if logits is not None:
        _at_least(logits, cfg.vocab_size, "logits")
    _check_model(cfg, model)
    _check("prefill", lib().prefill(
        ctypes.byref(cfg), ctypes.byref(model.c), ctypes.byref(pool),
        _dev(block_tables, (torch.int32,), "block_tables"), block_tables.shape[-1], int(start_pos),
        _dev(token_ids, (torch.int32,), "token_ids"), token_ids.numel(),
        None if logits is None else _dev(logits, (torch.float32,), "logits"),
        _dev(next_token, (torch.int32,), "next_token"), _dev(workspace, (torch.uint8,), "workspace"),
        workspace.numel(), _stream(stream)))


# ------------------------------------------------------- host -> device ---

def sample_workspace_bytes(batch, vocab):
    return lib().pkv_sample_workspace_bytes(batch, vocab)


def sample_tokens(logits, temperature, top_p, top_k, u, tokens, workspace, stream=None):
    """logits [B, V] FP32; temperature, top_p, u [B] FP32; top_k [B] int32;
    tokens [B] int32 (written)."""
    if logits.dim() != 2:
        raise ValueError("logits must be [B, V], got %s" % (tuple(logits.shape),))
    B, V = logits.shape
    for t, what in ((temperature, "temperature"), (top_p, "top_p"), (top_k, "top_k"), (u, "u"),
                    (tokens, "tokens")):
        _at_least(t, B, what)
    _check("sample_tokens", lib().sample_tokens(
        _dev(logits, (torch.float32,), "logits"), B, V, _dev(temperature, (torch.float32,), "temperature"),
        _dev(top_p, (torch.float32,), "top_p"), _dev(top_k, (torch.int32,), "top_k"),
        _dev(u, (torch.float32,), "u"), _dev(tokens, (torch.int32,), "tokens"),
        _dev(workspace, (torch.uint8,), "workspace"), workspace.numel(), _stream(stream)))


def to_device(a, device="cuda"):
    """numpy array -> contiguous device tensor (uint16 BF16 bits -> int16)."""
    import numpy as np
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def qkv_pack_kind(head_dim):
    """Packed layout of w_qkv for heads of width head_dim (64 or 128)."""
    if head_dim == 64:
        return PACK_QKV
    if head_dim == 128:
        return PACK_QKV128
    raise ValueError("head_dim must be 64 or 128, got %r" % (head_dim,))


def upload_layer(lw, device="cuda", head_dim=HEAD_DIM):
    """Row-major BF16 host matrices -> device, packed by the library."""
    pack = {"w_qkv": qkv_pack_kind(head_dim), "w_o": PACK_ROWS, "w_gate_up": PACK_GATE_UP,
            "w_down": PACK_ROWS}
    t = {}
    for k in LAYER_KEYS:
        d = to_device(lw[k], device)
        t[k] = pack_weight(d, pack[k]) if k in pack else d
    return DeviceLayer(t)


def upload_model(weights, theta, max_pos, device="cuda", head_dim=HEAD_DIM):
    """weights: {'embed', 'final_norm', 'layers': [layer dicts]} of BF16 bits
    (row-major); the matrices are packed on the device."""
    c, s = rope_table(theta, max_pos, head_dim=head_dim, device=device)
    embed = pack_weight(to_device(weights["embed"], device), PACK_ROWS)
    return DeviceModel(embed, to_device(weights["final_norm"], device),
                       [upload_layer(lw, device, head_dim) for lw in weights["layers"]], c, s)
