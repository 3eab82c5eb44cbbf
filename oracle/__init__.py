"""Plain CPU oracle of the batched paged-KV GQA decode step.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the product path
(``paged_kv_transformer_amd``) never does, and this package never imports it.

The decode arithmetic lives in ``oracle.c`` (FP32, single thread, contiguous
per-layer cache, two-pass softmax).  This module marshals numpy arrays into
it and loops over sequences, layers and tokens; every step of a batch is the
plain per-sequence computation repeated.  The sampler after the LM head is
plain numpy in float64 (a sort and a cumulative sum).

Parity pins (what each function is checked against, in tests/):
  bf16 rounding          torch's round-to-nearest-even conversion, and
                         hand-picked tie / carry / NaN cases
  rmsnorm                closed form RMS(y) = sqrt(ms / (ms + eps)) with w = 1,
                         scale invariance, division by w restores RMS
  matvec                 numpy float64 matmul on a non-square matrix
  rope                   identity at p = 0, pair norms kept, relative-position
                         inner products, pair 0 turns by exactly p radians,
                         per-pair frequency theta^(-2j/D), rotate-half pairing
  attention              n = 1 gives V_0, constant scores give the mean of V,
                         a dominant key gives its V, two-token closed form
                         fixes the 1/sqrt(D) scale, GQA equals MHA over
                         repeated KV, float64 online softmax equals two-pass
  pool gather / append   numpy views of each page as K [tile][head][d / 8]
                         [slot % 16][d % 8] and V [tile][head][d][slot % 16]
                         (16-token tiles), at 16- and 256-token pages
  split_pools /          the same views over separate K and V buffers; the
  whole_pool             two conversions undo each other
  layer, step            float64 brute force with a materialised softmax on
                         tiny shapes; all-zero weights leave x unchanged
  prefill                float64 brute force of the whole prompt at once with a
                         causal mask (last logits, argmax, every K/V row
                         written); a one-token prefill equals a decode step
  argmax                 numpy.argmax (first maximum)
  sample_token           closed forms: temperature 0, top-k 1 or top-p 0 give
                         the argmax; equal logits give token floor(u V); a
                         geometric distribution fixes the nucleus (the token
                         that crosses top-p is kept) and the renormalised
                         inverse CDF; temperature T on l equals 1 on l / T; a
                         grid of u reproduces the kept probabilities
Full-size layer and step outputs have no printed values on the source pages:
beyond the pins above they are "parity unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

_F = ctypes.c_float
_I = ctypes.c_int
_L = ctypes.c_long
_P = ctypes.c_void_p


def _load():
    global _LIB
    if _LIB is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        sig = {
            "orc_bf16_to_f32": (_F, [ctypes.c_uint16]),
            "orc_f32_to_bf16": (ctypes.c_uint16, [_F]),
            "orc_f32_to_bf16_array": (None, [_P, _P, _L]),
            "orc_rmsnorm": (None, [_P, _P, _I, _F, _P]),
            "orc_matvec": (None, [_P, _I, _I, _P, _P]),
            "orc_rope_cos_sin": (None, [_I, _I, _I, _F, _P, _P]),
            "orc_rope": (None, [_P, _I, _I, _I, _F]),
            "orc_silu": (_F, [_F]),
            "orc_argmax": (_I, [_P, _I]),
            "orc_attention": (None, [_P, _P, _P, _I, _I, _I, _I, _F, _P]),
            "orc_pool_gather": (None, [_P, _L, _I, _I, _I, _P, _I, _P, _P]),
            "orc_pool_append": (None, [_P, _L, _I, _I, _I, _P, _I, _P, _P]),
            "orc_layer_decode": (_I, [_I, _I, _I, _I, _I, _F, _F] + [_P] * 6
                                 + [_P, _P, _P, _I, _I, _P, _P, _I]),
            "orc_embed": (None, [_P, _I, _I, _P]),
            "orc_lm_head": (_I, [_P, _I, _I, _P, _F, _P, _P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _p(a, dtype):
    if a.dtype != dtype or not a.flags["C_CONTIGUOUS"]:
        raise TypeError("expected a C-contiguous %s array, got %s" % (np.dtype(dtype), a.dtype))
    return ctypes.c_void_p(a.ctypes.data)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("BF16 data must be passed as uint16 bit patterns")
    return a


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


# ------------------------------------------------------------------ BF16 ---

def bf16_to_f32(h):
    """Exact widening of BF16 bit patterns (uint16) to float32."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x):
    """Round float32 to BF16 (nearest, ties to even) with the oracle's C code."""
    x = _f32(x)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_f32_to_bf16_array(_p(x, np.float32), _p(out, np.uint16), x.size)
    return out


# ------------------------------------------------------------ basic ops ---

def rmsnorm(x, w, eps):
    x = _f32(x)
    w = _u16(w)
    y = np.empty_like(x)
    _load().orc_rmsnorm(_p(x, np.float32), _p(w, np.uint16), x.size, eps, _p(y, np.float32))
    return y


def matvec(W, x):
    W = _u16(W)
    x = _f32(x)
    rows, cols = W.shape
    assert x.size == cols
    y = np.empty(rows, dtype=np.float32)
    _load().orc_matvec(_p(W, np.uint16), rows, cols, _p(x, np.float32), _p(y, np.float32))
    return y


def rope_cos_sin(pos, j, D, theta):
    c, s = ctypes.c_float(), ctypes.c_float()
    _load().orc_rope_cos_sin(pos, j, D, theta, ctypes.byref(c), ctypes.byref(s))
    return np.float32(c.value), np.float32(s.value)


def rope(u, pos, theta):
    """Rotate a [heads, D] array (copy) by the RoPE angles of position pos."""
    u = np.array(u, dtype=np.float32, order="C", copy=True)
    heads, D = u.shape
    _load().orc_rope(_p(u, np.float32), heads, D, pos, theta)
    return u


def silu(z):
    return np.float32(_load().orc_silu(float(z)))


def argmax(v):
    v = _f32(v)
    return int(_load().orc_argmax(_p(v, np.float32), v.size))


def attention(q, kc, vc, kv_heads, scale):
    """q [hq, D] float32; kc, vc [n, kv_heads*D] float32 -> out [hq, D]."""
    q = _f32(q)
    kc = _f32(kc)
    vc = _f32(vc)
    hq, D = q.shape
    n = kc.shape[0]
    out = np.empty((hq, D), dtype=np.float32)
    _load().orc_attention(_p(q, np.float32), _p(kc, np.float32), _p(vc, np.float32), n,
                          hq, kv_heads, D, scale, _p(out, np.float32))
    return out


# ---------------------------------------------------------------- paging ---

class PoolGeometry:
    """Page geometry: T tokens per page; per page the BF16 K block
    followed by the V block, both in 16-token tiles: K [slot / 16][kv head]
    [d / 8][slot % 16][d % 8], V [slot / 16][kv head][d][slot % 16]."""

    def __init__(self, kv_heads, head_dim, page_tokens=16):
        self.kv_heads = kv_heads
        self.head_dim = head_dim
        self.page_tokens = page_tokens
        self.page_elems = 2 * kv_heads * page_tokens * head_dim


def pool_gather(pool, geo, bt_row, n):
    """Contiguous FP32 caches [n, kv_heads*D] of tokens 0..n-1 of one sequence."""
    pool = _u16(pool)
    bt_row = _i32(bt_row)
    row = geo.kv_heads * geo.head_dim
    kc = np.empty((n, row), dtype=np.float32)
    vc = np.empty((n, row), dtype=np.float32)
    _load().orc_pool_gather(_p(pool, np.uint16), geo.page_elems, geo.kv_heads, geo.head_dim,
                            geo.page_tokens, _p(bt_row, np.int32), n,
                            _p(kc, np.float32), _p(vc, np.float32))
    return kc, vc


def split_pools(pool, geo):
    """The same pages as separate K and V pools (the three-stage engine's
    paged KV cache keeps K and V in two caches indexed by one page number,
    its section 3.2): page p of the K pool is page p's K block, page p of
    the V pool its V block.  Returns (k_pool, v_pool), uint16 copies."""
    half = geo.page_elems // 2
    pages = np.asarray(_u16(pool)).reshape(-1, geo.page_elems)
    return pages[:, :half].reshape(-1).copy(), pages[:, half:].reshape(-1).copy()


def whole_pool(k_pool, v_pool, geo):
    """Inverse of split_pools: page p = K pool page p, then V pool page p."""
    half = geo.page_elems // 2
    k = np.asarray(_u16(k_pool)).reshape(-1, half)
    v = np.asarray(_u16(v_pool)).reshape(-1, half)
    return np.concatenate([k, v], axis=1).reshape(-1)


def pool_append(pool, geo, bt_row, pos, k_bits, v_bits):
    """Write one token's BF16 K and V ([kv_heads*D] uint16 each) in place."""
    _u16(pool)
    bt_row = _i32(bt_row)
    k_bits = _u16(k_bits)
    v_bits = _u16(v_bits)
    _load().orc_pool_append(_p(pool, np.uint16), geo.page_elems, geo.kv_heads, geo.head_dim,
                            geo.page_tokens, _p(bt_row, np.int32), pos,
                            _p(k_bits, np.uint16), _p(v_bits, np.uint16))


# ----------------------------------------------------------------- layer ---

_LAYER_KEYS = ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")


def layer_decode(shape, lw, x, kc, vc, pos, row_given=False):
    """One layer for one sequence.  kc/vc [cap, kv*D] float32 are updated in
    place (row pos).  Returns (x_out, k_new_bits, v_new_bits).  row_given:
    row pos already holds this token's K/V (teacher forcing in tests) and
    attention reads it as given; the returned bits are still this layer's
    own."""
    x = np.array(x, dtype=np.float32, copy=True)
    assert kc.dtype == np.float32 and kc.flags["C_CONTIGUOUS"]
    assert vc.dtype == np.float32 and vc.flags["C_CONTIGUOUS"]
    kvd = shape.kv_heads * shape.head_dim
    k_new = np.empty(kvd, dtype=np.uint16)
    v_new = np.empty(kvd, dtype=np.uint16)
    ws = [_u16(lw[k]) for k in _LAYER_KEYS]
    rc = _load().orc_layer_decode(
        shape.hidden, shape.heads, shape.kv_heads, shape.head_dim, shape.inter,
        shape.eps, shape.theta, *[_p(w, np.uint16) for w in ws],
        _p(x, np.float32), _p(kc, np.float32), _p(vc, np.float32), kc.shape[0], pos,
        _p(k_new, np.uint16), _p(v_new, np.uint16), int(bool(row_given)))
    if rc != 0:
        raise ValueError("position %d outside the cache of %d rows" % (pos, kc.shape[0]))
    return x, k_new, v_new


def embed(E, token):
    E = _u16(E)
    H = E.shape[1]
    x = np.empty(H, dtype=np.float32)
    _load().orc_embed(_p(E, np.uint16), H, int(token), _p(x, np.float32))
    return x


def lm_head(E, final_norm, eps, x):
    """(logits float32 [V], argmax) of the final RMSNorm + tied LM head."""
    E = _u16(E)
    fn = _u16(final_norm)
    x = _f32(x)
    V, H = E.shape
    logits = np.empty(V, dtype=np.float32)
    best = _load().orc_lm_head(_p(E, np.uint16), V, H, _p(fn, np.uint16), eps,
                               _p(x, np.float32), _p(logits, np.float32))
    return logits, int(best)


# ----------------------------------------------- batched, paged compositions ---

def paged_attention(pool, geo, q, block_table, lens, scale, seqs=None):
    """Attention-only call: q [B, hq, D] (float32 values), block_table
    [B, max_pages], lens [B] -> out [B, hq, D] float32.  Each sequence's
    pages are gathered into a contiguous cache, then the definition runs."""
    q = _f32(q)
    B = q.shape[0]
    out = np.zeros(q.shape, dtype=np.float32)
    for b in (range(B) if seqs is None else seqs):
        n = int(lens[b])
        kc, vc = pool_gather(pool, geo, block_table[b], n)
        out[b] = attention(q[b], kc, vc, geo.kv_heads, scale)
    return out


def layer_decode_paged(shape, lw, hidden, pool, geo, block_table, positions, seqs=None):
    """One layer over a batch.  Token p_b is new; 0..p_b-1 are read from the
    pool.  Returns (hidden_out [B,H], k_new [B,kv*D], v_new [B,kv*D]); the
    pool is not modified (apply the appends with pool_append)."""
    hidden = _f32(hidden)
    B = hidden.shape[0]
    out = hidden.copy()
    kvd = shape.kv_heads * shape.head_dim
    k_new = np.zeros((B, kvd), dtype=np.uint16)
    v_new = np.zeros((B, kvd), dtype=np.uint16)
    for b in (range(B) if seqs is None else seqs):
        p = int(positions[b])
        kc = np.zeros((p + 1, kvd), dtype=np.float32)
        vc = np.zeros((p + 1, kvd), dtype=np.float32)
        kc[:p], vc[:p] = pool_gather(pool, geo, block_table[b], p)
        out[b], k_new[b], v_new[b] = layer_decode(shape, lw, hidden[b], kc, vc, p)
    return out, k_new, v_new


def decode_step_paged(shape, weights, pool, geo, block_tables, positions, tokens,
                      seqs=None, want_logits=True):
    """Full decode step over a batch: embedding, every layer, final norm,
    tied LM head, argmax.  block_tables [L, B, max_pages].  Returns
    (logits [B, V] or None, next_tokens [B], k_new [L, B, kv*D],
    v_new [L, B, kv*D]).  Sequences not in `seqs` are left zero / -1."""
    B = len(tokens)
    seqs = list(range(B)) if seqs is None else list(seqs)
    L = shape.layers
    kvd = shape.kv_heads * shape.head_dim
    V = weights["embed"].shape[0]
    logits = np.zeros((B, V), dtype=np.float32) if want_logits else None
    nxt = np.full(B, -1, dtype=np.int32)
    k_new = np.zeros((L, B, kvd), dtype=np.uint16)
    v_new = np.zeros((L, B, kvd), dtype=np.uint16)
    for b in seqs:
        p = int(positions[b])
        x = embed(weights["embed"], int(tokens[b]))
        for l in range(L):
            kc = np.zeros((p + 1, kvd), dtype=np.float32)
            vc = np.zeros((p + 1, kvd), dtype=np.float32)
            kc[:p], vc[:p] = pool_gather(pool, geo, block_tables[l, b], p)
            x, k_new[l, b], v_new[l, b] = layer_decode(shape, weights["layers"][l], x, kc, vc, p)
        lg, best = lm_head(weights["embed"], weights["final_norm"], shape.eps, x)
        if want_logits:
            logits[b] = lg
        nxt[b] = best
    return logits, nxt, k_new, v_new


def prefill_paged(shape, weights, pool, geo, block_tables, start_pos, tokens, want_logits=True):
    """Prefill of one sequence's prompt: tokens[t] sits at position
    start_pos + t, and tokens 0..start_pos-1 are already in the pool.  The
    plain definition of causal prefill is the prompt run one token at a time:
    each token is a decode step of this sequence at its own position whose
    K and V are appended to the pool before the next token runs ("Inference
    from Scratch", dense causal prefill and page-pool bullets: prefill fills
    the prompt's pages, attention is causal).  block_tables [L, max_pages]
    is this sequence's table per layer.  Returns (logits of the last token
    [V] or None, its argmax, the pool after every append)."""
    pool = np.array(_u16(pool), copy=True)
    L = shape.layers
    lg = best = None
    for t, tok in enumerate(np.asarray(tokens)):
        p = int(start_pos) + t
        x = embed(weights["embed"], int(tok))
        for l in range(L):
            kc, vc = pool_gather(pool, geo, block_tables[l], p)
            kc = np.concatenate([kc, np.zeros((1, kc.shape[1]), np.float32)])
            vc = np.concatenate([vc, np.zeros((1, vc.shape[1]), np.float32)])
            x, k_bits, v_bits = layer_decode(shape, weights["layers"][l], x, kc, vc, p)
            pool_append(pool, geo, block_tables[l], p, k_bits, v_bits)
        if t == len(tokens) - 1:
            lg, best = lm_head(weights["embed"], weights["final_norm"], shape.eps, x)
    return (lg if want_logits else None), best, pool


# -------------------------------------------------------------- sampling ---

# Decisions of the sampler within this much probability mass (of a total
# of 1) of a boundary may go either way in a computation that is correct to
# FP32 rounding: the probabilities of a vocabulary-sized softmax come out of
# exponentials of arguments up to ~30 in magnitude, whose FP32 rounding moves
# each probability by up to ~2e-6 of itself.
SAMPLE_EPS = 1e-5


def sample_token(logits, temperature, top_p, top_k, u, eps=SAMPLE_EPS):
    """Sampling of one sequence's next token from its logits ("手写LLM推理引擎"
    §3.3 logits post-processing and §2.4 decoding strategies; llmc 五 plans
    temperature / top-k / top-p after greedy):
      1. z = logits / temperature; temperature <= 0 is greedy (first argmax);
      2. p = softmax(z);
      3. top-p: order the tokens by decreasing p (equal logits: lower index
         first) and keep the smallest prefix whose cumulative probability
         reaches top_p (at least one token; top_p >= 1 keeps all);
      4. then top-k: keep at most top_k of them (top_k <= 0: no limit);
      5. renormalise p over the kept tokens and return the first kept token,
         in vocabulary order, whose cumulative probability exceeds u (u in
         [0, 1), the uniform draw, an input).
    float64 throughout.  Returns (token, acceptable): acceptable holds every
    token a computation within eps of these decisions (the nucleus boundary
    and the inverse-CDF step) could also return."""
    l = np.asarray(logits, dtype=np.float64)
    V = l.size
    if temperature <= 0.0:
        t = int(np.argmax(l))
        return t, {t}
    e = np.exp((l - l.max()) / float(temperature))
    p = e / e.sum()
    order = np.lexsort((np.arange(V), -l))
    cum = np.cumsum(p[order])

    def prefix_len(target):
        if target >= 1.0:
            return V
        if target <= 0.0:
            return 1
        return min(V, int(np.searchsorted(cum, target, side="left")) + 1)

    def limit(n):
        return n if top_k <= 0 else min(n, int(top_k))

    def draw(n, uu):
        kept = np.sort(order[:n])
        c = np.cumsum(p[kept] / p[kept].sum())
        return kept, c, min(int(np.searchsorted(c, uu, side="right")), n - 1)

    L = limit(prefix_len(top_p))
    kept, c, i = draw(L, u)
    token = int(kept[i])
    acceptable = set()
    lens = {L}
    if 0.0 < top_p < 1.0:
        lens |= {limit(prefix_len(top_p - eps)), limit(prefix_len(top_p + eps))}
        lens |= set(range(min(lens), max(lens) + 1))
    for n in sorted(lens):
        kn, cn, _ = draw(n, u)
        lo = int(np.searchsorted(cn, u - eps, side="right"))
        hi = int(np.searchsorted(cn, u + eps, side="right"))
        acceptable |= {int(kn[j]) for j in range(min(lo, n - 1), min(hi, n - 1) + 1)}
    return token, acceptable
