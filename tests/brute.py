"""Float64 brute force of the decode step for tiny shapes (test helper).

Written independently of the oracle's C code and in a different form: whole
matrices, a materialised softmax over all scores, RoPE in the rotate-half
vector form x*cos + rotate_half(x)*sin, numpy indexing of the pool viewed
per page as a K block [kv head][slot][d] and a V block [kv head][d][slot].
Only the BF16 storage of appended K/V is mirrored (rounded with torch's
conversion), since the pool holds BF16.
"""
import numpy as np
import torch


def bf16_bits_to_f64(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_round_f64(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.float32).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def rmsnorm(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def rope(u, pos, theta):
    """u [..., heads, D] float64 rotated at position pos (rotate-half pairs)."""
    D = u.shape[-1]
    j = np.arange(D // 2, dtype=np.float64)
    ang = pos * theta ** (-2.0 * j / D)
    cos = np.concatenate([np.cos(ang), np.cos(ang)])
    sin = np.concatenate([np.sin(ang), np.sin(ang)])
    rot = np.concatenate([-u[..., D // 2:], u[..., :D // 2]], axis=-1)
    return u * cos + rot * sin


def softmax_attention(q, K, V, scale):
    """q [hq, D]; K, V [n, hkv, D] -> [hq, D], via repeated KV and a
    materialised softmax."""
    hq, D = q.shape
    hkv = K.shape[1]
    Kr = np.repeat(K, hq // hkv, axis=1)          # [n, hq, D]
    Vr = np.repeat(V, hq // hkv, axis=1)
    s = np.einsum("hd,nhd->hn", q, Kr) * scale     # [hq, n]
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    return np.einsum("hn,nhd->hd", p, Vr)


def pool_view(pool, kv_heads, head_dim, page_tokens=16):
    """Views of the pool's pages (writable, no copy), token slot = 16 tile +
    s (16-token tiles): K [page][tile][head][c][s][e] with d = 8 c + e, and V
    [page][tile][head][d][s]."""
    blk = kv_heads * page_tokens * head_dim
    pages = np.asarray(pool).reshape(-1, 2 * blk)
    return (pages[:, :blk].reshape(-1, page_tokens // 16, kv_heads, head_dim // 8, 16, 8),
            pages[:, blk:].reshape(-1, page_tokens // 16, kv_heads, head_dim, 16))


def k_of(kv, page, slot):
    """The K view's [head][d] entries of one token (a writable view)."""
    return kv[page, slot // 16, :, :, slot % 16, :]


def gather(pool, kv_heads, head_dim, bt_row, n, page_tokens=16):
    """K, V [n, hkv, D] float64 of tokens 0..n-1."""
    kv, vv = pool_view(pool, kv_heads, head_dim, page_tokens)
    t = np.arange(n)
    pages = np.asarray(bt_row)[t // page_tokens]
    slots = t % page_tokens
    K = bf16_bits_to_f64(kv[pages, slots // 16, :, :, slots % 16, :]).reshape(n, kv_heads, head_dim)
    V = bf16_bits_to_f64(vv[pages, slots // 16, :, :, slots % 16])
    return K, V


def layer(shape, lw, x, K, V, pos):
    """One layer, one sequence; K, V [pos, hkv, D] float64 cached rows.
    Returns (x_out, k_row, v_row) with k_row/v_row BF16-rounded float64."""
    H, hq, hkv, D, I = shape.hidden, shape.heads, shape.kv_heads, shape.head_dim, shape.inter
    W = {k: bf16_bits_to_f64(v) for k, v in lw.items()}
    xn = rmsnorm(x, W["attn_norm"], shape.eps)
    qkv = W["w_qkv"] @ xn
    q = qkv[:hq * D].reshape(hq, D)
    k = qkv[hq * D:(hq + hkv) * D].reshape(hkv, D)
    v = qkv[(hq + hkv) * D:].reshape(hkv, D)
    q = rope(q, pos, shape.theta)
    k = bf16_round_f64(rope(k, pos, shape.theta))
    v = bf16_round_f64(v)
    Kall = np.concatenate([K, k[None]], axis=0)
    Vall = np.concatenate([V, v[None]], axis=0)
    o = softmax_attention(q, Kall, Vall, 1.0 / np.sqrt(D)).reshape(-1)
    h1 = x + W["w_o"] @ o
    hn = rmsnorm(h1, W["mlp_norm"], shape.eps)
    gu = W["w_gate_up"] @ hn
    g, u = gu[:I], gu[I:]
    a = g / (1.0 + np.exp(-g)) * u
    return h1 + W["w_down"] @ a, k, v


def decode_step(shape, weights, pool, bts, positions, tokens):
    """Full step for every sequence; returns (logits [B, V], argmax [B])."""
    E = bf16_bits_to_f64(weights["embed"])
    fn = bf16_bits_to_f64(weights["final_norm"])
    out_logits, out_tok = [], []
    for b, (p, tok) in enumerate(zip(positions, tokens)):
        x = E[int(tok)].copy()
        for l in range(shape.layers):
            K, V = gather(pool, shape.kv_heads, shape.head_dim, bts[l, b], int(p))
            x, _, _ = layer(shape, weights["layers"][l], x, K, V, int(p))
        logits = E @ rmsnorm(x, fn, shape.eps)
        out_logits.append(logits)
        out_tok.append(int(np.argmax(logits)))
    return np.array(out_logits), np.array(out_tok)


def online_softmax_attention(q, K, V, scale, block):
    """Float64 online softmax over blocks of `block` tokens (running max,
    rescaled sum and accumulator), for one head: q [D], K, V [n, D]."""
    m, l, acc = -np.inf, 0.0, np.zeros(q.shape[0])
    for t0 in range(0, K.shape[0], block):
        s = K[t0:t0 + block] @ q * scale
        m_new = max(m, s.max())
        alpha = np.exp(m - m_new) if np.isfinite(m) else 0.0
        p = np.exp(s - m_new)
        l = l * alpha + p.sum()
        acc = acc * alpha + p @ V[t0:t0 + block]
        m = m_new
    return acc / l


def prefill(shape, weights, pool, bts, start, tokens):
    """Float64 prefill of one sequence's whole prompt at once: tokens[t] at
    position start + t over a cache of `start` tokens (bts [L, max_pages]).
    Every layer projects all prompt tokens together and applies causal
    attention through a materialised mask over [start + T] keys.  Returns
    (logits of the last token, [(K, V) BF16-rounded [T, hkv, D] per layer])."""
    H, hq, hkv, D, I = shape.hidden, shape.heads, shape.kv_heads, shape.head_dim, shape.inter
    tokens = np.asarray(tokens)
    T = len(tokens)
    E = bf16_bits_to_f64(weights["embed"])
    X = E[tokens].copy()                                    # [T, H]
    pos = start + np.arange(T)
    written = []
    for l in range(shape.layers):
        W = {k: bf16_bits_to_f64(v) for k, v in weights["layers"][l].items()}
        K0, V0 = gather(pool, hkv, D, bts[l], start)         # [start, hkv, D]
        QKV = rmsnorm(X, W["attn_norm"], shape.eps) @ W["w_qkv"].T
        Q = QKV[:, :hq * D].reshape(T, hq, D)
        K = QKV[:, hq * D:(hq + hkv) * D].reshape(T, hkv, D)
        V = QKV[:, (hq + hkv) * D:].reshape(T, hkv, D)
        Q = np.stack([rope(Q[t], pos[t], shape.theta) for t in range(T)])
        K = bf16_round_f64(np.stack([rope(K[t], pos[t], shape.theta) for t in range(T)]))
        V = bf16_round_f64(V)
        written.append((K, V))
        Kall = np.repeat(np.concatenate([K0, K]), hq // hkv, axis=1)   # [start+T, hq, D]
        Vall = np.repeat(np.concatenate([V0, V]), hq // hkv, axis=1)
        S = np.einsum("thd,nhd->thn", Q, Kall) / np.sqrt(D)
        causal = np.arange(start + T)[None, :] > pos[:, None]        # key after the query
        S = np.where(causal[:, None, :], -np.inf, S)
        P = np.exp(S - S.max(axis=2, keepdims=True))
        P = P / P.sum(axis=2, keepdims=True)
        O = np.einsum("thn,nhd->thd", P, Vall).reshape(T, hq * D)
        H1 = X + O @ W["w_o"].T
        GU = rmsnorm(H1, W["mlp_norm"], shape.eps) @ W["w_gate_up"].T
        G, U = GU[:, :I], GU[:, I:]
        X = H1 + (G / (1.0 + np.exp(-G)) * U) @ W["w_down"].T
    logits = E @ rmsnorm(X[-1], bf16_bits_to_f64(weights["final_norm"]), shape.eps)
    return logits, written
