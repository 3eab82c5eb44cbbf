"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws numbers and lays out tables: weights, hidden states,
token ids, context lengths, the random contents of the BF16 page pool and the
block tables that map each (layer, sequence, logical page) to a physical
page.  It holds none of the decode step's arithmetic; both the oracle and the
HIP path receive exactly the bytes produced here.

Every tensor is keyed by (seed, tensor id, *index).  Normal values come from
torch's CPU generator, one generator per chunk of 2^24 elements seeded from
``numpy.random.SeedSequence([seed, tensor id, *index, chunk])``, so any
tensor or chunk regenerates on its own and the result does not depend on how
many threads draw the chunks.  FP32 normals are turned into BF16 with
torch's round-to-nearest-even conversion.  Small integer draws (lengths,
token ids, page permutations) use ``numpy.random.default_rng`` with the same
key.

Model shapes follow the public configurations of the two model families the
source pages run (Llama 3.2 1B in the "Inference from Scratch" engine,
Qwen2.5-0.5B-Instruct in llmc), with random weights: no checkpoint is used.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE_TOKENS = 16

# tensor ids for the seed sequence
_ID = {"embed": 1, "final_norm": 2, "attn_norm": 10, "w_qkv": 11, "w_o": 12,
       "mlp_norm": 13, "w_gate_up": 14, "w_down": 15, "hidden": 20, "tokens": 21,
       "lens": 22, "pool": 23, "perm": 24, "q": 25, "k_new": 26, "v_new": 27,
       "prompt": 28, "logits": 29, "sample": 30, "pool_k": 31, "pool_v": 32}

LAYER_KEYS = ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate_up", "w_down")


@dataclass(frozen=True)
class ModelShape:
    name: str
    hidden: int
    layers: int
    heads: int
    kv_heads: int
    head_dim: int
    inter: int
    vocab: int
    eps: float
    theta: float
    max_pos: int

    @property
    def qkv_rows(self):
        return (self.heads + 2 * self.kv_heads) * self.head_dim

    def layer_param_count(self):
        H, D = self.hidden, self.head_dim
        return (self.qkv_rows * H + H * self.heads * D + 2 * self.inter * H
                + H * self.inter + 2 * H)


QWEN05 = ModelShape("qwen2.5-0.5b-shape", hidden=896, layers=24, heads=14, kv_heads=2,
                    head_dim=64, inter=4864, vocab=151936, eps=1e-6, theta=1e6,
                    max_pos=32768)
LLAMA1B = ModelShape("llama-3.2-1b-shape", hidden=2048, layers=16, heads=32, kv_heads=8,
                     head_dim=64, inter=8192, vocab=128256, eps=1e-5, theta=5e5,
                     max_pos=131072)
# The same GQA family with 128-wide heads (the head-width variant of the
# page geometry): Llama-3-8B's layer shape.
LLAMA8B = ModelShape("llama-3-8b-shape", hidden=4096, layers=32, heads=32, kv_heads=8,
                     head_dim=128, inter=14336, vocab=128256, eps=1e-5, theta=5e5,
                     max_pos=8192)


def tiny_shape(hidden=128, layers=2, heads=4, kv_heads=2, inter=256, vocab=1000,
               head_dim=64, eps=1e-5, theta=1e4, max_pos=4096, name="tiny"):
    return ModelShape(name, hidden, layers, heads, kv_heads, head_dim, inter, vocab,
                      eps, theta, max_pos)


# ----------------------------------------------------------- primitives ---

def rng(seed, name, *index):
    return np.random.default_rng([int(seed), _ID[name], *[int(i) for i in index]])


def to_bf16_bits(x):
    """float32 numpy -> uint16 BF16 bit patterns (torch's RNE conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


_CHUNK = 1 << 24


def torch_generator(seed, name, *index):
    """A torch CPU generator seeded from (seed, tensor id, *index)."""
    ss = np.random.SeedSequence([int(seed), _ID[name], *[int(i) for i in index]])
    return torch.Generator().manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] >> 1))


def _normal_bf16_into(out, seed, name, index, sigma, mean):
    n = out.size

    def chunk(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = torch_generator(seed, name, *index, c)
        x = torch.randn(hi - lo, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            x.mul_(sigma)
        if mean != 0.0:
            x.add_(mean)
        out[lo:hi] = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            chunk(c)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=min(16, nchunks)) as ex:
            list(ex.map(chunk, range(nchunks)))
    return out


def bf16_normal(seed, name, shape, sigma=1.0, mean=0.0, index=()):
    """N(mean, sigma^2) values rounded to BF16, as uint16 bit patterns."""
    out = np.empty(int(np.prod(shape)), dtype=np.uint16)
    return _normal_bf16_into(out, seed, name, tuple(index), float(sigma), float(mean)).reshape(shape)


# --------------------------------------------------------------- weights ---

def layer_weights(shape, seed, layer, sigma=0.02, norm_sigma=0.02):
    H, D, I = shape.hidden, shape.head_dim, shape.inter
    return {
        "attn_norm": bf16_normal(seed, "attn_norm", (H,), norm_sigma, 1.0, (layer,)),
        "w_qkv": bf16_normal(seed, "w_qkv", (shape.qkv_rows, H), sigma, 0.0, (layer,)),
        "w_o": bf16_normal(seed, "w_o", (H, shape.heads * D), sigma, 0.0, (layer,)),
        "mlp_norm": bf16_normal(seed, "mlp_norm", (H,), norm_sigma, 1.0, (layer,)),
        "w_gate_up": bf16_normal(seed, "w_gate_up", (2 * I, H), sigma, 0.0, (layer,)),
        "w_down": bf16_normal(seed, "w_down", (H, I), sigma, 0.0, (layer,)),
    }


def model_weights(shape, seed, sigma=0.02, norm_sigma=0.02, layers=None):
    L = shape.layers if layers is None else layers
    return {
        "embed": bf16_normal(seed, "embed", (shape.vocab, shape.hidden), sigma),
        "final_norm": bf16_normal(seed, "final_norm", (shape.hidden,), norm_sigma, 1.0),
        "layers": [layer_weights(shape, seed, l, sigma, norm_sigma) for l in range(L)],
    }


# ------------------------------------------------------- pool and tables ---

def page_elems(shape_or_kv_heads, head_dim=64, page_tokens=PAGE_TOKENS):
    """BF16 elements of one page; a model shape brings its own head width."""
    if hasattr(shape_or_kv_heads, "kv_heads"):
        kv, head_dim = shape_or_kv_heads.kv_heads, shape_or_kv_heads.head_dim
    else:
        kv = shape_or_kv_heads
    return 2 * kv * page_tokens * head_dim


def random_pool(seed, num_pages, elems_per_page):
    """The whole pool as N(0,1) BF16 values."""
    return bf16_normal(seed, "pool", (num_pages * elems_per_page,))


def random_split_pools(seed, num_pages, elems_per_page):
    """Separate K and V pools (half a page each per page) as N(0,1) BF16."""
    half = num_pages * elems_per_page // 2
    return bf16_normal(seed, "pool_k", (half,)), bf16_normal(seed, "pool_v", (half,))


def pages_for(n_tokens, page_tokens=PAGE_TOKENS):
    return (np.asarray(n_tokens, dtype=np.int64) + page_tokens - 1) // page_tokens


def block_tables(seed, layers, n_tokens, num_pages, max_pages=None, fill=-1, page_tokens=PAGE_TOKENS):
    """int32 [layers, B, max_pages]: the (layer, seq, logical page) entries
    that hold tokens 0..n_b-1 take physical pages from one random
    permutation of the pool, in that order; the other entries are `fill`."""
    n_tokens = np.asarray(n_tokens, dtype=np.int64)
    need = pages_for(n_tokens, page_tokens)
    if max_pages is None:
        max_pages = int(max(1, need.max()))
    total = int(need.sum()) * layers
    if total > num_pages:
        raise ValueError("pool of %d pages cannot hold %d pages" % (num_pages, total))
    perm = rng(seed, "perm").permutation(num_pages).astype(np.int32)
    bt = np.full((layers, len(n_tokens), max_pages), fill, dtype=np.int32)
    i = 0
    for l in range(layers):
        for b, k in enumerate(need):
            bt[l, b, :k] = perm[i:i + k]
            i += k
    return bt


# ----------------------------------------------------------- workloads ---

@dataclass
class Workload:
    name: str
    shape: ModelShape
    batch: int
    positions: np.ndarray          # int32 [B]: absolute position of the new token
    num_pages: int
    block_tables: np.ndarray       # int32 [L, B, max_pages]
    pool: np.ndarray = None        # uint16 [num_pages * page_elems]
    extra: dict = field(default_factory=dict)
    page_tokens: int = PAGE_TOKENS

    @property
    def max_pages(self):
        return self.block_tables.shape[2]

    @property
    def lens(self):
        return self.positions.astype(np.int32) + 1


def decode_workload(name, shape, seed, positions, layers=None, num_pages=None,
                    max_pages=None, with_pool=True, page_tokens=PAGE_TOKENS):
    """Inputs for a decode step: token p_b is new, 0..p_b-1 are cached in the
    pool.  The pool is sized to fit unless num_pages is given."""
    positions = np.asarray(positions, dtype=np.int32)
    L = shape.layers if layers is None else layers
    need = int(pages_for(positions + 1, page_tokens).sum()) * L
    npages = need if num_pages is None else num_pages
    bt = block_tables(seed, L, positions + 1, npages, max_pages, page_tokens=page_tokens)
    pool = random_pool(seed, npages, page_elems(shape, page_tokens=page_tokens)) if with_pool else None
    return Workload(name, shape, len(positions), positions, npages, bt, pool, page_tokens=page_tokens)


def qwen05_layer_b1(seed=1001):
    """One Qwen2.5-0.5B-shaped layer, batch 1, 127 cached + 1 new, 64-page pool."""
    shape = QWEN05
    wl = decode_workload("qwen2.5-0.5b-shape layer, batch 1, 127 cached + 1 new",
                         shape, seed, [127], layers=1, num_pages=64)
    wl.extra["weights"] = layer_weights(shape, seed, 0)
    wl.extra["hidden"] = rng(seed, "hidden").standard_normal((1, shape.hidden), dtype=np.float32)
    return wl


def attention_lens(seed=1002, batch=16, max_len=2048):
    return rng(seed, "lens").integers(1, max_len + 1, size=batch).astype(np.int32)


def attention_workload(seed=1002, batch=16, pool_bytes=128 << 20, shape=LLAMA1B, page_tokens=PAGE_TOKENS):
    """Paged GQA attention alone, Llama-3.2-1B heads (or another shape's),
    lengths U[1,2048], pages of page_tokens tokens drawn from a 128 MiB pool
    with shuffled tables; Q N(0,1) BF16, scale 1/sqrt(head_dim)."""
    lens = attention_lens(seed, batch)
    pe = page_elems(shape, page_tokens=page_tokens)
    npages = pool_bytes // (pe * 2)
    bt = block_tables(seed, 1, lens, npages, max_pages=2048 // page_tokens, page_tokens=page_tokens)[0]
    pool = random_pool(seed, npages, pe)
    q = bf16_normal(seed, "q", (batch, shape.heads, shape.head_dim))
    name = "paged GQA attention, %d/%d heads, d%d, batch %d, lens U[1,2048], %d-token pages, %d MiB pool" % (
        shape.heads, shape.kv_heads, shape.head_dim, batch, page_tokens, pool_bytes >> 20)
    return {"name": name, "shape": shape, "lens": lens, "num_pages": int(npages), "block_table": bt,
            "pool": pool, "q": q, "scale": 1.0 / float(np.sqrt(shape.head_dim)),
            "page_tokens": page_tokens}


def llama1b_step_b1(seed=1003, with_pool=True, layers=None):
    shape = LLAMA1B
    L = shape.layers if layers is None else layers
    wl = decode_workload("llama-3.2-1b-shape 16-layer step, batch 1, context 1024",
                         shape, seed, [1023], layers=L, with_pool=with_pool)
    wl.extra["tokens"] = rng(seed, "tokens").integers(0, shape.vocab, size=1).astype(np.int32)
    return wl


def llama1b_b64_positions(seed=1004, batch=64):
    return (rng(seed, "lens").integers(64, 2049, size=batch) - 1).astype(np.int32)


def llama1b_step_b64(seed=1004, batch=64, with_pool=True, layers=None):
    shape = LLAMA1B
    L = shape.layers if layers is None else layers
    wl = decode_workload("llama-3.2-1b-shape 16-layer step, batch 64, context U[64,2048]",
                         shape, seed, llama1b_b64_positions(seed, batch), layers=L, with_pool=with_pool)
    wl.extra["tokens"] = rng(seed, "tokens").integers(0, shape.vocab, size=batch).astype(np.int32)
    return wl


def qwen05_step_b128(seed=1005, batch=128, with_pool=True, layers=None):
    shape = QWEN05
    L = shape.layers if layers is None else layers
    wl = decode_workload("qwen2.5-0.5b-shape 24-layer step, batch 128, 4096 cached + 1 new",
                         shape, seed, np.full(batch, 4096, dtype=np.int32), layers=L,
                         with_pool=with_pool)
    wl.extra["tokens"] = rng(seed, "tokens").integers(0, shape.vocab, size=batch).astype(np.int32)
    return wl


def bench_step(seed=1002, batch=16, with_pool=True, layers=None):
    """Llama-3.2-1B-shaped 16-layer decode step at batch 16 whose attention
    lengths are the paged-attention workload's draw (U[1,2048])."""
    shape = LLAMA1B
    L = shape.layers if layers is None else layers
    positions = attention_lens(seed, batch) - 1
    wl = decode_workload("llama-3.2-1b-shape 16-layer decode step, batch 16, "
                         "attention lengths U[1,2048] (the paged-attention draw)",
                         shape, seed, positions, layers=L, with_pool=with_pool)
    wl.extra["tokens"] = rng(seed, "tokens").integers(0, shape.vocab, size=batch).astype(np.int32)
    return wl
