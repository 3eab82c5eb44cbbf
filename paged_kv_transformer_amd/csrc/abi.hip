// Host side of the C ABI declared in include/pkv.h: argument validation
// (pure host code, run before any HIP call), workspace carving and the
// launch sequence of each entry point.  Every step of the computation runs
// in the kernels of attention.hip, gemm.hip, fused_layer.hip, prefill.hip, sample.hip and misc.hip.
#include <errno.h>
#include <math.h>
#include <stdint.h>

#include <atomic>

#include "pkv.h"
#include "pkv_dev.h"

using namespace pkv;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Supported head widths and page sizes.
bool head_dim_ok(int D) { return D == 64 || D == 128; }
bool page_tokens_ok(int pt) { return pt == 16 || pt == 256; }
int pt_shift(int pt) { return pt == 256 ? 4 : 0; }

// A block table of max_pages pages as 16-token attention tiles.
int64_t table_tiles(int32_t max_pages, int32_t page_tokens) {
  return (int64_t)max_pages << pt_shift(page_tokens);
}

int check_pool(const pkv_pool* p) {
  if (!p || !p->base) return -EINVAL;
  if (!head_dim_ok(p->head_dim) || !page_tokens_ok(p->page_tokens)) return -ENOTSUP;
  if (p->num_kv_heads < 1 || p->num_pages < 1 || p->bytes < 0) return -EINVAL;
  const int64_t block = 2LL * p->num_kv_heads * p->page_tokens * p->head_dim;  // bytes of K (or V)
  if (p->page_bytes != (p->v_base ? block : 2 * block)) return -EINVAL;
  if ((int64_t)p->num_pages * p->page_bytes > p->bytes) return -EINVAL;
  if (!aligned(p->base, 256) || !aligned(p->v_base, 256)) return -EINVAL;
  return 0;
}

// The kernels' view of a pool: whole pages in one buffer, or K and V pools.
PoolView pool_view(const pkv_pool* p) {
  PoolView v{};
  const int64_t block = (int64_t)p->num_kv_heads * p->page_tokens * p->head_dim;  // elements
  v.k = (uint16_t*)p->base;
  v.v = p->v_base ? (uint16_t*)p->v_base : v.k + block;
  v.stride = p->v_base ? block : 2 * block;
  v.num_pages = p->num_pages;
  v.pt_shift = pt_shift(p->page_tokens);
  v.hkv = p->num_kv_heads;
  return v;
}

int check_heads(int32_t Hq, int32_t Hkv) {
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return -EINVAL;
  if (Hq / Hkv > kMaxGroup) return -ENOTSUP;
  return 0;
}

int check_cfg(const pkv_config* c) {
  if (!c) return -EINVAL;
  if (!head_dim_ok(c->head_dim)) return -ENOTSUP;
  int rc = check_heads(c->num_attention_heads, c->num_key_value_heads);
  if (rc) return rc;
  if (c->hidden_size < 1 || c->intermediate_size < 1 || c->max_position_embeddings < 1)
    return -EINVAL;
  if (c->hidden_size % 64 != 0 || c->intermediate_size % 64 != 0) return -ENOTSUP;
  // the kernels address every weight matrix and activation buffer through a
  // 32-bit byte range
  if (c->hidden_size > kMaxDim || c->intermediate_size > kMaxDim) return -ENOTSUP;
  const int64_t H = c->hidden_size, I = c->intermediate_size;
  const int64_t qkv_rows = (int64_t)(c->num_attention_heads + 2 * c->num_key_value_heads) * c->head_dim;
  if (c->vocab_size > 0 && (int64_t)c->vocab_size * H * 2 > kMaxMatrixBytes) return -ENOTSUP;
  if (qkv_rows * H * 2 > kMaxMatrixBytes || 2 * I * H * 2 > kMaxMatrixBytes) return -ENOTSUP;
  if (!(c->rms_norm_eps >= 0.f) || !isfinite(c->rms_norm_eps)) return -EINVAL;
  if (!(c->rope_theta > 0.f) || !isfinite(c->rope_theta)) return -EINVAL;
  return 0;
}

int check_layer_weights(const pkv_layer_weights* w) {
  if (!w || !w->attn_norm || !w->w_qkv || !w->w_o || !w->mlp_norm || !w->w_gate_up || !w->w_down)
    return -EINVAL;
  return 0;
}

int io(hipError_t e) {
  if (e == hipSuccess) return 0;
  (void)hipGetLastError();
  return -EIO;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

size_t layer_ws_bytes(const pkv_config* c, int batch, int64_t max_tiles);

// Common checks of decoder_layer_decode / decode_step.
int check_layer_call(const pkv_config* cfg, const pkv_pool* pool, const float* rope_cos,
                     const float* rope_sin, const int32_t* bt, int32_t max_pages,
                     const int32_t* positions, int32_t batch, void* ws, size_t ws_bytes) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  rc = check_pool(pool);
  if (rc) return rc;
  if (pool->num_kv_heads != cfg->num_key_value_heads || pool->head_dim != cfg->head_dim)
    return -EINVAL;
  if (batch < 0 || max_pages < 1) return -EINVAL;
  const int64_t tiles = table_tiles(max_pages, pool->page_tokens);
  if (batch > 65535 || attn_max_splits(tiles) > 65535) return -ENOTSUP;
  if (!rope_cos || !rope_sin || !bt || !positions || !ws) return -EINVAL;
  if (!aligned(ws, 256)) return -EINVAL;
  if (ws_bytes < layer_ws_bytes(cfg, batch, tiles)) return -ENOSPC;
  return 0;
}

// Launch one projection over the batch in chunks of kGemmMaxCols columns;
// `setup(a, b0)` points the per-chunk arguments at columns b0...
template <typename F>
int gemm_batched(int epi, int N, int batch, const GemmArgs& base, F setup, hipStream_t st) {
  for (int b0 = 0; b0 < batch; b0 += kGemmMaxCols) {
    const int bc = batch - b0 < kGemmMaxCols ? batch - b0 : kGemmMaxCols;
    GemmArgs a = base;
    a.B = bc;
    setup(a, b0);
    const GemmPlan p = plan_gemm(epi, N, bc, a.K);
    a.ksplit = p.ks;
    if (int rc = io(launch_gemm(epi, a, p, st))) return rc;
  }
  return 0;
}

float* packed_at(float* base, int b0, int K) { return base + packed_act_index(b0, 0, K); }

// One decoder layer over the whole batch.  hidden [batch][H] (plain) is
// updated in place and also left packed in the workspace (x_p) for the next
// projection; hidden_packed, if given, is hidden already packed.
int run_layer(const pkv_config* cfg, const pkv_layer_weights* w, const float* rope_cos,
              const float* rope_sin, const pkv_pool* pool, const int32_t* bt, int32_t max_pages,
              int32_t bt_row, const int32_t* pos, int32_t batch, float* hidden,
              const float* hidden_packed, void* ws, const WsLayout& L, hipStream_t st) {
  const int H = cfg->hidden_size, Hq = cfg->num_attention_heads;
  const int Hkv = cfg->num_key_value_heads, I = cfg->intermediate_size;
  const int D = cfg->head_dim, QD = Hq * D;
  uint16_t* q = at<uint16_t>(ws, L.q);  // [B][Hq][2][D] BF16 hi, lo
  float* o_p = at<float>(ws, L.o_p);
  float* h1 = at<float>(ws, L.h1);
  float* h1_p = at<float>(ws, L.h1_p);
  float* act_p = at<float>(ws, L.act_p);
  float* x_p = at<float>(ws, L.x_p);
  uint32_t* err = at<uint32_t>(ws, L.err);
  int rc;

  GemmArgs base{};
  base.eps = cfg->rms_norm_eps;
  base.err = err;

  // 1. RMSNorm + QKV + RoPE + KV append
  {
    GemmArgs a = base;
    a.W = w->w_qkv;
    a.w_groups = (Hq + 2 * Hkv) * (D / 16);
    a.xw = w->attn_norm;
    a.N = (Hq + 2 * Hkv) * D;
    a.D = D;
    a.K = H;
    a.x_plain = hidden_packed == nullptr;
    a.pv = pool_view(pool);
    a.bt_stride = max_pages;
    a.bt_row = bt_row;
    a.rcos = rope_cos;
    a.rsin = rope_sin;
    a.max_pos = cfg->max_position_embeddings;
    a.Hq = Hq;
    a.Hkv = Hkv;
    rc = gemm_batched(EPI_QKV, a.N, batch, a, [&](GemmArgs& c, int b0) {
      c.X = hidden_packed ? packed_at(const_cast<float*>(hidden_packed), b0, H) : hidden + (size_t)b0 * H;
      c.q_split = q + (size_t)b0 * 2 * QD;
      c.bt = bt + (size_t)b0 * bt_row;
      c.pos = pos + b0;
    }, st);
    if (rc) return rc;
  }

  // 2. paged attention over tokens 0..pos, output packed for the O projection
  {
    AttnArgs a{};
    a.q = q;
    a.pv = pool_view(pool);
    a.bt = bt;
    a.bt_stride = max_pages;
    a.bt_row = bt_row;
    a.lens = pos;
    a.len_add = 1;
    a.scale = 1.0f / sqrtf((float)D);
    a.out = o_p;
    a.out_packed = 1;
    a.D = D;
    a.part = at<float>(ws, L.attn_part);
    a.err = err;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.pw = attn_pw(batch, a.Hkv, table_tiles(max_pages, pool->page_tokens));
    a.max_splits = attn_max_splits(table_tiles(max_pages, pool->page_tokens), a.pw);
    if ((rc = io(launch_attention(a, batch, kQSplit, st)))) return rc;
  }

  // 3. output projection + residual: h1 = x + W_o o
  {
    GemmArgs a = base;
    a.W = w->w_o;
    a.w_groups = H / 16;
    a.N = H;
    a.K = QD;
    rc = gemm_batched(EPI_RESID, H, batch, a, [&](GemmArgs& c, int b0) {
      c.X = packed_at(o_p, b0, QD);
      c.out = h1 + (size_t)b0 * H;
      c.out_packed = packed_at(h1_p, b0, H);
      c.resid = hidden + (size_t)b0 * H;
      c.part = at<float>(ws, L.gemm_part);
    }, st);
    if (rc) return rc;
  }

  // 4. RMSNorm + gate/up + SwiGLU
  {
    GemmArgs a = base;
    a.W = w->w_gate_up;
    a.w_groups = I / 8;
    a.xw = w->mlp_norm;
    a.N = 2 * I;
    a.K = H;
    a.I = I;
    rc = gemm_batched(EPI_SWIGLU, 2 * I, batch, a, [&](GemmArgs& c, int b0) {
      c.X = packed_at(h1_p, b0, H);
      c.act = packed_at(act_p, b0, I);
    }, st);
    if (rc) return rc;
  }

  // 5. down projection + residual: x = h1 + W_down a
  {
    GemmArgs a = base;
    a.W = w->w_down;
    a.w_groups = H / 16;
    a.N = H;
    a.K = I;
    rc = gemm_batched(EPI_RESID, H, batch, a, [&](GemmArgs& c, int b0) {
      c.X = packed_at(act_p, b0, I);
      c.out = hidden + (size_t)b0 * H;
      c.out_packed = packed_at(x_p, b0, H);
      c.resid = h1 + (size_t)b0 * H;
      c.part = at<float>(ws, L.gemm_part);
    }, st);
    if (rc) return rc;
  }
  return 0;
}

// ---------------------------------------------------------------------------
// Batch 1: the whole layer as one launch (fused_layer.hip) when its weights
// fit the chip's LDS and its table the kernel's attention units.  Returns 1
// when the layer was launched, 0 when the multi-launch path must run, or a
// negative errno.
std::atomic<int> g_fused_layer{1};

bool fused_plan_for(const pkv_config* c, int64_t max_tiles, int nwg, FusedArgs* a) {
  // the plan depends only on the shapes: keep the last one
  struct Key {
    int H, Hq, Hkv, D, I, nwg;
    int64_t tiles;
    bool ok;
  };
  static thread_local Key key{-1, 0, 0, 0, 0, 0, 0, false};
  static thread_local FusedArgs plan{};
  const Key k{c->hidden_size, c->num_attention_heads, c->num_key_value_heads, c->head_dim,
              c->intermediate_size, nwg, max_tiles, false};
  if (!(key.H == k.H && key.Hq == k.Hq && key.Hkv == k.Hkv && key.D == k.D && key.I == k.I &&
        key.nwg == k.nwg && key.tiles == k.tiles)) {
    key = k;
    plan = FusedArgs{};
    key.ok = plan_fused_layer(k.H, k.Hq, k.Hkv, k.D, k.I, max_tiles, nwg, &plan);
  }
  if (key.ok) *a = plan;
  return key.ok;
}

int run_layer_fused(const pkv_config* cfg, const pkv_layer_weights* w, const float* rope_cos,
                    const float* rope_sin, const pkv_pool* pool, const int32_t* bt, int32_t max_pages,
                    const int32_t* pos, float* hidden, float* hidden_packed, void* ws, const WsLayout& L,
                    hipStream_t st) {
  if (!g_fused_layer.load(std::memory_order_relaxed)) return 0;
  const int nwg = fused_device_wgs();
  if (nwg < 1) return 0;
  const int64_t tiles = table_tiles(max_pages, pool->page_tokens);
  FusedArgs a{};
  if (!fused_plan_for(cfg, tiles, nwg, &a)) return 0;
  const int H = cfg->hidden_size, Hq = cfg->num_attention_heads, Hkv = cfg->num_key_value_heads;
  const int D = cfg->head_dim, I = cfg->intermediate_size;
  a.eps = cfg->rms_norm_eps;
  a.scale = 1.0f / sqrtf((float)D);
  a.attn_norm = w->attn_norm;
  a.w_qkv = w->w_qkv;
  a.w_o = w->w_o;
  a.mlp_norm = w->mlp_norm;
  a.w_gu = w->w_gate_up;
  a.w_down = w->w_down;
  a.rcos = rope_cos;
  a.rsin = rope_sin;
  a.max_pos = cfg->max_position_embeddings;
  a.pv = pool_view(pool);
  a.bt = bt;
  a.bt_stride = max_pages;
  a.pos = pos;
  a.hidden = hidden;
  a.hidden_packed = hidden_packed;
  a.err = at<uint32_t>(ws, L.err);
  a.epoch = at<uint32_t>(ws, L.fused_epoch);
  uint64_t* ll = at<uint64_t>(ws, L.fused_ll);
  a.q = ll;
  a.kn = a.q + (size_t)Hq * D;
  a.vn = a.kn + (size_t)Hkv * D;
  a.rec = a.vn + (size_t)Hkv * D;
  a.h1 = a.rec + (size_t)Hkv * a.ns * fused_rec_len(a.G, D);
  a.ypart = a.h1 + (size_t)kFusedCopies * H;
  (void)I;
  const int rc = io(launch_fused_layer(a, st));
  return rc ? rc : 1;
}

// ---------------------------------------------------------------------------
// Large batches (kTiledMinBatch sequences or more): the projections run as
// the tiled matrix-core GEMMs of the prefill path, which read every weight
// once per step and keep the activations in LDS, where the weight-streaming
// kernel would re-read 64 FP32 activation columns from L2 for every 16 weight
// rows.  Activations travel as packed BF16 hi/lo pairs; each residual
// projection splits K into FP32 partials and one per-token kernel adds the
// residual and the splits and applies the next RMSNorm.
constexpr int kTiledMinBatch = 64;

struct TiledLayout {
  size_t err, attn_part, q, x, xb, ob, act, part, amax, total;
};

// The tiled QKV projection of T tokens: one launch with the RoPE/append
// epilogue, or (too few tiles) K split into FP32 partials (`part`) + the
// finish kernel.  `a` holds every QKV argument; part must hold
// qkv_part_floats(...) floats.
PgemmPlan tiled_qkv_plan(const pkv_config* c, int T) {
  return plan_prefill_gemm((c->num_attention_heads + 2 * c->num_key_value_heads) * (c->head_dim / 16), T,
                           c->hidden_size, false);
}
size_t qkv_part_floats(const pkv_config* c, int T) {
  const int ks = qkv_splits(tiled_qkv_plan(c, T), c->hidden_size);
  return ks > 1 ? (size_t)ks * T * (c->num_attention_heads + 2 * c->num_key_value_heads) * c->head_dim : 0;
}
hipError_t launch_tiled_qkv(const pkv_config* c, PgemmArgs a, float* part, hipStream_t st) {
  PgemmPlan p = tiled_qkv_plan(c, a.T);
  const int ks = qkv_splits(p, a.K);
  if (ks == 1) return launch_prefill_gemm(EPI_QKV, a, p, st);
  p.ks = ks;
  a.part = part;
  a.ksplit = ks;
  const hipError_t e = launch_prefill_gemm(EPI_RESID, a, p, st);
  if (e != hipSuccess) return e;
  return launch_qkv_finish(part, ks, a, st);
}

PgemmPlan tiled_o_plan(const pkv_config* c, int B) {
  return plan_prefill_gemm(c->hidden_size / 16, B, c->num_attention_heads * c->head_dim, true);
}
PgemmPlan tiled_down_plan(const pkv_config* c, int B) {
  return plan_prefill_gemm(c->hidden_size / 16, B, c->intermediate_size, true);
}
PgemmPlan tiled_lm_plan(const pkv_config* c, int B) {
  return plan_prefill_gemm((c->vocab_size + 15) / 16, B, c->hidden_size, false);
}

// Row tiles of the tiled LM head (each leaves two argmax keys per token).
int lm_row_tiles(const pkv_config* c, int B) {
  const PgemmPlan p = tiled_lm_plan(c, B);
  const int groups = (c->vocab_size + 15) / 16;
  return (groups + 2 * p.rg - 1) / (2 * p.rg);
}

TiledLayout tiled_layout(const pkv_config* c, int B, int64_t max_tiles) {
  const size_t H = c->hidden_size, I = c->intermediate_size;
  const size_t QD = (size_t)c->num_attention_heads * c->head_dim;
  TiledLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
  L.err = take(kWsHeaderBytes);
  L.attn_part = take(sizeof(float) * (size_t)B * c->num_key_value_heads * attn_max_splits(max_tiles) *
                     attn_rec(c->head_dim));
  L.q = take(2 * (size_t)B * QD * 2);
  L.x = take(sizeof(float) * B * H);
  L.xb = take(2 * (size_t)packed_pair_elems(B, (int)H));
  L.ob = take(2 * (size_t)packed_pair_elems(B, (int)QD));
  L.act = take(2 * (size_t)packed_pair_elems(B, (int)I));
  const int ks = tiled_o_plan(c, B).ks > tiled_down_plan(c, B).ks ? tiled_o_plan(c, B).ks
                                                                    : tiled_down_plan(c, B).ks;
  const size_t pq = qkv_part_floats(c, B);
  L.part = take(sizeof(float) * ((size_t)ks * B * H > pq ? (size_t)ks * B * H : pq));
  if (c->vocab_size > 0) L.amax = take(sizeof(unsigned long long) * 2 * (size_t)lm_row_tiles(c, B) * B);
  L.total = off;
  return L;
}

// Workspace bytes of a layer call or step of `batch` sequences.
size_t layer_ws_bytes(const pkv_config* c, int batch, int64_t max_tiles) {
  if (batch >= kTiledMinBatch) return tiled_layout(c, batch, max_tiles).total;
  return ws_layout(batch, c->hidden_size, c->num_attention_heads, c->num_key_value_heads,
                   c->intermediate_size, c->vocab_size, max_tiles, true, c->head_dim)
      .total;
}

// One decoder layer over a large batch.  xb holds RMSNorm(x) (attention
// norm) as hi/lo pairs on entry; x [B][H] FP32 is updated in place, and xb
// holds RMSNorm(x, next_norm) on exit if next_norm is given.
int run_layer_tiled(const pkv_config* cfg, const pkv_layer_weights* w, const float* rope_cos,
                    const float* rope_sin, const pkv_pool* pool, const int32_t* bt, int32_t max_pages,
                    const int32_t* pos, int32_t B, float* x, const uint16_t* next_norm, void* ws,
                    const TiledLayout& L, hipStream_t st) {
  const int H = cfg->hidden_size, Hq = cfg->num_attention_heads;
  const int Hkv = cfg->num_key_value_heads, I = cfg->intermediate_size;
  const int D = cfg->head_dim, QD = Hq * D;
  const float eps = cfg->rms_norm_eps;
  uint16_t* q = at<uint16_t>(ws, L.q);
  uint16_t* xb = at<uint16_t>(ws, L.xb);
  uint16_t* ob = at<uint16_t>(ws, L.ob);
  uint16_t* act = at<uint16_t>(ws, L.act);
  float* part = at<float>(ws, L.part);
  uint32_t* err = at<uint32_t>(ws, L.err);
  int rc;
  PgemmArgs base{};
  base.T = B;
  base.err = err;
  {
    PgemmArgs a = base;
    a.W = w->w_qkv;
    a.w_groups = (Hq + 2 * Hkv) * (D / 16);
    a.X = xb;
    a.N = (Hq + 2 * Hkv) * D;
    a.K = H;
    a.D = D;
    a.q_split = q;
    a.pv = pool_view(pool);
    a.bt = bt;
    a.bt_row = max_pages;
    a.bt_stride = max_pages;
    a.pos = pos;
    a.max_pos = cfg->max_position_embeddings;
    a.rcos = rope_cos;
    a.rsin = rope_sin;
    a.Hq = Hq;
    a.Hkv = Hkv;
    if ((rc = io(launch_tiled_qkv(cfg, a, part, st)))) return rc;
  }
  {
    AttnArgs a{};
    a.q = q;
    a.pv = pool_view(pool);
    a.bt = bt;
    a.bt_stride = max_pages;
    a.bt_row = max_pages;
    a.lens = pos;
    a.len_add = 1;
    a.scale = 1.0f / sqrtf((float)D);
    a.out = (float*)ob;
    a.out_packed = 2;
    a.D = D;
    a.part = at<float>(ws, L.attn_part);
    a.err = err;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.pw = attn_pw(B, a.Hkv, table_tiles(max_pages, pool->page_tokens));
    a.max_splits = attn_max_splits(table_tiles(max_pages, pool->page_tokens), a.pw);
    if ((rc = io(launch_attention(a, B, kQSplit, st)))) return rc;
  }
  {
    const PgemmPlan p = tiled_o_plan(cfg, B);
    PgemmArgs a = base;
    a.W = w->w_o;
    a.w_groups = H / 16;
    a.X = ob;
    a.N = H;
    a.K = QD;
    a.part = part;
    a.ksplit = p.ks;
    if ((rc = io(launch_prefill_gemm(EPI_RESID, a, p, st)))) return rc;
    if ((rc = io(launch_prefill_resid(x, part, p.ks, B, H, w->mlp_norm, eps, xb, st)))) return rc;
  }
  {
    PgemmArgs a = base;
    a.W = w->w_gate_up;
    a.w_groups = I / 8;
    a.X = xb;
    a.N = 2 * I;
    a.K = H;
    a.act = act;
    a.I = I;
    if ((rc = io(launch_prefill_gemm(EPI_SWIGLU, a, plan_prefill_gemm(a.w_groups, B, H, false), st))))
      return rc;
  }
  {
    const PgemmPlan p = tiled_down_plan(cfg, B);
    PgemmArgs a = base;
    a.W = w->w_down;
    a.w_groups = H / 16;
    a.X = act;
    a.N = H;
    a.K = I;
    a.part = part;
    a.ksplit = p.ks;
    if ((rc = io(launch_prefill_gemm(EPI_RESID, a, p, st)))) return rc;
    if ((rc = io(launch_prefill_resid(x, part, p.ks, B, H, next_norm, eps, xb, st)))) return rc;
  }
  return 0;
}

}  // namespace

namespace pkv {

int prepare_attention_call(const pkv_pool* pool, const uint16_t* q, int32_t num_q_heads,
                           const int32_t* block_table, int32_t max_pages, const int32_t* context_lens,
                           int32_t batch, float scale, float* out, AttnArgs* args) {
  int rc = check_pool(pool);
  if (rc) return rc;
  rc = check_heads(num_q_heads, pool->num_kv_heads);
  if (rc) return rc;
  if (batch < 0 || max_pages < 1) return -EINVAL;
  const int64_t tiles = table_tiles(max_pages, pool->page_tokens);
  if (batch > 65535 || attn_max_splits(tiles) > 65535) return -ENOTSUP;
  if (batch == 0) return 0;
  if (!q || !block_table || !context_lens || !out || !isfinite(scale)) return -EINVAL;
  AttnArgs a{};
  a.q = q;
  a.pv = pool_view(pool);
  a.bt = block_table;
  a.bt_stride = max_pages;
  a.bt_row = max_pages;
  a.lens = context_lens;
  a.len_add = 0;
  a.scale = scale;
  a.out = out;
  a.Hq = num_q_heads;
  a.Hkv = pool->num_kv_heads;
  a.G = num_q_heads / pool->num_kv_heads;
  a.pw = attn_pw(batch, a.Hkv, tiles);
  a.max_splits = attn_max_splits(tiles, a.pw);
  a.D = pool->head_dim;
  *args = a;
  return 0;
}

}  // namespace pkv

extern "C" {

const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }

}  // extern "C"

namespace {

// Both pool constructors: v_base null for whole pages in one buffer.
int make_pool(void* k_base, void* v_base, int64_t bytes, int32_t num_kv_heads, int32_t head_dim,
              int32_t page_tokens, pkv_pool* out) {
  if (!out || !k_base || bytes < 0 || num_kv_heads < 1) return -EINVAL;
  if (!aligned(k_base, 256) || !aligned(v_base, 256)) return -EINVAL;
  if (!head_dim_ok(head_dim) || !page_tokens_ok(page_tokens)) return -ENOTSUP;
  const int64_t block = 2LL * num_kv_heads * page_tokens * head_dim;  // bytes of K (or V)
  const int64_t page_bytes = v_base ? block : 2 * block;
  const int64_t pages = bytes / page_bytes;
  if (pages < 1 || pages > INT32_MAX) return -ENOSPC;
  out->base = k_base;
  out->bytes = bytes;
  out->page_bytes = page_bytes;
  out->num_pages = (int32_t)pages;
  out->page_tokens = page_tokens;
  out->num_kv_heads = num_kv_heads;
  out->head_dim = head_dim;
  out->v_base = v_base;
  return 0;
}

}  // namespace

extern "C" {

int kv_pool_create(void* dev_base, int64_t bytes, int32_t num_kv_heads, int32_t head_dim,
                   int32_t page_tokens, pkv_pool* out) {
  return make_pool(dev_base, nullptr, bytes, num_kv_heads, head_dim, page_tokens, out);
}

int kv_pool_create_split(void* k_base, void* v_base, int64_t bytes, int32_t num_kv_heads,
                         int32_t head_dim, int32_t page_tokens, pkv_pool* out) {
  if (!v_base || k_base == v_base) return -EINVAL;
  const uintptr_t k0 = (uintptr_t)k_base, v0 = (uintptr_t)v_base;
  if (bytes > 0 && k0 < v0 + (uint64_t)bytes && v0 < k0 + (uint64_t)bytes) return -EINVAL;
  return make_pool(k_base, v_base, bytes, num_kv_heads, head_dim, page_tokens, out);
}

int kv_append(const pkv_pool* pool, const int32_t* block_table, int32_t max_pages,
              const int32_t* positions, const uint16_t* k_new, const uint16_t* v_new,
              int32_t batch, uint32_t* dev_error, void* stream) {
  int rc = check_pool(pool);
  if (rc) return rc;
  if (batch < 0 || max_pages < 1) return -EINVAL;
  if (batch == 0) return 0;
  if (!block_table || !positions || !k_new || !v_new) return -EINVAL;
  if (!aligned(dev_error, 4)) return -EINVAL;
  return io(launch_kv_append(pool_view(pool), block_table, max_pages, positions, k_new, v_new,
                             batch, pool->num_kv_heads, pool->head_dim, dev_error,
                             (hipStream_t)stream));
}

size_t pkv_attention_workspace_bytes(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     int32_t batch, int32_t max_pages, int32_t page_tokens) {
  if (check_heads(num_q_heads, num_kv_heads) || !head_dim_ok(head_dim) ||
      !page_tokens_ok(page_tokens) || batch < 0 || max_pages < 1)
    return 0;
  return ws_layout(batch, 0, num_q_heads, num_kv_heads, 0, 0, table_tiles(max_pages, page_tokens),
                   false, head_dim)
      .total;
}

size_t pkv_workspace_bytes(const pkv_config* cfg, int32_t batch, int32_t max_pages,
                           int32_t page_tokens) {
  if (check_cfg(cfg) || batch < 0 || max_pages < 1 || !page_tokens_ok(page_tokens)) return 0;
  return layer_ws_bytes(cfg, batch, table_tiles(max_pages, page_tokens));
}

int paged_gqa_decode(const pkv_pool* pool, const uint16_t* q, int32_t num_q_heads,
                     const int32_t* block_table, int32_t max_pages, const int32_t* context_lens,
                     int32_t batch, float scale, float* out, void* workspace, size_t ws_bytes,
                     void* stream) {
  AttnArgs a{};
  int rc = prepare_attention_call(pool, q, num_q_heads, block_table, max_pages, context_lens, batch,
                                  scale, out, &a);
  if (rc || batch == 0) return rc;
  if (!workspace) return -EINVAL;
  if (!aligned(workspace, 256)) return -EINVAL;
  const WsLayout L = ws_layout(batch, 0, num_q_heads, pool->num_kv_heads, 0, 0,
                               table_tiles(max_pages, pool->page_tokens), false, pool->head_dim);
  if (ws_bytes < L.total) return -ENOSPC;
  a.part = at<float>(workspace, L.attn_part);
  a.err = at<uint32_t>(workspace, L.err);
  return io(launch_attention(a, batch, kQBf16, (hipStream_t)stream));
}

int decoder_layer_decode(const pkv_config* cfg, const pkv_layer_weights* w,
                         const float* rope_cos, const float* rope_sin, const pkv_pool* pool,
                         const int32_t* block_table, int32_t max_pages, const int32_t* positions,
                         int32_t batch, float* hidden, void* workspace, size_t ws_bytes,
                         void* stream) {
  int rc = check_layer_call(cfg, pool, rope_cos, rope_sin, block_table, max_pages, positions,
                            batch, workspace, ws_bytes);
  if (rc) return rc;
  rc = check_layer_weights(w);
  if (rc) return rc;
  if (!hidden) return -EINVAL;
  if (batch == 0) return 0;
  const hipStream_t st = (hipStream_t)stream;
  if (batch >= kTiledMinBatch) {
    const TiledLayout T = tiled_layout(cfg, batch, table_tiles(max_pages, pool->page_tokens));
    if ((rc = io(launch_prefill_norm(hidden, w->attn_norm, cfg->hidden_size, batch, cfg->rms_norm_eps,
                                     at<uint16_t>(workspace, T.xb), st))))
      return rc;
    return run_layer_tiled(cfg, w, rope_cos, rope_sin, pool, block_table, max_pages, positions, batch,
                           hidden, nullptr, workspace, T, st);
  }
  const WsLayout L = ws_layout(batch, cfg->hidden_size, cfg->num_attention_heads,
                               cfg->num_key_value_heads, cfg->intermediate_size, cfg->vocab_size,
                               table_tiles(max_pages, pool->page_tokens), true, cfg->head_dim);
  if (batch == 1) {
    rc = run_layer_fused(cfg, w, rope_cos, rope_sin, pool, block_table, max_pages, positions, hidden,
                         nullptr, workspace, L, st);
    if (rc) return rc < 0 ? rc : 0;
  }
  return run_layer(cfg, w, rope_cos, rope_sin, pool, block_table, max_pages, max_pages, positions,
                   batch, hidden, nullptr, workspace, L, st);
}

int decode_step(const pkv_config* cfg, const pkv_model_weights* w, const pkv_pool* pool,
                const int32_t* block_tables, int32_t max_pages, const int32_t* positions,
                const int32_t* token_ids, int32_t batch, float* logits, int32_t* next_tokens,
                void* workspace, size_t ws_bytes, void* stream) {
  if (!w) return -EINVAL;
  int rc = check_layer_call(cfg, pool, w->rope_cos, w->rope_sin, block_tables, max_pages,
                            positions, batch, workspace, ws_bytes);
  if (rc) return rc;
  if (cfg->num_hidden_layers < 1 || cfg->vocab_size < 1) return -EINVAL;
  if (!w->embed || !w->final_norm || !w->layers || !token_ids || !next_tokens) return -EINVAL;
  for (int l = 0; l < cfg->num_hidden_layers; ++l) {
    rc = check_layer_weights(&w->layers[l]);
    if (rc) return rc;
  }
  if (batch == 0) return 0;
  const hipStream_t st = (hipStream_t)stream;
  const int H = cfg->hidden_size, V = cfg->vocab_size;
  if (batch >= kTiledMinBatch) {
    const TiledLayout T = tiled_layout(cfg, batch, table_tiles(max_pages, pool->page_tokens));
    float* x = at<float>(workspace, T.x);
    uint16_t* xb = at<uint16_t>(workspace, T.xb);
    uint32_t* err = at<uint32_t>(workspace, T.err);
    const int nl = cfg->num_hidden_layers;
    if ((rc = io(launch_embed(w->embed, V, H, token_ids, x, nullptr, batch, err, st)))) return rc;
    if ((rc = io(launch_prefill_norm(x, w->layers[0].attn_norm, H, batch, cfg->rms_norm_eps, xb, st))))
      return rc;
    for (int l = 0; l < nl; ++l) {
      const uint16_t* nn = l + 1 < nl ? w->layers[l + 1].attn_norm : w->final_norm;
      rc = run_layer_tiled(cfg, &w->layers[l], w->rope_cos, w->rope_sin, pool,
                           block_tables + (size_t)l * batch * max_pages, max_pages, positions, batch, x,
                           nn, workspace, T, st);
      if (rc) return rc;
    }
    // LM head on the final-normed rows, FP32 logits, argmax
    PgemmArgs a{};
    a.W = w->embed;
    a.w_groups = (V + 15) / 16;
    a.X = xb;
    a.N = V;
    a.K = H;
    a.T = batch;
    a.err = err;
    a.logits = logits;
    a.amax_part = at<unsigned long long>(workspace, T.amax);
    if ((rc = io(launch_prefill_gemm(EPI_LOGITS, a, tiled_lm_plan(cfg, batch), st)))) return rc;
    return io(launch_argmax_finalize(a.amax_part, 2 * lm_row_tiles(cfg, batch), batch, next_tokens, st));
  }
  const WsLayout L = ws_layout(batch, H, cfg->num_attention_heads, cfg->num_key_value_heads,
                               cfg->intermediate_size, V, table_tiles(max_pages, pool->page_tokens),
                               true, cfg->head_dim);
  float* x = at<float>(workspace, L.x);
  float* x_p = at<float>(workspace, L.x_p);
  uint32_t* err = at<uint32_t>(workspace, L.err);

  if ((rc = io(launch_embed(w->embed, V, H, token_ids, x, x_p, batch, err, st)))) return rc;
  for (int l = 0; l < cfg->num_hidden_layers; ++l) {
    const int32_t* btl = block_tables + (size_t)l * batch * max_pages;
    if (batch == 1) {
      rc = run_layer_fused(cfg, &w->layers[l], w->rope_cos, w->rope_sin, pool, btl, max_pages, positions,
                           x, x_p, workspace, L, st);
      if (rc < 0) return rc;
      if (rc == 1) continue;
    }
    rc = run_layer(cfg, &w->layers[l], w->rope_cos, w->rope_sin, pool, btl, max_pages, max_pages,
                   positions, batch, x, x_p, workspace, L, st);
    if (rc) return rc;
  }
  GemmArgs a{};
  a.W = w->embed;
  a.w_groups = (V + 15) / 16;
  a.xw = w->final_norm;
  a.N = V;
  a.K = H;
  a.eps = cfg->rms_norm_eps;
  a.err = err;
  a.amax_part = at<unsigned long long>(workspace, L.amax_part);
  rc = gemm_batched(EPI_LOGITS, V, batch, a, [&](GemmArgs& c, int b0) {
    c.X = packed_at(x_p, b0, H);
    c.logits = logits ? logits + (size_t)b0 * V : nullptr;
    c.next_tok = next_tokens + b0;
  }, st);
  if (rc) return rc;
  return 0;
}

// Prefill workspace: error word, the prompt's FP32 hidden rows, the packed
// BF16 hi/lo projection inputs (normed rows, attention output, SwiGLU
// output), q and the LM head's per-tile maxima.
struct PrefillLayout {
  size_t err, x, xb, q, ob, act, part, amax, total;
};

// The two residual projections of a prefill layer (output, down).
static PgemmPlan prefill_o_plan(const pkv_config* cfg, int32_t T) {
  return plan_prefill_gemm(cfg->hidden_size / 16, T, cfg->num_attention_heads * cfg->head_dim, true);
}
static PgemmPlan prefill_down_plan(const pkv_config* cfg, int32_t T) {
  return plan_prefill_gemm(cfg->hidden_size / 16, T, cfg->intermediate_size, true);
}

static PrefillLayout prefill_layout(const pkv_config* cfg, int32_t T) {
  const size_t H = cfg->hidden_size, I = cfg->intermediate_size;
  const size_t QD = (size_t)cfg->num_attention_heads * cfg->head_dim;
  PrefillLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
  L.err = take(kWsHeaderBytes);
  L.x = take(sizeof(float) * T * H);
  L.xb = take(2 * (size_t)packed_pair_elems(T, (int)H));
  L.q = take(2 * (size_t)T * QD * 2);
  L.ob = take(2 * (size_t)packed_pair_elems(T, (int)QD));
  L.act = take(2 * (size_t)packed_pair_elems(T, (int)I));
  const int ks_o = prefill_o_plan(cfg, T).ks, ks_d = prefill_down_plan(cfg, T).ks;
  const size_t pr = (size_t)(ks_o > ks_d ? ks_o : ks_d) * T * H, pq = qkv_part_floats(cfg, T);
  L.part = take(sizeof(float) * (pr > pq ? pr : pq));
  L.amax = take(sizeof(unsigned long long) * plan_gemm(EPI_LOGITS, cfg->vocab_size, 1, H).tiles);
  L.total = off;
  return L;
}

size_t pkv_prefill_workspace_bytes(const pkv_config* cfg, int32_t num_tokens, int32_t max_pages) {
  if (check_cfg(cfg) || num_tokens < 1 || max_pages < 1) return 0;
  return prefill_layout(cfg, num_tokens).total;
}

int prefill(const pkv_config* cfg, const pkv_model_weights* w, const pkv_pool* pool,
            const int32_t* block_tables, int32_t max_pages, int32_t start_pos,
            const int32_t* token_ids, int32_t num_tokens, float* logits, int32_t* next_token,
            void* workspace, size_t ws_bytes, void* stream) {
  if (!w) return -EINVAL;
  int rc = check_cfg(cfg);
  if (rc) return rc;
  rc = check_pool(pool);
  if (rc) return rc;
  if (pool->num_kv_heads != cfg->num_key_value_heads || pool->head_dim != cfg->head_dim)
    return -EINVAL;
  if (num_tokens < 0 || max_pages < 1 || start_pos < 0) return -EINVAL;
  if (num_tokens > 65535) return -ENOTSUP;
  if (num_tokens == 0) return 0;
  if ((int64_t)start_pos + num_tokens > (int64_t)max_pages * pool->page_tokens ||
      (int64_t)start_pos + num_tokens > cfg->max_position_embeddings)
    return -EINVAL;
  if (cfg->num_hidden_layers < 1 || cfg->vocab_size < 1) return -EINVAL;
  if (!w->embed || !w->final_norm || !w->layers || !w->rope_cos || !w->rope_sin) return -EINVAL;
  if (!block_tables || !token_ids || !next_token || !workspace) return -EINVAL;
  if (!aligned(workspace, 256)) return -EINVAL;
  for (int l = 0; l < cfg->num_hidden_layers; ++l)
    if ((rc = check_layer_weights(&w->layers[l]))) return rc;
  const int H = cfg->hidden_size, V = cfg->vocab_size, T = num_tokens;
  const int Hq = cfg->num_attention_heads, Hkv = cfg->num_key_value_heads;
  const int I = cfg->intermediate_size, D = cfg->head_dim, QD = Hq * D;
  // the projections address their packed BF16 hi/lo inputs through a
  // 32-bit byte range
  const int64_t widest = H > I ? (H > QD ? H : QD) : (I > QD ? I : QD);
  if (2 * packed_pair_elems(T, (int)widest) > kMaxMatrixBytes) return -ENOTSUP;
  if (ws_bytes < pkv_prefill_workspace_bytes(cfg, num_tokens, max_pages)) return -ENOSPC;

  const hipStream_t st = (hipStream_t)stream;
  const PrefillLayout L = prefill_layout(cfg, T);
  float* x = at<float>(workspace, L.x);
  uint16_t* xb = at<uint16_t>(workspace, L.xb);
  uint16_t* q = at<uint16_t>(workspace, L.q);
  uint16_t* ob = at<uint16_t>(workspace, L.ob);
  uint16_t* act = at<uint16_t>(workspace, L.act);
  uint32_t* err = at<uint32_t>(workspace, L.err);
  const float eps = cfg->rms_norm_eps;

  float* part = at<float>(workspace, L.part);
  const PgemmPlan p_o = prefill_o_plan(cfg, T);
  const PgemmPlan p_gu = plan_prefill_gemm(I / 8, T, H, false);
  const PgemmPlan p_down = prefill_down_plan(cfg, T);

  // x = E[tokens]; the first layer's RMSNorm; every later RMSNorm is done by
  // the residual kernel that finishes the row before it
  if ((rc = io(launch_embed(w->embed, V, H, token_ids, x, nullptr, T, err, st)))) return rc;
  if ((rc = io(launch_prefill_norm(x, w->layers[0].attn_norm, H, T, eps, xb, st)))) return rc;
  for (int l = 0; l < cfg->num_hidden_layers; ++l) {
    const pkv_layer_weights* lw = &w->layers[l];
    const int32_t* bt = block_tables + (size_t)l * max_pages;
    PgemmArgs base{};
    base.T = T;
    base.err = err;

    // QKV + RoPE at start_pos + t, K/V into the prompt's pages
    {
      PgemmArgs a = base;
      a.W = lw->w_qkv;
      a.w_groups = (Hq + 2 * Hkv) * (D / 16);
      a.X = xb;
      a.N = (Hq + 2 * Hkv) * D;
      a.K = H;
      a.D = D;
      a.q_split = q;
      a.pv = pool_view(pool);
      a.bt = bt;
      a.bt_row = 0;
      a.bt_stride = max_pages;
      a.pos = nullptr;
      a.start_pos = start_pos;
      a.max_pos = cfg->max_position_embeddings;
      a.rcos = w->rope_cos;
      a.rsin = w->rope_sin;
      a.Hq = Hq;
      a.Hkv = Hkv;
      if ((rc = io(launch_tiled_qkv(cfg, a, part, st)))) return rc;
    }
    // causal attention over positions 0 .. start_pos + t
    {
      PattnArgs a{};
      a.q = q;
      a.pv = pool_view(pool);
      a.bt = bt;
      a.start_pos = start_pos;
      a.T = T;
      a.scale = 1.0f / sqrtf((float)D);
      a.out = ob;
      a.D = D;
      a.err = err;
      a.Hq = Hq;
      a.Hkv = Hkv;
      a.G = Hq / Hkv;
      if ((rc = io(launch_prefill_attention(a, st)))) return rc;
    }
    // x += W_o o, then the MLP's RMSNorm
    {
      PgemmArgs a = base;
      a.W = lw->w_o;
      a.w_groups = H / 16;
      a.X = ob;
      a.N = H;
      a.K = QD;
      a.part = part;
      a.ksplit = p_o.ks;
      if ((rc = io(launch_prefill_gemm(EPI_RESID, a, p_o, st)))) return rc;
      if ((rc = io(launch_prefill_resid(x, part, p_o.ks, T, H, lw->mlp_norm, eps, xb, st)))) return rc;
    }
    // gate/up, SwiGLU
    {
      PgemmArgs a = base;
      a.W = lw->w_gate_up;
      a.w_groups = I / 8;
      a.X = xb;
      a.N = 2 * I;
      a.K = H;
      a.act = act;
      a.I = I;
      if ((rc = io(launch_prefill_gemm(EPI_SWIGLU, a, p_gu, st)))) return rc;
    }
    // x += W_down a, then the next layer's attention RMSNorm
    {
      PgemmArgs a = base;
      a.W = lw->w_down;
      a.w_groups = H / 16;
      a.X = act;
      a.N = H;
      a.K = I;
      a.part = part;
      a.ksplit = p_down.ks;
      if ((rc = io(launch_prefill_gemm(EPI_RESID, a, p_down, st)))) return rc;
      const uint16_t* nw = l + 1 < cfg->num_hidden_layers ? w->layers[l + 1].attn_norm : nullptr;
      if ((rc = io(launch_prefill_resid(x, part, p_down.ks, T, H, nw, eps, xb, st)))) return rc;
    }
  }
  // final norm, LM head and argmax of the last prompt token only
  GemmArgs a{};
  a.W = w->embed;
  a.w_groups = (V + 15) / 16;
  a.xw = w->final_norm;
  a.N = V;
  a.K = H;
  a.B = 1;
  a.eps = eps;
  a.err = err;
  a.amax_part = at<unsigned long long>(workspace, L.amax);
  a.X = x + (size_t)(T - 1) * H;
  a.x_plain = 1;
  a.logits = logits;
  a.next_tok = next_token;
  const GemmPlan p = plan_gemm(EPI_LOGITS, V, 1, H);
  a.ksplit = p.ks;
  return io(launch_gemm(EPI_LOGITS, a, p, st));
}

size_t pkv_sample_workspace_bytes(int32_t batch, int32_t vocab) {
  if (batch < 1 || vocab < 1 || batch > 65535) return 0;
  int chunk;
  const int W = sample_chunks(batch, vocab, &chunk);
  return sample_ws_carve(nullptr, batch, W, chunk).bytes;
}

int sample_tokens(const float* logits, int32_t batch, int32_t vocab, const float* temperature,
                  const float* top_p, const int32_t* top_k, const float* u, int32_t* tokens,
                  void* workspace, size_t ws_bytes, void* stream) {
  if (batch < 0 || vocab < 1) return -EINVAL;
  if (batch > 65535) return -ENOTSUP;
  if (batch == 0) return 0;
  if (!logits || !temperature || !top_p || !top_k || !u || !tokens || !workspace) return -EINVAL;
  if (!aligned(workspace, 256)) return -EINVAL;
  if (ws_bytes < pkv_sample_workspace_bytes(batch, vocab)) return -ENOSPC;
  int chunk;
  const int W = sample_chunks(batch, vocab, &chunk);
  const SampleWs ws = sample_ws_carve(workspace, batch, W, chunk);
  return io(launch_sample(logits, batch, vocab, temperature, top_p, top_k, u, tokens, ws, W, chunk,
                          (hipStream_t)stream));
}

size_t pkv_packed_weight_bytes(int32_t rows, int32_t cols, int32_t layout) {
  if (rows < 1 || cols < 32 || cols % 32 != 0 || layout < PACK_ROWS || layout > PACK_QKV128) return 0;
  if (layout == PKV_PACK_QKV && rows % 64 != 0) return 0;
  if (layout == PKV_PACK_QKV128 && rows % 128 != 0) return 0;
  if (layout == PKV_PACK_GATE_UP && rows % 16 != 0) return 0;
  return (size_t)packed_weight_elems(rows, cols, layout) * 2;
}

int pkv_pack_weight(const uint16_t* src, int32_t rows, int32_t cols, int32_t layout, uint16_t* dst,
                    void* stream) {
  if (!src || !dst || pkv_packed_weight_bytes(rows, cols, layout) == 0) return -EINVAL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return -EINVAL;
  if ((int64_t)rows * cols * 2 > INT32_MAX) return -ENOTSUP;
  return io(launch_pack_weight(src, rows, cols, layout, dst, (hipStream_t)stream));
}

int pkv_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace || !aligned(workspace, 256)) return -EINVAL;
  if (ws_bytes == 0) return 0;
  return io(launch_fill_zero(workspace, ws_bytes, (hipStream_t)stream));
}

int pkv_rope_table(float theta, int32_t head_dim, int32_t max_pos, float* cos_out, float* sin_out,
                   void* stream) {
  if (!cos_out || !sin_out || max_pos < 1 || !(theta > 0.f) || !isfinite(theta)) return -EINVAL;
  if (!head_dim_ok(head_dim)) return -ENOTSUP;
  return io(launch_rope_table((double)theta, head_dim, max_pos, cos_out, sin_out,
                              (hipStream_t)stream));
}

int pkv_probe_read(const void* buf, int64_t bytes, int32_t workgroups, float* sink, void* stream) {
  if (!buf || !sink || !aligned(buf, 16) || bytes < 16 || bytes % 16 != 0) return -EINVAL;
  if (workgroups < 1 || workgroups > 1 << 20) return -EINVAL;
  return io(launch_probe_read(buf, bytes, workgroups, sink, (hipStream_t)stream));
}

int pkv_probe_paged_read(const pkv_pool* pool, int32_t num_q_heads, const int32_t* block_table,
                         int32_t max_pages, const int32_t* context_lens, int32_t batch, float* sink,
                         void* stream) {
  AttnArgs a{};
  const uint16_t* any = (const uint16_t*)sink;  // q and out are not read or written
  int rc = prepare_attention_call(pool, any, num_q_heads, block_table, max_pages, context_lens, batch,
                                  1.0f, sink, &a);
  if (rc || batch == 0) return rc;
  return io(launch_probe_paged_read(a, batch, sink, (hipStream_t)stream));
}

int pkv_probe_empty(int32_t launches, int32_t workgroups, void* stream) {
  if (launches < 0 || workgroups < 1 || workgroups > 1 << 20) return -EINVAL;
  return io(launch_probe_empty(launches, workgroups, (hipStream_t)stream));
}

int pkv_set_fused_layer(int32_t enable) {
  return g_fused_layer.exchange(enable ? 1 : 0);
}

int pkv_fused_layer_plan(const pkv_config* cfg, int32_t batch, int32_t max_pages, int32_t page_tokens,
                         int32_t compute_units) {
  int rc = check_cfg(cfg);
  if (rc) return rc;
  if (batch < 0 || max_pages < 1 || compute_units < 1) return -EINVAL;
  if (!page_tokens_ok(page_tokens)) return -ENOTSUP;
  if (batch != 1) return 0;
  FusedArgs a{};
  return plan_fused_layer(cfg->hidden_size, cfg->num_attention_heads, cfg->num_key_value_heads,
                          cfg->head_dim, cfg->intermediate_size, table_tiles(max_pages, page_tokens),
                          compute_units, &a)
             ? 1
             : 0;
}

int pkv_device_error(void* workspace, void* stream) {
  if (!workspace || !aligned(workspace, 256)) return -EINVAL;
  const hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return io(hipErrorUnknown);
  uint32_t bits = 0;
  if (hipMemcpy(&bits, workspace, sizeof bits, hipMemcpyDeviceToHost) != hipSuccess)
    return io(hipErrorUnknown);
  const uint32_t zero = 0;
  if (hipMemcpy(workspace, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
    return io(hipErrorUnknown);
  return (int)(bits & 0x7fffffffu);
}

}  // extern "C"
