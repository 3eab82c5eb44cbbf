// Internal declarations of the gfx950 paged-KV decode library: device
// helpers, kernel argument blocks, the workspace layout and the launch plans
// shared by the host entry points (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct pkv_pool;

namespace pkv {

constexpr int kPageTokens = 16;   // the default page size; 256 is also supported
constexpr int kTile = 16;          // tokens of one attention tile (one matrix-core tile)
constexpr int kHeadDim = 64;       // the default head width; 128 is also supported
constexpr int kMaxHeadDim = 128;
constexpr int kMaxGroup = 16;      // GQA group: one 16-wide matrix-core tile

enum : uint32_t { ERR_PAGE = 1u, ERR_LENGTH = 2u, ERR_ROPE = 4u, ERR_TOKEN = 8u, ERR_SYNC = 16u };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- device ---

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// FP32 -> BF16 bits, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Across the four 16-lane rows of a wave (lanes l, l ^ 16, l ^ 32, l ^ 48)
// by the row-swap permutes: each step is one VALU instruction pair instead
// of a round trip through the LDS crossbar, and computes what an exchange
// with lane l ^ 16, then l ^ 32, would (the two operands of each add or max
// are the same two values, so the result is bitwise the same).
__device__ __forceinline__ float rows_sum4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows_max4(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Over all 64 lanes of a wave, the result in every lane: pairs and quads
// by quad permutes, 8 and 16 lanes by the row half-mirror and row mirror
// (after the quads every lane of a quad holds its quad's value, so a
// mirror adds the neighbouring quad, then the neighbouring half-row), then
// the four rows by the row-swap permutes.  VALU only.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += __uint_as_float(dpp_u<0xb1>(__float_as_uint(v)));   // quad_perm [1,0,3,2]
  v += __uint_as_float(dpp_u<0x4e>(__float_as_uint(v)));   // quad_perm [2,3,0,1]
  v += __uint_as_float(dpp_u<0x141>(__float_as_uint(v)));  // row_half_mirror
  v += __uint_as_float(dpp_u<0x140>(__float_as_uint(v)));  // row_mirror
  return rows_sum4(v);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp_u<0xb1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u<0x4e>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u<0x141>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp_u<0x140>(__float_as_uint(v))));
  return rows_max4(v);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint64_t wave_sum(uint64_t v) {
  v += dpp_u64<0xb1>(v);
  v += dpp_u64<0x4e>(v);
  v += dpp_u64<0x141>(v);
  v += dpp_u64<0x140>(v);
  const auto a0 = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  const auto a1 = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
  v = (((uint64_t)a1[0] << 32) | a0[0]) + (((uint64_t)a1[1] << 32) | a0[1]);
  const auto b0 = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  const auto b1 = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
  return (((uint64_t)b1[0] << 32) | b0[0]) + (((uint64_t)b1[1] << 32) | b0[1]);
}

// The value of lane l ^ 32.
__device__ __forceinline__ float xor32_lane(float v) {
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? b[0] : b[1]);
}

__device__ __forceinline__ void set_error(uint32_t* err, uint32_t bits) {
  __hip_atomic_fetch_or(err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------- packed layouts ---
//
// Weights (BF16), packed once at load time: the matrix is cut into groups
// of 16 rows (rows past the end are zero) and each group's K into 32-wide
// steps; block (group G, step s) is 1 KiB holding, for lane l = 16 i + m,
// the 8 values W[row(G, m)][32 s + 8 i .. + 8].  A wave streams a group's
// K range as contiguous 1 KiB blocks, already in the A-operand layout of
// v_mfma_f32_16x16x32_bf16.  row(G, m) depends on the layout kind:
enum PackKind { PACK_ROWS = 0, PACK_QKV = 1, PACK_GATE_UP = 2, PACK_QKV128 = 3 };

// Matrix row held by row m (0..15) of 16-row group G, or -1 (zero rows).
__host__ __device__ inline int packed_row(int kind, int rows, int G, int m) {
  if (kind == PACK_QKV || kind == PACK_QKV128) {
    // head width D: group G is head G / (D / 16), RoPE pairs
    // j = 8 (G % (D / 16)) + i, rows j and j + D / 2
    const int D = kind == PACK_QKV ? 64 : 128, gph = D / 16;
    const int j0 = 8 * (G % gph);
    const int r = (G / gph) * D + (m < 8 ? j0 + m : D / 2 + j0 + (m - 8));
    return r < rows ? r : -1;
  }
  if (kind == PACK_GATE_UP) {
    // group G: gate rows i .. i + 7 then the matching up rows (I = rows / 2)
    const int I = rows / 2, i = 8 * G + (m & 7);
    return i < I ? (m < 8 ? i : I + i) : -1;
  }
  const int r = 16 * G + m;
  return r < rows ? r : -1;
}

inline int64_t packed_weight_elems(int rows, int cols, int kind) {
  const int per = kind == PACK_GATE_UP ? 8 : 16;  // matrix rows of each kind per group
  const int64_t groups = kind == PACK_GATE_UP ? ((rows / 2) + per - 1) / per : (rows + per - 1) / per;
  return groups * 16 * (int64_t)cols;
}

// Activations (FP32) that feed a projection, [B][K] re-laid out so that a
// lane's B operand of one step is 32 contiguous bytes: column block cb of
// 16 columns, step s, lane l = 16 i + c holds X[16 cb + c][32 s + 8 i .. + 8].
__host__ __device__ inline int64_t packed_act_index(int b, int k, int K) {
  const int S = K >> 5;
  return ((((int64_t)(b >> 4) * S + (k >> 5)) * 64 + ((k & 31) >> 3) * 16 + (b & 15)) << 3) + (k & 7);
}

inline int64_t packed_act_elems(int B, int K) { return (int64_t)((B + 15) / 16) * 16 * K; }

// --------------------------------------------------------- arguments ---

// Where the pages live.  Page p of PT = kTile << pt_shift tokens holds a K
// block at k + p * stride and a V block at v + p * stride: one buffer of
// whole pages (v = k + the K block, stride = both blocks), or separate K and
// V pools (stride = one block).  Both blocks are stored in 16-token tiles,
// so that a tile of one kv head is one contiguous matrix-core operand
// whatever the page size:
//   K [PT / 16][Hkv][D / 8][16 slots][8 dims]  (dims in chunks of 8: a
//     lane's 16-byte A operand of the score product is one chunk of one
//     slot, and a wave's 64 lanes read 1 KiB contiguously);
//   V [PT / 16][Hkv][D][16 slots]              (V transposed: a lane's
//     4-token B operand of the value product is 8 contiguous bytes).
struct PoolView {
  uint16_t* k;
  uint16_t* v;
  int64_t stride;      // BF16 elements from one page to the next
  int32_t num_pages;
  int32_t pt_shift;    // log2(PT / 16): 0 (16-token pages) or 4 (256)
  int32_t hkv;         // kv heads
};

// Dimension d of token `slot`'s K (kv head h) of page `page`; dimensions
// d .. d | 7 follow contiguously.
__host__ __device__ inline int64_t pv_k_elem(const PoolView& p, int page, int h, int slot, int d, int D) {
  return (int64_t)page * p.stride +
         (((((int64_t)(slot >> 4) * p.hkv + h) * (D >> 3) + (d >> 3)) * kTile + (slot & (kTile - 1))) << 3) +
         (d & 7);
}
// V of dimension d, token `slot`; dimension d + 1 is kTile elements further.
__host__ __device__ inline int64_t pv_v_index(const PoolView& p, int page, int h, int d, int slot,
                                               int D) {
  return (int64_t)page * p.stride + (((int64_t)(slot >> 4) * p.hkv + h) * D + d) * kTile +
         (slot & (kTile - 1));
}

struct AttnArgs {
  const uint16_t* q;       // BF16: [B][Hq][D], or [B][Hq][2][D] hi/lo split (kQSplit)
  PoolView pv;
  const int32_t* bt;       // sequence b's table starts at bt + b * bt_row
  int32_t bt_stride;       // table width (max_pages)
  int32_t bt_row;          // elements between sequences' rows (0: one shared row)
  const int32_t* lens;     // [B]: attention length, or position (len_add = 1)
  int32_t len_add;
  float scale;
  float* out;              // out_packed 0: [B][Hq][D] FP32; 1: packed FP32 [B][Hq * D]
  int32_t out_packed;      // (packed_act_index); 2: packed BF16 hi/lo pairs (packed_pair_index)
  float* part;             // split partial records [B][Hkv][max_splits][attn_rec(D)]
  uint32_t* err;
  int32_t Hq, Hkv, G;
  int32_t max_splits;      // splits per sequence: the table's tiles / (kAttnWaves * pw)
  int32_t pw;              // tiles per wave (kAttnPW or kAttnPWLarge)
  int32_t D;               // head width, 64 or 128
};

enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3 };

struct GemmArgs {
  const uint16_t* W;       // packed BF16 weights of N rows x K
  const float* X;          // FP32 activations, packed ([B][K] if x_plain)
  int32_t x_plain;         // X is a plain row-major [B][K] array
  const uint16_t* xw;      // RMSNorm weight [K] (epilogues that normalise)
  int32_t N, K, B;
  int32_t w_groups;        // 16-row groups in the packed W
  float eps;
  uint32_t* err;
  // EPI_RESID: out[b][n] = resid[b][n] + y (plain), and packed into
  // out_packed (if not null) for the next projection.  With ksplit > 1 the
  // workgroups of K split s write their sums to part[s][b][n] and a reduce
  // kernel adds resid and the splits in split order.
  float* out;
  const float* resid;
  float* out_packed;
  float* part;
  int32_t ksplit;
  // EPI_QKV
  uint16_t* q_split;       // [B][Hq][2][D]: each head's q as BF16 hi, then lo
  PoolView pv;
  const int32_t* bt;
  int32_t bt_stride;       // table width (max_pages)
  int32_t bt_row;          // elements between columns' rows (0: one shared row)
  const int32_t* pos;
  const float* rcos;
  const float* rsin;
  int32_t max_pos;
  int32_t Hq, Hkv;
  int32_t D;               // head width, 64 or 128
  // EPI_SWIGLU: act[b][i], i < I, packed (the down projection's input)
  float* act;
  int32_t I;
  // EPI_LOGITS
  float* logits;                 // [B][N] or null
  unsigned long long* amax_part; // [tiles][B] per-tile packed maxima
  int32_t* next_tok;             // [B]
};

// Prefill of one sequence's prompt of T tokens.  Activations feeding a
// projection are FP32 values stored as two BF16 halves x = hi + lo (~16
// significant bits, as the decode projections keep), packed like the
// weights with tokens in place of rows: token group c (16 tokens), step s,
// half h: a 1 KiB block whose 16-byte chunk l = 16 i + m holds
// half h of X[16 c + m][32 s + 8 i .. + 8]; a step's hi block is followed by
// its lo block.  Both operands of the matrix-core product are thus
// contiguous 1 KiB blocks.  Tokens T .. 16 ceil(T / 16) - 1 are padding.
__host__ __device__ inline int64_t packed_pair_index(int t, int k, int K, int h) {
  const int S = K >> 5;
  return (((((int64_t)(t >> 4) * S + (k >> 5)) * 2 + h) * 64 + ((k & 31) >> 3) * 16 + (t & 15)) << 3) +
         (k & 7);
}

inline int64_t packed_pair_elems(int T, int K) { return (int64_t)((T + 15) / 16) * 16 * K * 2; }

struct PgemmArgs {
  const uint16_t* W;       // packed BF16 weights, w_groups 16-row groups x K
  int32_t w_groups;
  const uint16_t* X;       // packed BF16 hi/lo activation pairs
  int32_t N, K, T;
  uint32_t* err;
  // EPI_RESID: workgroups of K split s write their sums y_s to
  // part[s][t][n] (plain [ksplit][T][N]); a per-token kernel then adds the
  // residual and the splits in split order
  float* part;
  int32_t ksplit;
  // EPI_QKV: q as BF16 hi, lo halves [T][Hq][2][D]; k, v into the pages of
  // position pos[t] (or start_pos + t if pos is null) through the table row
  // bt + t * bt_row (bt_row 0: one sequence's table); positions outside
  // [0, max_pos) or past the table's bt_stride pages set device errors
  uint16_t* q_split;
  PoolView pv;
  const int32_t* bt;
  int32_t bt_row, bt_stride;
  const int32_t* pos;
  int32_t start_pos, max_pos;
  const float* rcos;
  const float* rsin;
  int32_t Hq, Hkv;
  int32_t D;               // head width, 64 or 128
  // EPI_SWIGLU: act = silu(gate) * up, packed BF16 hi/lo pairs
  uint16_t* act;
  int32_t I;
  // EPI_LOGITS: FP32 logits [T][N] (if not null) and, per token and
  // half row tile (2 per tile), the largest logit packed with its index:
  // amax_part[2 * row_tiles][T], reduced by the argmax kernel
  float* logits;
  unsigned long long* amax_part;
};

struct PattnArgs {
  const uint16_t* q;       // [T][Hq][2][D] BF16 hi, lo
  PoolView pv;
  const int32_t* bt;       // the sequence's table for this layer
  int32_t start_pos, T;
  float scale;
  uint16_t* out;           // packed BF16 hi/lo pairs (the output projection's input)
  uint32_t* err;
  int32_t Hq, Hkv, G;
  int32_t D;               // head width, 64 or 128
};

// A prefill GEMM launch: 2 x 2 waves per workgroup, each 16 rg rows by
// 16 cg tokens, and ks workgroups splitting K per tile (tiles * ks in all).
struct PgemmPlan {
  int rg, cg, tiles, ks;
};

constexpr int kPfTargetWgs = 240;     // about one workgroup per compute unit
// 32-wide K steps per split, at least: 8 for decode-sized batches (up to
// 128 tokens), whose few row tiles need many splits to fill the chip; 16
// for prompts, whose token tiles already do
constexpr int kPfMinSplitSteps = 8;
constexpr int kPfMinSplitStepsLong = 16;
constexpr int kPfMaxSplits = 16;

inline int pf_tiles(int w_groups, int T, int rg, int cg) {
  return ((w_groups + 2 * rg - 1) / (2 * rg)) * ((T + 32 * cg - 1) / (32 * cg));
}

// Tile shape (and K split) of a prefill projection.  Large tiles read each
// operand byte fewer times; where they give too few workgroups, a residual
// projection (can_split) splits K instead, and the other epilogues, which
// need whole sums, take smaller tiles.
inline PgemmPlan plan_prefill_gemm(int w_groups, int T, int K, bool can_split) {
  PgemmPlan p{};
  if (can_split) {
    static const int cand[4][2] = {{8, 4}, {4, 4}, {2, 4}, {2, 2}};
    const int steps = K / 32;
    const int min_steps = T <= 128 ? kPfMinSplitSteps : kPfMinSplitStepsLong;
    for (const auto& c : cand) {
      if (c[0] == 2 && c[1] == 4 && T <= 64) continue;  // as below
      p.rg = c[0];
      p.cg = c[1];
      p.tiles = pf_tiles(w_groups, T, p.rg, p.cg);
      int ks = (kPfTargetWgs + p.tiles - 1) / p.tiles;
      const int most = steps / min_steps > 1 ? steps / min_steps : 1;
      p.ks = ks < most ? ks : most;
      // more partials than this cost the residual kernel that adds them more
      // than the extra workgroups gain
      if (p.ks > kPfMaxSplits) p.ks = kPfMaxSplits;
      if (p.tiles * p.ks >= kPfTargetWgs) break;
    }
    return p;
  }
  static const int cand[4][2] = {{8, 4}, {4, 4}, {2, 4}, {2, 2}};
  p.ks = 1;
  for (const auto& c : cand) {
    // 64-row tiles 128 tokens wide for at most 64 tokens: the 64-token
    // tiles of the same rows give as many workgroups without the empty half
    if (c[0] == 2 && c[1] == 4 && T <= 64) continue;
    p.rg = c[0];
    p.cg = c[1];
    p.tiles = pf_tiles(w_groups, T, p.rg, p.cg);
    if (p.tiles >= kPfTargetWgs) break;
  }
  return p;
}

// K splits of the tiled QKV projection: 1 when its row and token tiles
// alone give at least half the target workgroups; otherwise enough to reach
// the target, at least 8 K steps each.  The split sums are finished by
// qkv_finish_kernel (RoPE needs whole sums).
inline int qkv_splits(const PgemmPlan& p, int K) {
  if (p.tiles * 2 >= kPfTargetWgs) return 1;
  const int most = (K / 32) / 8;
  const int ks = (kPfTargetWgs + p.tiles - 1) / p.tiles;
  return ks < most ? (ks > 1 ? ks : 1) : (most > 1 ? most : 1);
}

// Sampling after the LM head: per-sequence workspace of the radix select
// (the first level's 2048-bucket count and fixed-point mass histograms, the
// tokens of the bucket it chooses, which the later levels select from), the
// choice record passed between its launches, and per-chunk partials.
constexpr int kSampleChoiceBytes = 24;
struct SampleWs {
  uint32_t* cnt;      // [B][2048] first-level token counts
  uint64_t* mass;     // [B][2048] first-level masses
  uint64_t* sum;      // [B][W] the softmax normaliser's per-chunk parts (fixed point)
  void* choice;       // [B] records: the choice after the first level
  float* wmax;        // [B][W] chunk maxima
  uint64_t* wmass;    // [B][W] chunk mass above the chosen first-level bucket
  uint32_t* ncand;    // [B][W] per chunk, its tokens in the chosen first-level bucket
  uint32_t* cand;     // [B][W][chunk][2] their (key, vocabulary index), per chunk
  size_t bytes;
};
SampleWs sample_ws_carve(void* base, int B, int W, int chunk);
// workgroups per sequence for B sequences of V logits; *chunk = logits each
int sample_chunks(int B, int V, int* chunk);
hipError_t launch_sample(const float* logits, int B, int V, const float* temperature,
                         const float* top_p, const int32_t* top_k, const float* u, int32_t* tokens,
                         const SampleWs& ws, int W, int chunk, hipStream_t st);

// ------------------------------------------------------------ plans ---

// Attention: kAttnWaves waves per workgroup, kAttnPW pages per wave per
// split.
#ifndef PKV_ATTN_WAVES
#define PKV_ATTN_WAVES 4
#endif
constexpr int kAttnWaves = PKV_ATTN_WAVES;
constexpr int kAttnPW = 2;       // tiles per wave of a small call
constexpr int kAttnPWLarge = 4;  // tiles per wave of a large one
constexpr int kAttnPagesPerSplit = kAttnWaves * kAttnPW;
// From this many workgroups at kAttnPW (batch x kv heads x splits of the
// table) a call takes kAttnPWLarge tiles per wave: half the workgroups,
// records and merge work, more loads in flight per wave.  Below it the
// shorter waves finish sooner.
constexpr int64_t kAttnLargeWgs = 4096;
// One split's partial record: m[16], l[16], o[16][64] floats.
constexpr int attn_rec(int D) { return 16 + 16 + 16 * D; }

// Splits of a block table of max_tiles 16-token tiles (max_pages pages of
// 16 << pt_shift tokens: max_tiles = max_pages << pt_shift).
inline int attn_max_splits(int64_t max_tiles, int pw = kAttnPW) {
  const int cp = kAttnWaves * pw;
  return (int)((max_tiles + cp - 1) / cp);
}
// Tiles per wave of a call over `batch` sequences of Hkv kv heads.
inline int attn_pw(int batch, int Hkv, int64_t max_tiles) {
  return (int64_t)batch * Hkv * attn_max_splits(max_tiles) >= kAttnLargeWgs ? kAttnPWLarge : kAttnPW;
}

// A GEMM launch: `rg` groups of 16 output rows per workgroup, `nw` waves
// splitting K inside the workgroup, `ct` groups of 16 batch columns, `ks`
// workgroups splitting K per row tile (tiles * ks workgroups in all).
struct GemmPlan {
  int tiles, ct, rg, nw, ks;
};

constexpr int kGemmMaxCols = 64;  // batch columns per launch (ct <= 4)
constexpr int kMaxDim = 65536;    // largest hidden / intermediate size
constexpr int64_t kMaxMatrixBytes = (int64_t)1 << 31;  // largest weight matrix

// 16-column groups per launch: the weights stream once per launch, so a
// batch of 64 reads them once
inline int gemm_ct(int B) { return B <= 16 ? 1 : (B <= 32 ? 2 : 4); }

// A residual projection whose row tiles alone give few workgroups and whose
// K is long (the down projection) splits K over workgroups (up to about one
// workgroup per compute unit), where one workgroup per row tile would leave
// most of the chip idle.
constexpr int kSplitMinK = 4096;
constexpr int kSplitTargetWgs = 512;
// The split count aims at one workgroup per compute unit (256): one round,
// with no second, partly filled one.  Measured per split count of the
// Llama-shape down projection (64 row tiles) on the batch-16 step: 2, 3, 4,
// 6, 8 splits give 1.021, 0.991, 0.962, 0.995, 0.969 ms; the batch-1 Qwen
// layer (28 tiles): 4, 6, 9, 18 splits give 27.8, 27.6, 27.2, 28.2 us.
constexpr int kSplitRoundWgs = 256;
constexpr int kSplitMinSteps = 8;  // 32-wide K steps per split, at least
// The QKV and O launches of one 16-column group (one 16-row tile per
// workgroup) run 8 waves for a few sequences and 4 from this many on:
// measured 1 % faster per batch-16 step with 4, 2 % slower per batch-1
// layer (the threshold between the two is not measured).
constexpr int kGemmFourWaveCols = 9;

inline bool gemm_split(int epi, int N, int K) {
  return epi == EPI_RESID && K >= kSplitMinK && (N + 15) / 16 < kSplitTargetWgs / 2;
}

// The LM head of one column group with at least this many sequences takes
// 64-row tiles: each workgroup reads the whole activation block once for
// its rows, and with 32-row tiles those reads matched the head's 525 MB of
// weights (Llama-1B shape) byte for byte.  Measured on the batch-16 step:
// 0.966 -> 0.961 ms; at batch 1 (no activation reads to save) the halved
// workgroup count made the step 1 % slower.
constexpr int kLmWideTileCols = kGemmFourWaveCols;

inline int gemm_rows_per_tile(int epi, int ct, bool split, int B) {
  if (ct == 4) return 16;  // 4 column groups: one row group keeps the registers in bounds
  if (split) return 32;
  if (epi == EPI_QKV || epi == EPI_RESID) return 16;
  if (epi == EPI_LOGITS && ct == 1 && B >= kLmWideTileCols) return 64;
  return ct == 1 ? 32 : 16;
}

inline GemmPlan plan_gemm(int epi, int N, int B, int K) {
  GemmPlan p;
  p.ct = gemm_ct(B);
  const bool split = gemm_split(epi, N, K);
  const int R = gemm_rows_per_tile(epi, p.ct, split, B);
  p.rg = R / 16;
  p.nw = split ? 4
         : (epi == EPI_RESID || epi == EPI_QKV ? (p.ct == 1 && B >= kGemmFourWaveCols ? 4 : 8) : 4);
  // the gate/up tile holds R/2 gate rows and the R/2 matching up rows
  const int rows = epi == EPI_SWIGLU ? N / 2 : N;
  const int per = epi == EPI_SWIGLU ? R / 2 : R;
  p.tiles = (rows + per - 1) / per;
  p.ks = 1;
  if (split) {
    const int steps = K / 32;
    int ks = kSplitRoundWgs / p.tiles;
    if (ks > steps / kSplitMinSteps) ks = steps / kSplitMinSteps;
    p.ks = ks < 1 ? 1 : ks;
  }
  return p;
}

// Floats of split partial sums a residual projection needs for any launch
// of at most Bc columns (the split count depends on the column tiling, so
// both tilings' largest launches are checked).
inline size_t gemm_part_floats(int N, int Bc, int K) {
  size_t most = 0;
  const int cand[2] = {Bc < 16 ? Bc : 16, Bc};
  for (int b : cand) {
    if (b < 1) continue;
    const GemmPlan p = plan_gemm(EPI_RESID, N, b, K);
    const size_t f = p.ks > 1 ? (size_t)p.ks * b * N : 0;
    most = f > most ? f : most;
  }
  return most;
}

// ------------------------------------------------- single-launch layer ---
//
// A batch-1 decoder layer in one launch (fused_layer.hip): one workgroup per
// compute unit; kFusedWaves loader waves stream the workgroup's share of the
// layer's weights into LDS from kernel start, and as many worker waves
// compute, passing the small vectors between the layer's phases as 8-byte
// (value, epoch) words.
constexpr int kFusedWaves = 4;          // worker waves (and loader waves) per workgroup
constexpr int kFusedThreads = 2 * kFusedWaves * 64;
constexpr int kFusedMaxHidden = 8 * kFusedWaves * 64;  // one 8-value chunk of the hidden vector per worker lane
constexpr int kFusedCap = 33;           // 1 KiB weight slots per worker wave
constexpr int kFusedX = 5632;           // floats of the phase-input buffer
constexpr int kFusedMaxUnits = 8;       // units of one phase per workgroup
constexpr int kFusedMaxWgs = 512;       // workgroups (compute units) at most
constexpr int kFusedAttnTiles = kFusedWaves * 2;  // 16-token tiles per attention unit
constexpr int kFusedRedRows = kFusedWaves;        // output rows per reduction unit (one per worker wave)
// copies of the h1 exchange words: every workgroup reads them, so each copy
// serves one eighth of the grid
constexpr int kFusedCopies = 8;

// Every workspace, whatever call it serves, starts with this header: the
// sticky device-error word at byte 0 and, from byte kWsFusedEpochs, the
// single-launch layer's per-workgroup launch counters.  The counters have
// to survive the calls of other shapes and entry points that may use the
// same workspace between two launches of that layer, so no layout puts
// anything else there.
constexpr size_t kWsFusedEpochs = 256;
constexpr size_t kWsHeaderBytes = kWsFusedEpochs + 4 * (size_t)kFusedMaxWgs;

// The epoch half of the single-launch layer's (value, epoch) exchange
// words: the launch counter's low 21 bits inside a signalling-NaN bit
// pattern.  No arithmetic result, BF16 pair, count or index that another
// call stores in a workspace has these bits, so a word left at the same
// place by a call of another shape never passes for the current launch's
// (the counter itself is kept plain).
__host__ __device__ inline uint32_t fused_epoch_tag(uint32_t n) { return 0x7FA00000u | (n & 0x1FFFFFu); }

// Phases, in order: QKV; attention; O; gate/up with the down projection's
// matching columns (each gate/up unit multiplies its 8 SwiGLU outputs into
// a partial of the layer output); the reduction of those partials.
enum FusedPhase { FP_QKV = 0, FP_ATT = 1, FP_O = 2, FP_GU = 3, FP_RED = 4, FP_COUNT = 5 };

// Units of a phase: n units of `slots` 1 KiB weight slots each (a 16-row
// group of the matrix over `slots` 32-wide K steps) and, for gate/up,
// `extra` slots of the down projection (its 8 matching columns, four 16-row
// groups per slot).
struct FusedGeo {
  int n, slots, extra;
};

__host__ __device__ inline FusedGeo fused_geo(int P, int H, int Hq, int Hkv, int D, int I, int ns) {
  FusedGeo g{0, 0, 0};
  switch (P) {
    case FP_QKV: g = {(Hq + 2 * Hkv) * D / 16, H / 32, 0}; break;
    case FP_ATT: g = {Hkv * ns, 0, 0}; break;
    case FP_O: g = {H / 16, Hq * D / 32, 0}; break;
    case FP_GU: g = {I / 8, H / 32, H / 64}; break;
    default: g = {H / kFusedRedRows, 0, 0}; break;
  }
  return g;
}

// Units of phase P are dealt round-robin over the workgroups from workgroup
// first[P]: unit u runs on workgroup (first[P] + u) mod nwg.
__host__ __device__ inline int fused_first_unit(int wg, int first, int nwg) {
  return ((wg - first) % nwg + nwg) % nwg;
}
__host__ __device__ inline int fused_unit_count(int n, int k0, int nwg) {
  return n > k0 ? (n - k0 + nwg - 1) / nwg : 0;
}
// Slots of wave w among `slots` (slots j = w, w + kFusedWaves, ...).
__host__ __device__ inline int fused_wave_slots(int slots, int w) {
  return slots > w ? (slots - w + kFusedWaves - 1) / kFusedWaves : 0;
}

// Words of one attention split's record: m and l per head, then O.
__host__ __device__ inline int fused_rec_len(int G, int D) { return G * (D + 2); }

struct FusedArgs {
  int32_t H, Hq, Hkv, D, I, G;
  float eps, scale;
  const uint16_t *attn_norm, *w_qkv, *w_o, *mlp_norm, *w_gu, *w_down;
  const float *rcos, *rsin;
  int32_t max_pos;
  PoolView pv;
  const int32_t* bt;
  int32_t bt_stride;
  const int32_t* pos;
  float* hidden;          // [H] in / out
  float* hidden_packed;   // packed copy of the output (or null)
  uint32_t* err;
  uint32_t* epoch;        // [nwg] per-workgroup launch counters
  // (value, epoch) words passed between phases: q, the new K and V rows, the
  // attention output (or split records), h1 (kFusedCopies copies), every
  // workgroup's partial of the layer output ([H / 4][nwg][4])
  uint64_t *q, *kn, *vn, *rec, *h1, *ypart;
  int32_t nwg, ns;        // workgroups, attention splits per kv head
  int32_t first[FP_COUNT];
};

// Plan of a single-launch layer: false if the layer does not fit (then the
// multi-launch path runs).  Host code.
bool plan_fused_layer(int H, int Hq, int Hkv, int D, int I, int64_t max_tiles, int nwg, FusedArgs* a);
// Words of the exchange arrays.
inline size_t fused_ll_pairs(int H, int Hq, int Hkv, int D, int I, int ns) {
  (void)I;
  return (size_t)Hq * D + 2 * (size_t)Hkv * D + (size_t)Hkv * ns * fused_rec_len(Hq / Hkv, D) +
         (size_t)kFusedCopies * H + (size_t)H * kFusedMaxWgs;
}
inline int fused_splits(int64_t max_tiles) { return (int)((max_tiles + kFusedAttnTiles - 1) / kFusedAttnTiles); }
hipError_t launch_fused_layer(const FusedArgs& a, hipStream_t st);
// Compute units of the current device if one fused workgroup fits on each, else -1.
int fused_device_wgs();

struct WsLayout {
  size_t err, q, o_p, h1, h1_p, act_p, x, x_p;
  size_t attn_part, amax_part, gemm_part;
  size_t fused_ll, fused_epoch;  // single-launch layer (batch 1): exchange words, epochs
  size_t total;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Workspace layout.  layer == false: attention only (no activations).
// max_tiles: the block table's width in 16-token tiles.
inline WsLayout ws_layout(int B, int H, int Hq, int Hkv, int I, int V, int64_t max_tiles, bool layer,
                          int D = kHeadDim) {
  WsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align256(off + bytes); return at; };
  w.err = take(kWsHeaderBytes);
  w.attn_part = take(sizeof(float) * (size_t)B * Hkv * attn_max_splits(max_tiles) * attn_rec(D));
  if (layer) {
    w.q = take(sizeof(float) * (size_t)B * Hq * D);  // BF16 hi + lo per value
    w.o_p = take(sizeof(float) * (size_t)packed_act_elems(B, Hq * D));
    w.h1 = take(sizeof(float) * (size_t)B * H);
    w.h1_p = take(sizeof(float) * (size_t)packed_act_elems(B, H));
    w.act_p = take(sizeof(float) * (size_t)packed_act_elems(B, I));
    w.x = take(sizeof(float) * (size_t)B * H);
    w.x_p = take(sizeof(float) * (size_t)packed_act_elems(B, H));
    const int Bc = B < kGemmMaxCols ? B : kGemmMaxCols;
    const GemmPlan lm = plan_gemm(EPI_LOGITS, V, Bc, H);
    w.amax_part = take(sizeof(unsigned long long) * (size_t)lm.tiles * (Bc > 0 ? Bc : 1));
    const size_t po = gemm_part_floats(H, Bc, Hq * D);
    const size_t pd = gemm_part_floats(H, Bc, I);
    w.gemm_part = take(sizeof(float) * (po > pd ? po : pd));
    if (B == 1) {
      w.fused_ll = take(8 * fused_ll_pairs(H, Hq, Hkv, D, I, fused_splits(max_tiles)));
      w.fused_epoch = kWsFusedEpochs;
    }
  }
  w.total = off;
  return w;
}

// ---------------------------------------------------------- launchers ---

// Each returns hipSuccess or the launch error.
// The split kernel, then the merge of sequences that took several splits.
// q formats of the attention kernel
constexpr int kQBf16 = 0;   // BF16 q, the matrix operand as it is
constexpr int kQSplit = 1;  // an FP32 q stored as BF16 hi and lo halves
hipError_t launch_attention(const AttnArgs& a, int batch, int qmode, hipStream_t st);
// Bytes of split records an attention call with these arguments writes
// (0 when every sequence fits one split).
inline size_t attention_record_bytes(const AttnArgs& a, int batch) {
  return a.max_splits > 1 ? sizeof(float) * (size_t)batch * a.Hkv * a.max_splits * attn_rec(a.D) : 0;
}
hipError_t launch_gemm(int epi, const GemmArgs& a, const GemmPlan& p, hipStream_t st);
hipError_t launch_kv_append(const PoolView& pv, const int32_t* bt, int32_t bt_stride,
                            const int32_t* pos, const uint16_t* k, const uint16_t* v, int batch,
                            int Hkv, int D, uint32_t* err, hipStream_t st);
hipError_t launch_embed(const uint16_t* E_packed, int V, int H, const int32_t* tok, float* x,
                        float* x_packed, int batch, uint32_t* err, hipStream_t st);
hipError_t launch_pack_weight(const uint16_t* src, int rows, int cols, int kind, uint16_t* dst,
                              hipStream_t st);
hipError_t launch_rope_table(double theta, int D, int max_pos, float* c, float* s,
                             hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
// prefill: RMSNorm (xw, or none if null) of plain FP32 rows into packed
// BF16 hi/lo pairs
hipError_t launch_prefill_norm(const float* x, const uint16_t* xw, int K, int T, float eps,
                               uint16_t* out, hipStream_t st);
hipError_t launch_prefill_gemm(int epi, const PgemmArgs& a, const PgemmPlan& p, hipStream_t st);
// argmax over the per-tile keys of EPI_LOGITS (either GEMM): one token per column
hipError_t launch_argmax_finalize(const unsigned long long* part, int tiles, int B, int32_t* next_tok,
                                  hipStream_t st);
// x[t] += sum over splits of part[s][t] (in split order); then, if nw is
// given, the RMSNorm of the new row into packed hi/lo pairs xb
// Split QKV: add the K splits' partial sums, then RoPE, q halves, K/V append.
hipError_t launch_qkv_finish(const float* part, int ks, const PgemmArgs& a, hipStream_t st);
hipError_t launch_prefill_resid(float* x, const float* part, int ks, int T, int N,
                                const uint16_t* nw, float eps, uint16_t* xb, hipStream_t st);
hipError_t launch_prefill_attention(const PattnArgs& a, hipStream_t st);

// Measurement kernels (probe.hip): a streaming read of `bytes`, the K/V
// loads of one attention call without its arithmetic, and empty launches.
hipError_t launch_probe_read(const void* buf, int64_t bytes, int workgroups, float* sink, hipStream_t st);
hipError_t launch_probe_paged_read(const AttnArgs& a, int batch, float* sink, hipStream_t st);
hipError_t launch_probe_empty(int launches, int workgroups, hipStream_t st);

// Host: validation of a paged_gqa_decode call's arguments other than its
// scratch, and its kernel arguments except `part` and `err`.  Returns 0 or a
// negative errno (the entry point's contract); batch 0 returns 0 with *args
// untouched.
int prepare_attention_call(const pkv_pool* pool, const uint16_t* q, int32_t num_q_heads,
                           const int32_t* block_table, int32_t max_pages, const int32_t* context_lens,
                           int32_t batch, float scale, float* out, AttnArgs* args);

}  // namespace pkv
