// Weight-streaming skinny GEMM for the decode projections, gfx950.
//
//   y[b][n] = sum_k W[n][k] * x[b][k] * xw[k]        (xw: RMSNorm weight or 1)
//
// W is BF16 [N][K] (the Hugging Face [out][in] orientation, packed into
// 16-row x 32-column blocks at load time) and is read from HBM exactly once
// per launch; the batch of FP32 activations is tiny and is read from L2.  This is the decode step's dense contraction (the engine
// packs one token of every active sequence into each step), so it runs on
// the matrix cores: v_mfma_f32_16x16x32_bf16 with W rows as the A operand
// (each lane streams 16-byte pieces of one row) and the batch as the B
// operand.  The FP32 activations are split into two BF16 halves x = hi + lo
// and both are multiplied (two MFMAs per weight tile), which keeps about 16
// significant bits of every activation while the weights, the only large
// operand, stay BF16.  Accumulation is FP32.
//
// A workgroup owns RG groups of 16 output rows over the whole of K; its NW
// waves split K (interleaved steps), run a two-stage software pipeline (the loads of the next
// U steps are in flight while the current ones multiply), and are summed
// in LDS in wave order.  No workgroup ever waits on another, so the
// result is deterministic and needs no cross-workgroup synchronisation.
// The same workgroup accumulates the sum of squares of its activations, so
// the RMSNorm row scale 1/sqrt(mean x^2 + eps) is applied in the epilogue.
//
// Fused epilogues:
//   EPI_QKV     16 rows = 8 RoPE pairs (j, j+D/2) of one head: RoPE on q and
//               k heads (angle from the FP32 cos/sin tables at the
//               sequence's position); q -> BF16 hi + lo halves (the
//               attention's matrix operand, ~16 bits), k and v -> BF16
//               (nearest even) into the sequence's page at its position
//               (the KV append).
//   EPI_RESID   out = resid + y (output projection, down projection), also
//               written packed for the next projection.
//   EPI_SWIGLU  each 16-row group = 8 gate rows + the 8 matching up rows:
//               a = silu(gate) * up, written packed for the down projection.
//   EPI_LOGITS  FP32 logits (optional store) and, per tile and sequence,
//               the largest logit packed with its index; a small kernel
//               then reduces the tiles to the token ids.
#include "pkv_dev.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Raw buffer descriptor over `bytes` bytes at p (gfx9 dword 3: 32-bit data).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// A byte offset past every activation descriptor: they cover at most 64
// batch columns of at most 65536 FP32 values, 16 MiB.
constexpr int kOutOfRange = 0x40000000;

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

// The same load with the non-temporal cache policy (gfx950 cache-policy
// bit 1, `nt`): for the weights, which each launch reads exactly once.
// With both the weights and the attention's K/V streamed this way the
// batch-16 step runs 1.3 % faster and a batch-1 layer 5 % faster than with
// ordinary loads; the weights alone gain nothing.
constexpr int kCpolNt = 2;
__device__ __forceinline__ u32x4 bload_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kCpolNt);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return (uint32_t)to_bf16_bits(a) | ((uint32_t)to_bf16_bits(b) << 16);
}

// Order-preserving map of an FP32 value to 32 bits, paired with the
// inverted index so that the 64-bit maximum is the largest value and, among
// equal values, the lowest index.
__device__ __forceinline__ unsigned long long argmax_key(float v, int n) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xffffffffu - (uint32_t)n);
}

template <int CT, int RG, int NW, int EPI, bool XPLAIN>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(const GemmArgs a) {
  constexpr bool NORM = EPI != EPI_RESID;
  constexpr int U = 2;        // 32-wide K steps per pipeline stage
  constexpr int R = 16 * RG;  // output rows per tile
  constexpr int NC = 16 * CT; // batch columns per launch
  constexpr int TS = R + 1;   // tile column stride (floats)

  __shared__ f32x4 red[NW][CT][RG][64];
  __shared__ float tile[NC * TS];
  __shared__ float ssq_w[NW][NC];
  __shared__ float ssq_col[NC];

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  // workgroup = (row tile t, K split ks); the split's 32-wide K steps are
  // shared out over the waves
  const int nks = EPI == EPI_RESID ? a.ksplit : 1;
  const int t = blockIdx.x / nks;
  const int ksi = blockIdx.x - t * nks;
  const int steps = a.K >> 5;
  const int sps = (steps + nks - 1) / nks;
  const int ks0 = ksi * sps;
  const int ks1 = min(ks0 + sps, steps);
  const int spw = (ks1 - ks0 + NW - 1) / NW;
  const int s0 = ks0 + w * spw;
  const int s1 = s0 + max(0, min(spw, (ks1 - ks0 - w + NW - 1) / NW));

  // Buffer loads: one descriptor per operand in scalar registers, a fixed
  // per-lane byte offset in a vector register, and the step's offset as a
  // scalar, so the loop carries no vector address arithmetic (which would
  // otherwise make the prefetch wait on its own registers).  W is packed:
  // a 16-row group's step is one contiguous 1 KiB block in lane order.  X is
  // packed (a lane's 8 values of a step are 32 contiguous bytes) except for
  // a caller's plain [B][K] input.  Every instruction thus reads contiguous
  // memory: spreading one instruction over 16 rows of a large matrix costs
  // one address translation per row and serialises the L1 TLB.
  // Groups past the matrix read its last group; columns past B read zeros
  // or column 0; neither is ever stored.
  const int koff = 8 * (l >> 4);
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(a.W, (uint32_t)a.w_groups * (uint32_t)a.K * 32u);
  const __amdgpu_buffer_rsrc_t xres =
      make_rsrc(a.X, (uint32_t)(XPLAIN ? a.B : (a.B + 15) / 16 * 16) * (uint32_t)a.K * 4u);
  const __amdgpu_buffer_rsrc_t xwres = make_rsrc(NORM ? a.xw : a.W, (uint32_t)a.K * 2u);
  int woff[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) woff[g] = (min(t * RG + g, a.w_groups - 1) * steps * 64 + l) * 16;
  // Lanes of batch columns past B get an offset beyond the descriptor's
  // range: buffer loads there return zeros without a memory request, so a
  // small batch reads only its own activations.
  int xoff[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int b = 16 * c + (l & 15);
    if (b >= a.B)
      xoff[c] = kOutOfRange;
    else if (XPLAIN)
      xoff[c] = (b * a.K + koff) * 4;
    else
      xoff[c] = (c * steps * 64 + l) * 32;
  }
  const int xwoff = koff * 2;

  f32x4 acc[RG][CT];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[g][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float ssq[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) ssq[c] = 0.f;

  struct Stage {
    u32x4 w[U][RG];
    float4 x[U][CT][2];
    uint4 xw[U];
  };
  // Loads of steps st .. st+U-1, clamped into this wave's K range (steps
  // past the end are loaded again and skipped by compute): no branch, so
  // the compiler's wait counts stay exact and the prefetch is never waited
  // on early.
  // The waves interleave their steps (wave w's j-th step is ks0 + j NW + w),
  // so a workgroup streams each row group as one contiguous run rather than
  // NW separate ones (measured faster: fewer concurrent DRAM streams).
  auto load = [&](Stage& S, int st) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = min(st + u, s1 - 1) - s0;
      const int k = min(ks0 + jj * NW + w, ks1 - 1) * 32;
#pragma unroll
      for (int g = 0; g < RG; ++g) S.w[u][g] = bload_nt(wres, woff[g], k * 32);
      const int xs = XPLAIN ? k * 4 : k * 64;
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        S.x[u][c][0] = __builtin_bit_cast(float4, bload(xres, xoff[c], xs));
        S.x[u][c][1] = __builtin_bit_cast(float4, bload(xres, xoff[c] + 16, xs));
      }
      if (NORM) S.xw[u] = __builtin_bit_cast(uint4, bload(xwres, xwoff, k * 2));
    }
  };
  auto compute = [&](const Stage& S, int st) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (st + u >= s1) break;
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        float v[8] = {S.x[u][c][0].x, S.x[u][c][0].y, S.x[u][c][0].z, S.x[u][c][0].w,
                      S.x[u][c][1].x, S.x[u][c][1].y, S.x[u][c][1].z, S.x[u][c][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) ssq[c] += v[e] * v[e];
        if (NORM) {
          v[0] *= bf16_lo(S.xw[u].x); v[1] *= bf16_hi(S.xw[u].x);
          v[2] *= bf16_lo(S.xw[u].y); v[3] *= bf16_hi(S.xw[u].y);
          v[4] *= bf16_lo(S.xw[u].z); v[5] *= bf16_hi(S.xw[u].z);
          v[6] *= bf16_lo(S.xw[u].w); v[7] *= bf16_hi(S.xw[u].w);
        }
        float hi[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          hi[e] = (float)(__bf16)v[e];
          lo[e] = v[e] - hi[e];
        }
        const u32x4 bh = {pack_bf16(hi[0], hi[1]), pack_bf16(hi[2], hi[3]),
                          pack_bf16(hi[4], hi[5]), pack_bf16(hi[6], hi[7])};
        const u32x4 bl = {pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]),
                          pack_bf16(lo[4], lo[5]), pack_bf16(lo[6], lo[7])};
#pragma unroll
        for (int g = 0; g < RG; ++g) {
          acc[g][c] = mfma32(S.w[u][g], bh, acc[g][c]);
          acc[g][c] = mfma32(S.w[u][g], bl, acc[g][c]);
        }
      }
    }
  };

  // Epilogue inputs whose addresses do not depend on the products (the
  // sequence's position, then its RoPE row and the page that takes the
  // appended slot; the residual) are loaded around the first weight stage,
  // so their round trips overlap the weight stream instead of following it.
  // This thread's first epilogue item is idx = tid.  Indices are clamped
  // here and validated where the values are used.
  constexpr int NT = NW * 64;
  int pf_p = 0, pf_page = 0;
  float pf_r = 0.f, pf_cs = 1.f, pf_sn = 0.f;
  int hd = 0, j0 = 0;
  bool is_q = false, is_k = false;
  if constexpr (EPI == EPI_QKV) {
    const int gph = a.D / 16;  // 16-row groups per head
    hd = t / gph;
    j0 = 8 * (t % gph);
    is_q = hd < a.Hq;
    is_k = !is_q && hd < a.Hq + a.Hkv;
    if (tid < 8 * a.B) pf_p = a.pos[tid >> 3];
  }
  if constexpr (EPI == EPI_RESID) {
    if (nks == 1 && tid < R * a.B) {
      const int n = t * R + tid % R;
      if (n < a.N) pf_r = a.resid[(size_t)(tid / R) * a.N + n];
    }
  }
  auto prefetch2 = [&]() {
    if constexpr (EPI == EPI_QKV) {
      if (tid < 8 * a.B) {
        const int j = j0 + (tid & 7), half = a.D / 2;
        const int pc = max(pf_p, 0);
        if ((is_q || is_k) && a.max_pos > 0) {
          const size_t r = (size_t)min(pc, a.max_pos - 1) * half + j;
          pf_cs = a.rcos[r];
          pf_sn = a.rsin[r];
        }
        if (!is_q && a.bt_stride > 0)
          pf_page = a.bt[(size_t)(tid >> 3) * a.bt_row + min(pc >> (4 + a.pv.pt_shift), a.bt_stride - 1)];
      }
    }
  };

  if (s0 >= s1) prefetch2();
  if (s0 < s1) {
    Stage A, B;
    load(A, s0);
    prefetch2();
    for (int st = s0;; st += 2 * U) {
      load(B, st + U);
      compute(A, st);
      if (st + U >= s1) break;
      load(A, st + 2 * U);
      compute(B, st + U);
      if (st + 2 * U >= s1) break;
    }
  }

  // ---- sum the waves (in wave order) into tile[col * TS + row]
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    ssq[c] = rows_sum4(ssq[c]);
    if (l < 16) ssq_w[w][16 * c + l] = ssq[c];
#pragma unroll
    for (int g = 0; g < RG; ++g) red[w][c][g][l] = acc[g][c];
  }
  __syncthreads();
  for (int i = tid; i < CT * RG * 64 * 4; i += NW * 64) {
    const int r = i & 3, ln = (i >> 2) & 63, g = (i >> 8) % RG, c = (i >> 8) / RG;
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += red[ww][c][g][ln][r];
    const int row = 16 * g + 4 * (ln >> 4) + r;
    const int col = 16 * c + (ln & 15);
    tile[col * TS + row] = v;
  }
  if (tid < NC) {
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) v += ssq_w[ww][tid];
    ssq_col[tid] = v;
  }
  __syncthreads();

  // ---- epilogues
  if (EPI == EPI_RESID) {
    for (int i = tid; i < R * a.B; i += NT) {
      const int c = i / R, row = i % R;
      const int n = t * R + row;
      if (n < a.N) {
        const size_t o = (size_t)c * a.N + n;
        if (nks > 1) {
          a.part[(size_t)ksi * a.B * a.N + o] = tile[c * TS + row];
        } else {
          const float v = (i == tid ? pf_r : a.resid[o]) + tile[c * TS + row];
          a.out[o] = v;
          if (a.out_packed) a.out_packed[packed_act_index(c, n, a.N)] = v;
        }
      }
    }
  } else if (EPI == EPI_QKV) {
    // head width D: a 16-row group holds 8 RoPE pairs (j, j + D/2) of one head
    const int D = a.D, half = D / 2;
    for (int idx = tid; idx < 8 * a.B; idx += NT) {
      const int c = idx >> 3, i = idx & 7, j = j0 + i;
      const bool first = idx == tid;
      const float rs = 1.0f / sqrtf(ssq_col[c] / (float)a.K + a.eps);
      const float x0 = tile[c * TS + i] * rs;
      const float x1 = tile[c * TS + 8 + i] * rs;
      const int p = first ? pf_p : a.pos[c];
      float y0 = x0, y1 = x1;
      if (is_q || is_k) {
        if (p < 0 || p >= a.max_pos) {
          set_error(a.err, ERR_ROPE);
          continue;
        }
        const float cs = first ? pf_cs : a.rcos[(size_t)p * half + j];
        const float sn = first ? pf_sn : a.rsin[(size_t)p * half + j];
        y0 = __fsub_rn(__fmul_rn(x0, cs), __fmul_rn(x1, sn));
        y1 = __fadd_rn(__fmul_rn(x0, sn), __fmul_rn(x1, cs));
      }
      if (is_q) {
        // q leaves as the attention's matrix operand: BF16 hi and lo halves
        uint16_t* qo = a.q_split + ((size_t)c * a.Hq + hd) * 2 * D;
        const uint16_t h0 = to_bf16_bits(y0), h1 = to_bf16_bits(y1);
        qo[j] = h0;
        qo[j + half] = h1;
        qo[D + j] = to_bf16_bits(y0 - bf16_lo(h0));
        qo[D + j + half] = to_bf16_bits(y1 - bf16_lo(h1));
      } else {
        const int psh = 4 + a.pv.pt_shift, PT = 1 << psh;  // page tokens
        if (p < 0 || (p >> psh) >= a.bt_stride) {
          set_error(a.err, ERR_LENGTH);
          continue;
        }
        const int page = first ? pf_page : a.bt[(size_t)c * a.bt_row + (p >> psh)];
        if ((unsigned)page >= (unsigned)a.pv.num_pages) {
          set_error(a.err, ERR_PAGE);
          continue;
        }
        const int slot = p & (PT - 1);
        if (is_k) {
          a.pv.k[pv_k_elem(a.pv, page, hd - a.Hq, slot, j, D)] = to_bf16_bits(y0);
          a.pv.k[pv_k_elem(a.pv, page, hd - a.Hq, slot, j + half, D)] = to_bf16_bits(y1);
        } else {
          uint16_t* vp = a.pv.v + pv_v_index(a.pv, page, hd - a.Hq - a.Hkv, 0, slot, D);
          vp[j * kTile] = to_bf16_bits(y0);
          vp[(j + half) * kTile] = to_bf16_bits(y1);
        }
      }
    }
  } else if (EPI == EPI_SWIGLU) {
    for (int idx = tid; idx < 8 * RG * a.B; idx += NT) {
      const int c = idx / (8 * RG), gi = idx % (8 * RG), g = gi >> 3, m = gi & 7;
      const int i = 8 * (t * RG + g) + m;
      if (i >= a.I) continue;
      const float rs = 1.0f / sqrtf(ssq_col[c] / (float)a.K + a.eps);
      const float gv = tile[c * TS + 16 * g + m] * rs;
      const float uv = tile[c * TS + 16 * g + 8 + m] * rs;
      a.act[packed_act_index(c, i, a.I)] = gv / (1.0f + expf(-gv)) * uv;
    }
  } else {  // EPI_LOGITS
    for (int i = tid; i < R * a.B; i += NT) {
      const int c = i / R, row = i % R;
      const int n = t * R + row;
      if (n < a.N && a.logits) {
        const float rs = 1.0f / sqrtf(ssq_col[c] / (float)a.K + a.eps);
        a.logits[(size_t)c * a.N + n] = tile[c * TS + row] * rs;
      }
    }
    if (tid < a.B) {
      const int c = tid;
      const float rs = 1.0f / sqrtf(ssq_col[c] / (float)a.K + a.eps);
      unsigned long long best = 0ull;
      for (int row = 0; row < R; ++row) {
        const int n = t * R + row;
        if (n >= a.N) break;
        const unsigned long long key = argmax_key(tile[c * TS + row] * rs, n);
        best = key > best ? key : best;
      }
      a.amax_part[(size_t)t * a.B + c] = best;
    }
  }
}

// out = resid + the K splits' partial sums, added in split order (so the
// result does not depend on which workgroup finished first), plain and
// packed.  One thread per 4 consecutive outputs of one batch column; the
// partials of 16 splits are loaded together (split index clamped, masked).
__global__ __launch_bounds__(64) void resid_reduce_kernel(const float* part, int nks, int B, int N,
                                                           const float* resid, float* out,
                                                           float* out_packed) {
  constexpr int CH = 16;
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int n4 = N >> 2;
  if (i >= B * n4) return;
  const int c = i / n4, n = (i - c * n4) * 4;
  const size_t o = (size_t)c * N + n;
  const size_t stride = (size_t)B * N;
  float4 v = *(const float4*)(resid + o);
  for (int s0 = 0; s0 < nks; s0 += CH) {
    float4 p[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) p[j] = *(const float4*)(part + (size_t)min(s0 + j, nks - 1) * stride + o);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (s0 + j < nks) {
        v.x += p[j].x;
        v.y += p[j].y;
        v.z += p[j].z;
        v.w += p[j].w;
      }
    }
  }
  *(float4*)(out + o) = v;
  if (out_packed) *(float4*)(out_packed + packed_act_index(c, n, N)) = v;
}

// Token id per sequence: the largest packed key over the LM head's tiles.
__global__ void argmax_finalize_kernel(const unsigned long long* part, int tiles, int B,
                                       int32_t* next_tok) {
  __shared__ unsigned long long sm[256];
  constexpr int U = 16;  // keys loaded together per thread
  const int c = blockIdx.x;
  unsigned long long best = 0ull;
  for (int t0 = threadIdx.x; t0 < tiles; t0 += blockDim.x * U) {
    unsigned long long k[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * blockDim.x;
      k[u] = part[(size_t)min(t, tiles - 1) * B + c];  // clamped: loads issue unconditionally
    }
#pragma unroll
    for (int u = 0; u < U; ++u) best = k[u] > best ? k[u] : best;  // a repeated key changes nothing
  }
  sm[threadIdx.x] = best;
  __syncthreads();
  for (int s = blockDim.x / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s && sm[threadIdx.x + s] > sm[threadIdx.x]) sm[threadIdx.x] = sm[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) next_tok[c] = (int32_t)(0xffffffffu - (uint32_t)(sm[0] & 0xffffffffull));
}

template <int CT, int RG, int NW, int EPI, bool XPLAIN = false>
hipError_t go(const GemmArgs& a, int tiles, hipStream_t st) {
  gemm_kernel<CT, RG, NW, EPI, XPLAIN><<<tiles, NW * 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(int epi, const GemmArgs& a, const GemmPlan& p, hipStream_t st) {
  hipError_t e = hipErrorInvalidValue;
  const int ct = p.ct;
  switch (epi) {
    case EPI_QKV:
      if (a.x_plain)
        e = ct == 1 ? (p.nw == 4 ? go<1, 1, 4, EPI_QKV, true>(a, p.tiles, st)
                                 : go<1, 1, 8, EPI_QKV, true>(a, p.tiles, st))
            : ct == 2 ? go<2, 1, 8, EPI_QKV, true>(a, p.tiles, st)
                      : go<4, 1, 8, EPI_QKV, true>(a, p.tiles, st);
      else
        e = ct == 1 ? (p.nw == 4 ? go<1, 1, 4, EPI_QKV>(a, p.tiles, st) : go<1, 1, 8, EPI_QKV>(a, p.tiles, st))
            : ct == 2 ? go<2, 1, 8, EPI_QKV>(a, p.tiles, st)
                      : go<4, 1, 8, EPI_QKV>(a, p.tiles, st);
      break;
    case EPI_RESID:
      if (p.ks > 1) {
        e = ct == 1 ? go<1, 2, 4, EPI_RESID>(a, p.tiles * p.ks, st)
            : ct == 2 ? go<2, 2, 4, EPI_RESID>(a, p.tiles * p.ks, st)
                      : go<4, 1, 4, EPI_RESID>(a, p.tiles * p.ks, st);
        if (e != hipSuccess) return e;
        // small blocks: the partial sums are a few MB, spread over enough
        // workgroups that no CU streams more than a few KB of them
        const int n = a.B * (a.N / 4);
        resid_reduce_kernel<<<(n + 63) / 64, 64, 0, st>>>(a.part, p.ks, a.B, a.N, a.resid, a.out,
                                                          a.out_packed);
        e = hipGetLastError();
      } else {
        e = ct == 1 ? (p.nw == 4 ? go<1, 1, 4, EPI_RESID>(a, p.tiles, st) : go<1, 1, 8, EPI_RESID>(a, p.tiles, st))
            : ct == 2 ? go<2, 1, 8, EPI_RESID>(a, p.tiles, st)
                      : go<4, 1, 8, EPI_RESID>(a, p.tiles, st);
      }
      break;
    case EPI_SWIGLU:
      e = ct == 1 ? go<1, 2, 4, EPI_SWIGLU>(a, p.tiles, st)
          : ct == 2 ? go<2, 1, 4, EPI_SWIGLU>(a, p.tiles, st)
                    : go<4, 1, 4, EPI_SWIGLU>(a, p.tiles, st);
      break;
    case EPI_LOGITS:
      if (a.x_plain)  // one plain activation row (the last prompt token)
        e = ct == 1 && p.rg == 2 ? go<1, 2, 4, EPI_LOGITS, true>(a, p.tiles, st) : hipErrorInvalidValue;
      else
        e = ct == 1 ? (p.rg == 4 ? go<1, 4, 4, EPI_LOGITS>(a, p.tiles, st) : go<1, 2, 4, EPI_LOGITS>(a, p.tiles, st))
            : ct == 2 ? go<2, 1, 4, EPI_LOGITS>(a, p.tiles, st)
                      : go<4, 1, 4, EPI_LOGITS>(a, p.tiles, st);
      if (e != hipSuccess) return e;
      argmax_finalize_kernel<<<a.B, 256, 0, st>>>(a.amax_part, p.tiles, a.B, a.next_tok);
      e = hipGetLastError();
      break;
    default:
      break;
  }
  return e;
}

hipError_t launch_argmax_finalize(const unsigned long long* part, int tiles, int B, int32_t* next_tok,
                                  hipStream_t st) {
  argmax_finalize_kernel<<<B, 256, 0, st>>>(part, tiles, B, next_tok);
  return hipGetLastError();
}

}  // namespace pkv
