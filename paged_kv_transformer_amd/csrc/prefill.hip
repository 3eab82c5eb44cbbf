// Dense causal prefill of one sequence's prompt, gfx950.
//
// Prefill pushes all T prompt tokens of a sequence through each layer
// together ("Inference from Scratch": prefill is the step before decode and
// fills the prompt's pages).  Its projections are real matrix products,
// T tokens by N rows by K, so they run as tiled matrix-core GEMMs that
// reuse every weight block across a tile of tokens, rather than as the
// decode step's weight-streaming kernel.  Activations entering a projection
// are FP32 values carried as two BF16 halves (hi + lo, ~16 significant bits:
// with plain BF16 activations the error compounds over the layers of a
// 16-layer model to several percent of the logits' RMS), produced packed in
// the same 1 KiB block order as the weights, so a workgroup moves both
// operands as whole blocks and every matrix-core operand is one 16-byte read
// per lane.
//
//   prefill_norm_kernel       RMSNorm of FP32 rows -> packed BF16 hi/lo
//   prefill_gemm_kernel       256 x 128 (or smaller) output tiles; epilogues
//                             as the decode projections: RoPE + q split +
//                             K/V page writes, SwiGLU, or (residual
//                             projections) K-split partial sums
//   prefill_resid_kernel      residual + partial sums, then the next RMSNorm
//   prefill_attention_kernel  causal paged attention: a workgroup takes up to
//                             16 (token, head) query columns of one kv head;
//                             its waves split the pages 0 .. the last position
#include "pkv_dev.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)to_bf16_bits(a) | ((uint32_t)to_bf16_bits(b) << 16);
}

// Order-preserving map of an FP32 logit to 32 bits, paired with the inverted
// index: the 64-bit maximum is the largest logit and, among equal ones, the
// lowest index.
__device__ __forceinline__ unsigned long long logit_key(float v, int n) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xffffffffu - (uint32_t)n);
}

// ------------------------------------------------------------- norm ---
// Eight FP32 values as BF16 hi halves and the BF16 rounding of what remains.
__device__ __forceinline__ void split8(const float* v, uint4& hi, uint4& lo) {
  uint16_t h[8];
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = to_bf16_bits(v[e]);
    r[e] = v[e] - bf16_lo(h[e]);
  }
  hi = make_uint4((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16),
                  (uint32_t)h[4] | ((uint32_t)h[5] << 16), (uint32_t)h[6] | ((uint32_t)h[7] << 16));
  lo = make_uint4(pack2(r[0], r[1]), pack2(r[2], r[3]), pack2(r[4], r[5]), pack2(r[6], r[7]));
}

// One workgroup per (padded) token row: out = x * rs * xw as hi/lo pairs,
// rs = 1 / sqrt(mean x^2 + eps); padding rows are zeros.
__global__ __launch_bounds__(256) void prefill_norm_kernel(const float* x, const uint16_t* xw,
                                                           int K, int T, float eps, uint16_t* out) {
  __shared__ float part[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (t >= T) {
    for (int k = 8 * tid; k < K; k += 8 * 256) {
      *(uint4*)(out + packed_pair_index(t, k, K, 0)) = make_uint4(0u, 0u, 0u, 0u);
      *(uint4*)(out + packed_pair_index(t, k, K, 1)) = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }
  const float* row = x + (size_t)t * K;
  float ss = 0.f;
  for (int k = 8 * tid; k < K; k += 8 * 256) {
    const float4 a = *(const float4*)(row + k), b = *(const float4*)(row + k + 4);
    ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z +
          b.w * b.w;
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  const float rs = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)K + eps);
  for (int k = 8 * tid; k < K; k += 8 * 256) {
    const float4 a = *(const float4*)(row + k), b = *(const float4*)(row + k + 4);
    float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    if (xw) {
      const uint4 w = *(const uint4*)(xw + k);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] *= bf16_lo(ww[e]);
        v[2 * e + 1] *= bf16_hi(ww[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= rs;
    uint4 hi, lo;
    split8(v, hi, lo);
    *(uint4*)(out + packed_pair_index(t, k, K, 0)) = hi;
    *(uint4*)(out + packed_pair_index(t, k, K, 1)) = lo;
  }
}

// ------------------------------------------------------------- GEMM ---
// One global -> LDS copy of a 1 KiB block by a wave (buffer_load_dwordx4 ...
// lds: lane l's 16 bytes land at LDS byte address lds + 16 l, the block's
// own order).  M0 carries the wave's LDS address; the statement sets it
// itself (nothing else in these kernels uses M0).  The load is counted by
// vmcnt like any
// buffer load and is waited for explicitly (wait_stages): the compiler does
// not see it, so it adds no conservative wait of its own before LDS reads.
// An offset past the descriptor's range reads zeros.
__device__ __forceinline__ void lds_copy16(uint32_t lds, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory");
}
// The same copy with the non-temporal cache policy, for weight blocks:
// each is read by the token tiles of one row tile, which run together on
// one XCD, and never again in the launch (prompt 3.5 % faster, batch-64
// decode step 2 %).
__device__ __forceinline__ void lds_copy16_nt(uint32_t lds, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory");
}

// Raw buffer descriptor words over `bytes` bytes at p (32-bit data format).
__device__ __forceinline__ i32x4 rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  return (i32x4){(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `pend` stages of LPW copies each are still in flight.
template <int LPW, int K>
__device__ __forceinline__ void wait_stages(int pend) {
  if constexpr (K == 0) {
    wait_vm<0>();
  } else {
    if (pend >= K)
      wait_vm<K * LPW>();
    else
      wait_stages<LPW, K - 1>(pend);
  }
}

// y[t][n] = sum_k W[n][k] X[t][k].  A workgroup of 4 waves (2 x 2) owns
// 32 RG rows by 32 CG tokens; each wave a 16 RG x 16 CG sub-tile held as
// RG x CG accumulator tiles of v_mfma_f32_16x16x32_bf16 (W block as the A
// operand, the X hi and lo blocks as two B operands).  A stage is one
// 32-wide K step: 2 RG W blocks and 2 CG (hi, lo) X block pairs, copied
// straight from global memory into a ring of NSTG stages in LDS, so that
// NSTG - 1 stages of loads are in flight while a stage is multiplied (the
// latency of a load under load is far longer than one stage's products).
// Workgroups are mapped to tiles XCD by XCD, so the token tiles of one row
// tile run on one XCD and share its L2 copy of the weights.  Out-of-range
// row and token groups read zeros and are never stored.
// WR wave rows by 2 wave columns: each wave owns RG row groups (16 RG
// rows) by CG token groups.  The tall tiles run with WR = 4 (8 waves, two
// per SIMD, so one wave's LDS operand reads overlap the other's products);
// the small ones and the LM head with WR = 2.
template <int RG, int CG, int WR>
struct PgemmShape {
  static constexpr int NW = 2 * WR;        // waves
  static constexpr int AR = WR * RG;       // row groups per tile
  static constexpr int BC = 2 * CG;        // token groups per tile
  static constexpr int NA = AR;            // W blocks per stage
  static constexpr int NB = AR + 2 * BC;   // blocks per stage
  static constexpr int LPW = NB / NW;      // copies per wave per stage
  static constexpr int NSTG = NB * 6 <= 144 ? 6 : 144 / NB;  // ring of at most 144 KiB
};

template <int EPI, int RG, int CG, int WR>
__global__ __launch_bounds__(128 * WR) void prefill_gemm_kernel(const PgemmArgs a) {
  using SH = PgemmShape<RG, CG, WR>;
  constexpr int AR = SH::AR, BC = SH::BC, NA = SH::NA, NB = SH::NB, LPW = SH::LPW, NW = SH::NW;
  constexpr int NSTG = SH::NSTG;
  static_assert(NA % NW == 0 && NB % NW == 0, "stage blocks split evenly over the waves");
  static_assert((NSTG - 2) * LPW <= 63, "vmcnt range");
  static_assert(EPI != EPI_LOGITS || WR == 2, "the argmax keys assume two wave rows");
  __shared__ u32x4 ring[NSTG][NB][64];

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = w % WR, wc = w / WR;
  const int nrt = (a.w_groups + AR - 1) / AR;
  const int ntt = (a.T + 16 * BC - 1) / (16 * BC);
  const int nks = EPI == EPI_RESID ? a.ksplit : 1;
  const int nwork = nrt * nks * ntt;
  // workgroup id -> work item (row tile, K split, token tile), token tile
  // fastest: ids i, i + 8, i + 16 .. (one XCD) take consecutive items, so
  // the token tiles sharing one slice of weights run on one XCD
  const int id = blockIdx.x;
  const int per = nwork >> 3, rem = nwork & 7, xcd = id & 7, slot0 = id >> 3;
  const int item = xcd < rem ? xcd * (per + 1) + slot0 : rem * (per + 1) + (xcd - rem) * per + slot0;
  const int rt = item / (nks * ntt);
  const int ksi = (item / ntt) % nks, tt = item % ntt;
  const int S = a.K >> 5;
  const int sps = (S + nks - 1) / nks;
  const int s0 = ksi * sps, ns = min(S, s0 + sps) - s0;  // this split's K steps
  const int g0 = rt * AR, c0 = tt * BC;

  const i32x4 wres = rsrc_words(a.W, (uint32_t)a.w_groups * (uint32_t)S * 1024u);
  const i32x4 xres = rsrc_words(a.X, (uint32_t)((a.T + 15) / 16) * (uint32_t)S * 2048u);
  // wave w copies blocks j = NW i + w of each stage: W row group j for
  // i < NA / NW, then X block j - NA = 2 c + h (token group c, half h)
  uint32_t boff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int j = NW * i + w;
    if (i < NA / NW) {
      boff[i] = (uint32_t)(g0 + j) * S * 1024u + l * 16;
    } else {
      const int jb = j - NA;
      boff[i] = (uint32_t)(c0 + (jb >> 1)) * S * 2048u + (jb & 1) * 1024u + l * 16;
    }
  }
  const uint32_t ring0 = (uint32_t)(uintptr_t)&ring[0][0][0];
  // stage st (0 .. ns - 1) is K step s0 + st
  auto issue = [&](int st) {
    const uint32_t base = ring0 + (uint32_t)((st % NSTG) * NB) * 1024u;
    const uint32_t ks = (uint32_t)(s0 + st);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const bool isw = i < NA / NW;
      if (isw)
        lds_copy16_nt(base + (uint32_t)(NW * i + w) * 1024u, boff[i] + ks * 1024u, wres);
      else
        lds_copy16(base + (uint32_t)(NW * i + w) * 1024u, boff[i] + ks * 2048u, xres);
    }
  };

  f32x4 acc[RG][CG];
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int c = 0; c < CG; ++c) acc[r][c] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int st = 0; st < NSTG - 1 && st < ns; ++st) issue(st);
  for (int st = 0; st < ns; ++st) {
    // this wave's copies of stage st have landed, then everyone's; every
    // wave is also done with stage st - 1, whose slot is refilled next
    wait_stages<LPW, NSTG - 2>(min(NSTG - 2, ns - 1 - st));
    __syncthreads();
    if (st + NSTG - 1 < ns) issue(st + NSTG - 1);
    const int sl = st % NSTG;
    u32x4 af[RG], bh[CG], bl[CG];
#pragma unroll
    for (int r = 0; r < RG; ++r) af[r] = ring[sl][wr * RG + r][l];
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      bh[c] = ring[sl][NA + 2 * (wc * CG + c)][l];
      bl[c] = ring[sl][NA + 2 * (wc * CG + c) + 1][l];
    }
#pragma unroll
    for (int r = 0; r < RG; ++r)
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        acc[r][c] = mfma_k32(af[r], bh[c], acc[r][c]);
        acc[r][c] = mfma_k32(af[r], bl[c], acc[r][c]);
      }
  }

  // ---- epilogues: lane holds rows 16 G + 4 grp + e (e = 0..3) of token
  // 16 tg + col for each accumulator tile
  const int grp = l >> 4, col = l & 15;
  if (EPI == EPI_LOGITS) {
    // FP32 logits, and per token the largest logit of this wave's rows
    // packed with its index (the lower index wins ties); the two waves of a
    // token half write the two key slots of this row tile
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      const int t = 16 * (c0 + wc * CG + c) + col;
      unsigned long long best = 0ull;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const int G = g0 + wr * RG + r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = 16 * G + 4 * grp + e;
          if (n < a.N) {
            const float v = acc[r][c][e];
            if (a.logits && t < a.T) a.logits[(size_t)t * a.N + n] = v;
            const unsigned long long key = logit_key(v, n);
            best = key > best ? key : best;
          }
        }
      }
      unsigned long long o = __shfl_xor(best, 16);
      best = o > best ? o : best;
      o = __shfl_xor(best, 32);
      best = o > best ? o : best;
      if (grp == 0 && t < a.T) a.amax_part[(size_t)(2 * rt + wr) * a.T + t] = best;
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      const int G = g0 + wr * RG + r;
      const int t = 16 * (c0 + wc * CG + c) + col;
      const f32x4 v = acc[r][c];
      if (EPI == EPI_RESID) {
        if (G < a.w_groups && t < a.T) {
          const size_t o = ((size_t)ksi * a.T + t) * a.N + 16 * G + 4 * grp;
          *(float4*)(a.part + o) = make_float4(v[0], v[1], v[2], v[3]);
        }
      } else if (EPI == EPI_SWIGLU) {
        // rows 0..7 of a group are gate rows, 8..15 the matching up rows:
        // lane l holds gate rows, lane l + 32 the up rows of the same token
        f32x4 up;
#pragma unroll
        for (int e = 0; e < 4; ++e) up[e] = xor32_lane(v[e]);
        const int i0 = 8 * G + 4 * grp;
        if (l < 32 && t < a.T && i0 < a.I) {
          uint16_t h[4];
          float lo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float y = v[e] / (1.0f + expf(-v[e])) * up[e];
            h[e] = to_bf16_bits(y);
            lo[e] = y - bf16_lo(h[e]);
          }
          *(u32x2*)(a.act + packed_pair_index(t, i0, a.I, 0)) =
              (u32x2){(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
          *(u32x2*)(a.act + packed_pair_index(t, i0, a.I, 1)) =
              (u32x2){pack2(lo[0], lo[1]), pack2(lo[2], lo[3])};
        }
      } else if (EPI == EPI_QKV) {
        // group G: head G / (D/16), RoPE pairs j = 8 (G % (D/16)) + m, rows
        // j (lanes 0..31) and j + D/2 (lanes 32..63, the same j in lane l - 32)
        f32x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = xor32_lane(v[e]);
        const int D = a.D, half = D / 2, gph = D / 16;
        const int hd = G / gph;
        const int p = t < a.T ? (a.pos ? a.pos[t] : a.start_pos + t) : 0;
        const bool is_q = hd < a.Hq, is_k = !is_q && hd < a.Hq + a.Hkv;
        bool ok = hd < a.Hq + 2 * a.Hkv && t < a.T;
        if (ok && (is_q || is_k) && (p < 0 || p >= a.max_pos)) {
          set_error(a.err, ERR_ROPE);
          ok = false;
        }
        const int psh = 4 + a.pv.pt_shift, PT = 1 << psh;  // page tokens
        if (ok && !is_q && (p < 0 || (p >> psh) >= a.bt_stride)) {
          set_error(a.err, ERR_LENGTH);
          ok = false;
        }
        if (ok) {
          const bool first = l < 32;
          const int jb = 8 * (G % gph) + 4 * (grp & 1);
          const int jj = first ? jb : jb + half;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            y[e] = v[e];
            if (is_q || is_k) {
              const float x0 = first ? v[e] : pv[e], x1 = first ? pv[e] : v[e];
              const float cs = a.rcos[(size_t)p * half + jb + e];
              const float sn = a.rsin[(size_t)p * half + jb + e];
              y[e] = first ? __fsub_rn(__fmul_rn(x0, cs), __fmul_rn(x1, sn))
                           : __fadd_rn(__fmul_rn(x0, sn), __fmul_rn(x1, cs));
            }
          }
          if (is_q) {
            uint16_t* qo = a.q_split + ((size_t)t * a.Hq + hd) * 2 * D + jj;
            uint16_t h[4];
            float lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              h[e] = to_bf16_bits(y[e]);
              lo[e] = y[e] - bf16_lo(h[e]);
            }
            *(u32x2*)qo = (u32x2){(uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                  (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
            *(u32x2*)(qo + D) = (u32x2){pack2(lo[0], lo[1]), pack2(lo[2], lo[3])};
          } else {
            const int page = a.bt[(size_t)t * a.bt_row + (p >> psh)];
            if ((unsigned)page >= (unsigned)a.pv.num_pages) {
              set_error(a.err, ERR_PAGE);
            } else {
              const int slot = p & (PT - 1);
              if (is_k) {
                // jj is a multiple of 4: its 4 dims lie in one 8-dim chunk
                uint16_t* kp = a.pv.k + pv_k_elem(a.pv, page, hd - a.Hq, slot, jj, D);
                *(u32x2*)kp = (u32x2){pack2(y[0], y[1]), pack2(y[2], y[3])};
              } else {
                uint16_t* vp = a.pv.v + pv_v_index(a.pv, page, hd - a.Hq - a.Hkv, jj, slot, D);
#pragma unroll
                for (int e = 0; e < 4; ++e) vp[e * kTile] = to_bf16_bits(y[e]);
              }
            }
          }
        }
      }
    }
}

// ------------------------------------------------ split QKV finish ---
// The QKV projection with K split over workgroups (too few row tiles to
// fill the chip otherwise): the splits' partial sums part[s][t][n] (n in
// the packed row order: group G = head * D/16 + j / 8 holds pair element j
// in row j % 8 and j + D/2 in row 8 + j % 8) are added in split order, then
// RoPE, the q halves and the K/V append as in the projection's own
// epilogue.  One thread per (token, head, pair j).
__global__ __launch_bounds__(256) void qkv_finish_kernel(const float* part, int ks,
                                                         const PgemmArgs a) {
  const int D = a.D, half = D >> 1, gph = D >> 4;
  const int heads = a.Hq + 2 * a.Hkv;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.T * heads * half) return;
  const int t = (int)(idx / (heads * half));
  const int r = (int)(idx - (int64_t)t * heads * half);
  const int hd = r / half, j = r - hd * half;
  const int n0 = 16 * (hd * gph + (j >> 3)) + (j & 7), n1 = n0 + 8;
  const size_t N = (size_t)heads * D;
  float x0 = 0.f, x1 = 0.f;
  for (int sp = 0; sp < ks; ++sp) {
    const float* ps = part + ((size_t)sp * a.T + t) * N;
    x0 += ps[n0];
    x1 += ps[n1];
  }
  const int p = a.pos ? a.pos[t] : a.start_pos + t;
  const bool is_q = hd < a.Hq, is_k = !is_q && hd < a.Hq + a.Hkv;
  float y0 = x0, y1 = x1;
  if (is_q || is_k) {
    if (p < 0 || p >= a.max_pos) {
      set_error(a.err, ERR_ROPE);
      return;
    }
    const float cs = a.rcos[(size_t)p * half + j], sn = a.rsin[(size_t)p * half + j];
    y0 = __fsub_rn(__fmul_rn(x0, cs), __fmul_rn(x1, sn));
    y1 = __fadd_rn(__fmul_rn(x0, sn), __fmul_rn(x1, cs));
  }
  if (is_q) {
    uint16_t* qo = a.q_split + ((size_t)t * a.Hq + hd) * 2 * D;
    const uint16_t h0 = to_bf16_bits(y0), h1 = to_bf16_bits(y1);
    qo[j] = h0;
    qo[j + half] = h1;
    qo[D + j] = to_bf16_bits(y0 - bf16_lo(h0));
    qo[D + j + half] = to_bf16_bits(y1 - bf16_lo(h1));
    return;
  }
  const int psh = 4 + a.pv.pt_shift;  // log2 of the page's tokens
  if (p < 0 || (p >> psh) >= a.bt_stride) {
    set_error(a.err, ERR_LENGTH);
    return;
  }
  const int page = a.bt[(size_t)t * a.bt_row + (p >> psh)];
  if ((unsigned)page >= (unsigned)a.pv.num_pages) {
    set_error(a.err, ERR_PAGE);
    return;
  }
  const int slot = p & ((1 << psh) - 1);
  if (is_k) {
    a.pv.k[pv_k_elem(a.pv, page, hd - a.Hq, slot, j, D)] = to_bf16_bits(y0);
    a.pv.k[pv_k_elem(a.pv, page, hd - a.Hq, slot, j + half, D)] = to_bf16_bits(y1);
  } else {
    uint16_t* vp = a.pv.v + pv_v_index(a.pv, page, hd - a.Hq - a.Hkv, 0, slot, D);
    vp[j * kTile] = to_bf16_bits(y0);
    vp[(j + half) * kTile] = to_bf16_bits(y1);
  }
}

// ------------------------------------------------- residual + norm ---
// One workgroup per token row: x[t] += sum_s part[s][t] (splits in order,
// so the result does not depend on scheduling), then, if nw is given, the
// next RMSNorm of the new row into packed hi/lo pairs (padding rows zero).
// Each thread owns 8 consecutive columns per 2048.  The first kHold such
// chunks (rows up to 4096 wide) stay in registers between the two passes,
// and their norm weights are loaded before the sums: the second pass then
// needs no memory round trip of its own (wider rows re-read the rest).
constexpr int kHold = 2;

__device__ __forceinline__ void resid_chunk(float* row, const float* part, size_t split, int t, int N,
                                            int k, int ks, float4& a, float4& b) {
  a = *(const float4*)(row + k);
  b = *(const float4*)(row + k + 4);
#pragma unroll 8
  for (int sp = 0; sp < ks; ++sp) {
    const float* pr = part + sp * split + (size_t)t * N + k;
    const float4 pa = *(const float4*)pr, pb = *(const float4*)(pr + 4);
    a.x += pa.x; a.y += pa.y; a.z += pa.z; a.w += pa.w;
    b.x += pb.x; b.y += pb.y; b.z += pb.z; b.w += pb.w;
  }
  *(float4*)(row + k) = a;
  *(float4*)(row + k + 4) = b;
}

__device__ __forceinline__ void norm_chunk(uint16_t* xb, int t, int N, int k, float4 a, float4 b, uint4 w,
                                           float rs) {
  float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = v[2 * e] * bf16_lo(ww[e]) * rs;
    v[2 * e + 1] = v[2 * e + 1] * bf16_hi(ww[e]) * rs;
  }
  uint4 hi, lo;
  split8(v, hi, lo);
  *(uint4*)(xb + packed_pair_index(t, k, N, 0)) = hi;
  *(uint4*)(xb + packed_pair_index(t, k, N, 1)) = lo;
}

__global__ __launch_bounds__(256) void prefill_resid_kernel(float* x, const float* part, int ks,
                                                            int T, int N, const uint16_t* nw,
                                                            float eps, uint16_t* xb) {
  __shared__ float red[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (t >= T) {
    for (int k = 8 * tid; k < N; k += 8 * 256) {
      *(uint4*)(xb + packed_pair_index(t, k, N, 0)) = make_uint4(0u, 0u, 0u, 0u);
      *(uint4*)(xb + packed_pair_index(t, k, N, 1)) = make_uint4(0u, 0u, 0u, 0u);
    }
    return;
  }
  float* row = x + (size_t)t * N;
  const size_t split = (size_t)T * N;
  float4 ha[kHold], hb[kHold];
  uint4 hw[kHold];
#pragma unroll
  for (int h = 0; h < kHold; ++h) {
    const int k = 8 * tid + 2048 * h;
    hw[h] = nw && k < N ? *(const uint4*)(nw + k) : make_uint4(0u, 0u, 0u, 0u);
  }
  float ss = 0.f;
#pragma unroll
  for (int h = 0; h < kHold; ++h) {
    const int k = 8 * tid + 2048 * h;
    if (k < N) {
      resid_chunk(row, part, split, t, N, k, ks, ha[h], hb[h]);
      const float4 a = ha[h], b = hb[h];
      ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z +
            b.w * b.w;
    }
  }
  for (int k = 8 * tid + 2048 * kHold; k < N; k += 8 * 256) {
    float4 a, b;
    resid_chunk(row, part, split, t, N, k, ks, a, b);
    ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z +
          b.w * b.w;
  }
  if (!nw) return;
  ss = wave_sum(ss);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float rs = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)N + eps);
#pragma unroll
  for (int h = 0; h < kHold; ++h) {
    const int k = 8 * tid + 2048 * h;
    if (k < N) norm_chunk(xb, t, N, k, ha[h], hb[h], hw[h], rs);
  }
  for (int k = 8 * tid + 2048 * kHold; k < N; k += 8 * 256) {
    const float4 a = *(const float4*)(row + k), b = *(const float4*)(row + k + 4);
    norm_chunk(xb, t, N, k, a, b, *(const uint4*)(nw + k), rs);
  }
}

// -------------------------------------------------------- attention ---
// Causal paged attention of the prompt.  A workgroup's 16 query columns are
// (token, head) pairs: tpw = 16 / G consecutive tokens times the G heads of
// one kv head, column = G * (token - t0) + head.  Its 4 waves split the
// pages 0 .. the last token's position into 4 contiguous ranges (a prompt
// position attends to every page before it, so without the split one wave
// would walk them all, one dependent round trip per two pages).  For each
// page a wave forms S^T[key][column] = K q^T (v_mfma_f32_16x16x32_bf16, q as
// BF16 hi and lo halves) and then O[column][d] += P[column][key] V[key][d]
// (v_mfma_f32_16x16x16_bf16, P as hi and lo halves); the score tile's
// register layout is the P operand's, and V is stored [d][slot] in the
// page.  Key position kp is visible to a column whose position is at least
// kp.  The softmax is online in base 2 (scale * log2 e applied in the
// exponent), two pages per rescale, the next two pages' loads in flight
// meanwhile; the waves' (m, l, O) are merged in LDS in wave order by the
// log-sum-exp rule.  Workgroups with the latest tokens (the most pages) are
// launched first.
constexpr int kPW = 2;
template <bool B>
struct BoolC {
  static constexpr bool value = B;
};

template <int D>
__global__ __launch_bounds__(256) void prefill_attention_kernel(const PattnArgs a) {
  constexpr int NH = D / 32;  // 32-wide q.K blocks
  constexpr int NC = D / 16;  // 16-wide output column blocks
  __shared__ float sm_m[4][16];
  __shared__ float sm_l[4][16];
  __shared__ float sm_o[4][16][D + 1];
  const int kvh = blockIdx.y;
  const int blk = gridDim.x - 1 - blockIdx.x;
  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = l & 15, grp = l >> 4;
  const int G = a.G, tpw = 16 / G;
  const int t0 = blk * tpw;
  if (t0 >= a.T) return;
  const int tend = min(t0 + tpw, a.T);
  const int pmax = a.start_pos + tend - 1;  // the group's last position
  const int npages = pmax / kTile + 1;      // 16-token tiles
  const int pmin = a.start_pos + t0;        // its first: keys up to here need no mask
  // this wave's tiles [pb, pe); a page holds 1 << sh tiles
  const int sh = a.pv.pt_shift;
  const int npw = (npages + 3) / 4;
  const int pb = w * npw, pe = min(npages, pb + npw);

  // this lane's query column
  const int tk = col / G, gh = col - tk * G;
  const bool cval = col < tpw * G && t0 + tk < a.T;
  const int lim = cval ? a.start_pos + t0 + tk : -1;
  const float c2 = fabsf(a.scale) * kLog2e;
  const unsigned sgn = a.scale < 0.f ? 0x80008000u : 0u;
  u32x4 qh[NH], ql[NH];
  {
    const uint16_t* qp =
        a.q + ((size_t)(cval ? t0 + tk : 0) * a.Hq + (size_t)kvh * G + gh) * 2 * D + 8 * grp;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const u32x4 hv = *(const u32x4*)(qp + 32 * h), lv = *(const u32x4*)(qp + D + 32 * h);
      qh[h] = cval ? hv ^ sgn : z;
      ql[h] = cval ? lv ^ sgn : z;
    }
  }

  struct Chunk {
    u32x4 k[kPW][NH];
    u32x2 v[kPW][NC];
  };
  bool bad = false;
  // A lane's element offsets inside a tile do not change from tile to tile
  // (K: slot col, dims 32 h + 8 grp.., i.e. chunk 4 h + grp, 1 KiB per
  // block h; V: dim col, slots 4 grp..): the address of a load is the
  // tile's base, uniform across the wave, plus these.
  const uint32_t klane = (uint32_t)(8 * l);
  const uint32_t vlane = (uint32_t)(col * kTile + 4 * grp);
  // tiles past the wave's range read its last tile and are masked
  auto load = [&](Chunk& C, int lp0) {
#pragma unroll
    for (int i = 0; i < kPW; ++i) {
      const int lt = min(lp0 + i, pe - 1);
      int page = a.bt[lt >> sh];
      const int sub = (lt & ((1 << sh) - 1)) * kTile;
      const bool ok = (unsigned)page < (unsigned)a.pv.num_pages;
      bad |= !ok;
      page = ok ? page : 0;
      const uint16_t* kb = a.pv.k + pv_k_elem(a.pv, page, kvh, sub, 0, D);
#pragma unroll
      for (int h = 0; h < NH; ++h) C.k[i][h] = *(const u32x4*)(kb + klane + 512 * h);
      const uint16_t* vb = a.pv.v + pv_v_index(a.pv, page, kvh, 0, sub, D);
#pragma unroll
      for (int c = 0; c < NC; ++c) C.v[i][c] = *(const u32x2*)(vb + vlane + c * 16 * kTile);
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4 o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = (f32x4){0.f, 0.f, 0.f, 0.f};

  // MASKED false: every tile of the chunk lies in the wave's range and below
  // the group's first position, so no score, probability or V slot needs a
  // mask (the masked variant computes the same values for such tiles).
  auto step = [&](const Chunk& C, int lp0, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    f32x4 s[kPW];
    bool full[kPW], inr[kPW];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPW; ++i) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        acc = mfma_k32(C.k[i][h], qh[h], acc);
        acc = mfma_k32(C.k[i][h], ql[h], acc);
      }
      const int kp0 = (lp0 + i) * kTile;
      inr[i] = !MASKED || lp0 + i < pe;                              // uniform
      full[i] = !MASKED || (inr[i] && kp0 + kTile - 1 <= pmin);  // uniform
      if (!full[i]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = inr[i] && kp0 + 4 * grp + r <= lim ? acc[r] : -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, acc[r]);
      s[i] = acc;
    }
    mx = rows_max4(mx);
    const float mn = fmaxf(m, mx);
    const float msub = mn == -INFINITY ? 0.f : mn;
    const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mn) * c2);
    m = mn;
    float ps = 0.f;
    s16x4 ph[kPW], pl[kPW];
#pragma unroll
    for (int i = 0; i < kPW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = (s[i][r] - msub) * c2;
        if (!full[i]) x = s[i][r] == -INFINITY ? -INFINITY : x;
        const float p = __builtin_amdgcn_exp2f(x);
        ps += p;
        const __bf16 hi = (__bf16)p;
        ph[i][r] = __builtin_bit_cast(short, hi);
        pl[i][r] = __builtin_bit_cast(short, (__bf16)(p - (float)hi));
      }
    ps = rows_sum4(ps);
    lsum = lsum * alpha + ps;
    // O row 4 grp + r belongs to column 4 grp + r: its factor lives in lane 4 grp + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * grp + r);
#pragma unroll
      for (int c = 0; c < NC; ++c) o[c][r] *= ar;
    }
#pragma unroll
    for (int i = 0; i < kPW; ++i) {
      // slots past the group's last position, or pages past the wave's
      // range, may hold anything: zero them
      const int nv = inr[i] ? pmax - ((lp0 + i) * kTile + 4 * grp) + 1 : 0;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        u32x2 vv = C.v[i][c];
        if (MASKED && nv < 4) {
          vv.x = nv >= 2 ? vv.x : (nv == 1 ? (vv.x & 0xffffu) : 0u);
          vv.y = nv == 3 ? (vv.y & 0xffffu) : 0u;
        }
        const s16x4 vb = __builtin_bit_cast(s16x4, vv);
        o[c] = mfma_k16(ph[i], vb, o[c]);
        o[c] = mfma_k16(pl[i], vb, o[c]);
      }
    }
  };

  if (pb < pe) {
    Chunk A, B;
    load(A, pb);
    // chunks starting before `lfull` hold only full tiles in range
    const int lfull = min(pe, (pmin + 1) / kTile) - kPW + 1;
    auto run = [&](const Chunk& C, int lp) {
      if (lp < lfull)
        step(C, lp, BoolC<false>{});
      else
        step(C, lp, BoolC<true>{});
    };
    for (int lp = pb;; lp += 2 * kPW) {
      if (lp + kPW < pe) load(B, lp + kPW);
      run(A, lp);
      if (lp + kPW >= pe) break;
      if (lp + 2 * kPW < pe) load(A, lp + 2 * kPW);
      run(B, lp + kPW);
      if (lp + 2 * kPW >= pe) break;
    }
  }
  if (bad && l == 0) set_error(a.err, ERR_PAGE);

  // ---- the waves' (m, l, O) into LDS, merged in wave order
  if (grp == 0) {
    sm_m[w][col] = m;
    sm_l[w][col] = lsum;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) sm_o[w][4 * grp + r][col + 16 * c] = o[c][r];
  __syncthreads();

  // ---- O / l, stored as BF16 hi/lo pairs into the output projection's
  // packed input; thread tid takes outputs (g, d) = idx / D, idx % D
  const int QD = a.Hq * D;
  for (int idx = tid; idx < 16 * D; idx += 256) {
    const int g = idx / D, d = idx % D;
    const int t = t0 + g / G, h = kvh * G + g % G;
    if (g >= tpw * G || t >= a.T) continue;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, sm_m[ww][g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const float mw = sm_m[ww][g];
      const float sc = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((mw - M) * c2);
      L += sc * sm_l[ww][g];
      O += sc * sm_o[ww][g][d];
    }
    const float y = O / L;
    const uint16_t hb = to_bf16_bits(y);
    const int k = h * D + d;
    a.out[packed_pair_index(t, k, QD, 0)] = hb;
    a.out[packed_pair_index(t, k, QD, 1)] = to_bf16_bits(y - bf16_lo(hb));
  }
}

// A plan's (rg, cg) names the workgroup tile as 32 rg rows by 32 cg tokens;
// the 256- and 128-row tiles run on 8 waves (4 x 2), the others on 4.
template <int EPI>
hipError_t launch_pg(const PgemmArgs& a, const PgemmPlan& p, hipStream_t st) {
  const int wgs = p.tiles * (EPI == EPI_RESID ? p.ks : 1);
  if (p.rg == 8 && p.cg == 4) {
    if constexpr (EPI != EPI_LOGITS)
      prefill_gemm_kernel<EPI, 4, 4, 4><<<wgs, 512, 0, st>>>(a);
    else
      prefill_gemm_kernel<EPI, 8, 4, 2><<<wgs, 256, 0, st>>>(a);
  } else if (p.rg == 4 && p.cg == 4) {
    if constexpr (EPI != EPI_LOGITS)
      prefill_gemm_kernel<EPI, 2, 4, 4><<<wgs, 512, 0, st>>>(a);
    else
      prefill_gemm_kernel<EPI, 4, 4, 2><<<wgs, 256, 0, st>>>(a);
  } else if (p.rg == 2 && p.cg == 4) {
    prefill_gemm_kernel<EPI, 2, 4, 2><<<wgs, 256, 0, st>>>(a);
  } else if (p.rg == 2 && p.cg == 2) {
    prefill_gemm_kernel<EPI, 2, 2, 2><<<wgs, 256, 0, st>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_norm(const float* x, const uint16_t* xw, int K, int T, float eps,
                               uint16_t* out, hipStream_t st) {
  prefill_norm_kernel<<<(T + 15) / 16 * 16, 256, 0, st>>>(x, xw, K, T, eps, out);
  return hipGetLastError();
}

hipError_t launch_prefill_gemm(int epi, const PgemmArgs& a, const PgemmPlan& p, hipStream_t st) {
  if (a.K % 32 != 0 || a.T < 1) return hipErrorInvalidValue;
  if (epi == EPI_RESID && a.ksplit != p.ks) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_QKV: return launch_pg<EPI_QKV>(a, p, st);
    case EPI_RESID: return launch_pg<EPI_RESID>(a, p, st);
    case EPI_SWIGLU: return launch_pg<EPI_SWIGLU>(a, p, st);
    case EPI_LOGITS: return launch_pg<EPI_LOGITS>(a, p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_qkv_finish(const float* part, int ks, const PgemmArgs& a, hipStream_t st) {
  const int64_t n = (int64_t)a.T * (a.Hq + 2 * a.Hkv) * (a.D / 2);
  qkv_finish_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(part, ks, a);
  return hipGetLastError();
}

hipError_t launch_prefill_resid(float* x, const float* part, int ks, int T, int N,
                                const uint16_t* nw, float eps, uint16_t* xb, hipStream_t st) {
  const int rows = nw ? (T + 15) / 16 * 16 : T;
  prefill_resid_kernel<<<rows, 256, 0, st>>>(x, part, ks, T, N, nw, eps, xb);
  return hipGetLastError();
}

hipError_t launch_prefill_attention(const PattnArgs& a, hipStream_t st) {
  const int tpw = 16 / a.G;
  const dim3 grid((a.T + tpw - 1) / tpw, a.Hkv);
  if (a.D == 64)
    prefill_attention_kernel<64><<<grid, 256, 0, st>>>(a);
  else if (a.D == 128)
    prefill_attention_kernel<128><<<grid, 256, 0, st>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
