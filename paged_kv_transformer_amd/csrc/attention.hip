// Direct paged GQA decode attention with FP32 online softmax, gfx950.
//
// The operation is the paged decode attention of the "Inference from
// Scratch" engine summary (its paged-attention bullet): the cached tokens
// are read where the block table says they are, folded into a running
// softmax, and no copy of the prefix or of the scores is ever made.  Here
// one workgroup takes one
// (sequence, kv head, split of 8 16-token tiles); its 4 waves take 2 tiles
// each.  Calls of many sequences (at least kAttnLargeWgs such workgroups)
// take 4 tiles per wave and 16 per split instead: half the workgroups and
// split records, more loads in flight per wave.  The whole GQA group of the
// kv head shares every tile load.
//
// One 16-token tile is exactly one matrix-core tile:
//   scores  S[t][g] = sum_d K[t][d] * q[g][d]      v_mfma_f32_16x16x32_bf16 x4
//   output  O[g][d] += sum_t P[g][t] * V[t][d]     v_mfma_f32_16x16x16_bf16 x8
// The score tile comes out of the first product in exactly the register
// layout the second product wants for P (lane l holds tokens 4*(l/16)+r of
// head l%16), and the page stores V as [d][slot], so a lane reads its four
// tokens of one dimension as 8 contiguous bytes.  q and P are FP32 values
// split into two BF16 halves (hi + lo) so that the products keep ~16
// significant bits on both sides; the accumulation is FP32.
//
// Softmax: scores are kept in base-2 units (q is prescaled by the
// attention scale times log2 e), so e^x becomes the hardware 2^x.  Each wave
// takes the maximum over its pages, exponentiates, and keeps (m, l, O);
// waves and then splits are merged with the log-sum-exp rule m = max m_i,
// l = sum l_i 2^(m_i - m), O = sum O_i 2^(m_i - m), in a
// fixed order, so the result depends only on the logical page sequence
// (never on where pages sit in the pool).  When the block table allows a
// single split, the workgroup finishes its sequence; otherwise every split
// leaves its (m, l, O) record and a second, small kernel merges them:
// workgroups never wait on one another (on this GPU a cross-workgroup
// handoff inside a kernel costs more than the extra launch).
//
// Latency matters as much as bandwidth here (a 16-sequence call moves tens
// of MB, a few microseconds at HBM speed), so every dependent round trip is
// counted: the length and block-table entries are loaded together, then
// all K, V and q loads of a wave are issued back to back before any use,
// and the merge kernel reads nothing but its records.
#include "pkv_dev.h"

namespace pkv {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Output element idx = g * D + d of kv head kvh of sequence b: plain
// [B][Hq][D], or packed as the output projection's input ([B][Hq * D]):
// FP32 for the weight-streaming projection, BF16 hi/lo pairs for the tiled
// one.
template <int D>
__device__ __forceinline__ void store_out(const AttnArgs& a, int b, int kvh, int idx, float v) {
  const int k = kvh * a.G * D + idx;
  const int QD = a.Hq * D;
  if (a.out_packed == 2) {
    uint16_t* o = (uint16_t*)a.out;
    const uint16_t h = to_bf16_bits(v);
    o[packed_pair_index(b, k, QD, 0)] = h;
    o[packed_pair_index(b, k, QD, 1)] = to_bf16_bits(v - bf16_lo(h));
  } else if (a.out_packed) {
    a.out[packed_act_index(b, k, QD)] = v;
  } else {
    a.out[(size_t)b * QD + k] = v;
  }
}

// Keep the first `nv` of the four BF16 values in v (the rest -> +0).
__device__ __forceinline__ u32x2 keep_first(u32x2 v, int nv) {
  if (nv >= 4) return v;
  u32x2 r;
  r.x = nv >= 2 ? v.x : (nv == 1 ? (v.x & 0xffffu) : 0u);
  r.y = nv == 3 ? (v.y & 0xffffu) : 0u;
  return r;
}

template <int QM, int D, int PW>
__global__ __launch_bounds__(kAttnWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 5))) void
paged_attention_kernel(const AttnArgs a) {
  constexpr int NH = D / 32;  // 32-wide q.K blocks
  constexpr int NC = D / 16;  // 16-wide output column blocks
  constexpr int REC = attn_rec(D);
  constexpr int CP = kAttnWaves * PW;  // tiles per split
  constexpr int NW = kAttnWaves;
  constexpr int NT = NW * 64;
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ float sm_o[NW][16][D + 1];

  // the highest splits are launched first: only long sequences have them,
  // and starting the longest work first keeps it out of the kernel's tail
  const int kvh = blockIdx.x, b = blockIdx.y, split = a.max_splits - 1 - (int)blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = l & 15, grp = l >> 4;
  const int G = a.G;

  // ---- the length and this wave's block-table entries (index clamped to
  // the table row; entries past the sequence are masked below), in flight
  // together: the empty asm makes the entries live before the length test,
  // so they are not sunk below it into a second round trip.
  // Tiles are 16 tokens; a page holds 1 << sh of them (sh = 0 or 4).
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int sh = a.pv.pt_shift, PT = kTile << sh;
  const int32_t* btrow = a.bt + (size_t)b * a.bt_row;
  int page[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i)
    page[i] = btrow[min((split * CP + NW * i + wu) >> sh, a.bt_stride - 1)];
  const int n = a.lens[b] + a.len_add;
#pragma unroll
  for (int i = 0; i < PW; ++i) asm volatile("" ::"s"(page[i]));
  // With one split per sequence (max_splits == 1) the workgroup writes the
  // output itself; otherwise every workgroup leaves a record, an empty one
  // (m = -inf) when it has no tokens, and the merge kernel writes every
  // output.
  const bool single = a.max_splits == 1;
  float* rec = a.part + (((size_t)b * a.Hkv + kvh) * a.max_splits + split) * REC;
  const bool bad_len = n < 0 || (int64_t)n > (int64_t)a.bt_stride * PT;
  if (bad_len && split == 0 && tid == 0) set_error(a.err, ERR_LENGTH);
  const int npages = bad_len ? 0 : (n + kTile - 1) / kTile;  // tiles
  const int ns = npages > 0 ? (npages + CP - 1) / CP : 1;
  if (npages == 0 || split >= ns) {
    if (single) {
      for (int i = tid; i < G * D; i += NT) store_out<D>(a, b, kvh, i, 0.f);
    } else if (tid < G) {
      rec[tid] = -INFINITY;
    }
    return;
  }

  // ---- every remaining load of the wave, issued back to back before any
  // use (the scheduling barrier keeps the compiler from interleaving them
  // with the arithmetic): q, then per page K (2 x 16 B) and V (4 x 8 B).  A
  // page past the sequence or outside the pool reads page 0 and is masked.
  int lpv[PW];
  bool bad = false;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int lp = split * CP + NW * i + wu;  // uniform across the wave
    const bool live = lp < npages;
    const bool ok = (unsigned)page[i] < (unsigned)a.pv.num_pages;
    bad |= live && !ok;
    lpv[i] = live && ok ? lp : -1;
    page[i] = live && ok ? page[i] : 0;
  }
  // q^T operand: lane holds head g = col, dims 8*grp + e + 32*h; lanes past
  // the group read head 0 of the group and use zeros.  Both q formats are
  // the matrix operand as loaded: BF16 q, or an FP32 q's BF16 hi and lo
  // halves (two products per block).
  constexpr bool kSplitQ = QM == kQSplit;
  const int gq = col < G ? col : 0;
  const size_t qhead = (size_t)b * a.Hq + (size_t)kvh * G + gq;
  const uint16_t* qp = a.q + qhead * (kSplitQ ? 2 : 1) * D + 8 * grp;
  u32x4 qraw[NH], qlraw[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    qraw[h] = *(const u32x4*)(qp + 32 * h);
    if (kSplitQ) qlraw[h] = *(const u32x4*)(qp + D + 32 * h);
  }
  // the tile's first slot in its page
  int sub[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) sub[i] = ((split * CP + NW * i + wu) & ((1 << sh) - 1)) * kTile;
  // K and V are read once per call (one workgroup per kv head and split
  // takes the whole query group): non-temporal loads, so the stream does
  // not displace what the rest of the step keeps in the caches (measured
  // 9 % faster per call than ordinary loads).
  u32x4 kr[PW][NH];
  u32x2 vr[PW][NC];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    // lane l = 16 grp + col holds slot col, dims 32 h + 8 grp ..: chunk
    // 4 h + grp of the tile, 16 bytes at (chunk * 16 + col) * 8 elements,
    // so a load instruction reads 1 KiB contiguously
    const uint16_t* kp = a.pv.k + pv_k_elem(a.pv, page[i], kvh, sub[i], 0, D) + 8 * l;
#pragma unroll
    for (int h = 0; h < NH; ++h) kr[i][h] = __builtin_nontemporal_load((const u32x4*)(kp + 512 * h));
  }
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const uint16_t* vp = a.pv.v + pv_v_index(a.pv, page[i], kvh, col, sub[i], D) + 4 * grp;
#pragma unroll
    for (int c = 0; c < NC; ++c) vr[i][c] = __builtin_nontemporal_load((const u32x2*)(vp + c * 16 * kTile));
  }
  __builtin_amdgcn_sched_barrier(0);
  if (bad && l == 0) set_error(a.err, ERR_PAGE);
  // The scores q.K come out unscaled; the softmax applies scale * log2 e in
  // the exponent, so that every exponential is one hardware 2^x and the
  // maxima m kept in the records are in base-2 units.
  // A negative scale flips the sign of q instead (exact in BF16), so that
  // the factor in the exponent is never negative and the row maximum of the
  // raw scores is the maximum of the scaled ones.
  const float c2 = fabsf(a.scale) * kLog2e;
  const unsigned sgn = a.scale < 0.f ? 0x80008000u : 0u;
  bf16x8 qh[NH], ql[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    qh[h] = __builtin_bit_cast(bf16x8, col < G ? qraw[h] ^ sgn : z);
    if (kSplitQ) ql[h] = __builtin_bit_cast(bf16x8, col < G ? qlraw[h] ^ sgn : z);
  }

  // ---- scores: lane holds S[t = 4*grp + r][g = col] of each page
  bool full[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) full[i] = lpv[i] >= 0 && (lpv[i] + 1) * kTile <= n;
  f32x4 s[PW];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      acc = mfma_k32(kr[i][h], qh[h], acc);
      if (kSplitQ) acc = mfma_k32(kr[i][h], ql[h], acc);
    }
    // a full page (every page of a sequence but its last) needs no mask;
    // the test is uniform across the wave
    if (!full[i]) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = lpv[i] * kTile + 4 * grp + r;
        acc[r] = lpv[i] >= 0 && t < n ? acc[r] : -INFINITY;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, acc[r]);
    s[i] = acc;
  }
  mx = rows_max4(mx);

  // ---- P = 2^((S - m) scale log2 e) split hi/lo; row sums.  Masked scores
  // are -inf and give 0; a wave with no token at all (m = -inf) subtracts 0.
  const float msub = mx == -INFINITY ? 0.f : mx;
  const float m2 = mx == -INFINITY ? -INFINITY : mx * c2;  // base-2 units
  float lsum = 0.f;
  s16x4 ph[PW], pl[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = (s[i][r] - msub) * c2;
      // masked scores stay -inf (a zero scale would otherwise make them NaN)
      if (!full[i]) x = s[i][r] == -INFINITY ? -INFINITY : x;
      const float p = __builtin_amdgcn_exp2f(x);
      lsum += p;
      const __bf16 hi = (__bf16)p;
      ph[i][r] = __builtin_bit_cast(short, hi);
      pl[i][r] = __builtin_bit_cast(short, (__bf16)(p - (float)hi));
    }
  lsum = rows_sum4(lsum);

  // ---- O[g][d]: lane holds rows g = 4*grp + r, column d = col + 16*c
  f32x4 o[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) o[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    // unused slots of a partial page may hold anything (NaN included): zero them
    const int nv = full[i] ? 4 : (lpv[i] < 0 ? 0 : n - (lpv[i] * kTile + 4 * grp));
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const s16x4 vb = __builtin_bit_cast(s16x4, keep_first(vr[i][c], nv));
      o[c] = mfma_k16(ph[i], vb, o[c]);
      o[c] = mfma_k16(pl[i], vb, o[c]);
    }
  }

  // ---- merge the four waves
  if (grp == 0) {
    sm_m[w][col] = m2;
    sm_l[w][col] = lsum;
  }
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int g = 4 * grp + r;
      if (g < G) sm_o[w][g][col + 16 * c] = o[c][r];
    }
  __syncthreads();

  for (int idx = tid; idx < G * D; idx += NT) {
    const int g = idx / D, d = idx % D;
    float M = sm_m[0][g];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sm_m[ww][g]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = sm_m[ww][g];
      const float e = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += e * sm_l[ww][g];
      O += e * sm_o[ww][g][d];
    }
    if (single) {
      store_out<D>(a, b, kvh, idx, L > 0.f ? O / L : 0.f);
    } else {
      if (d == 0) {
        rec[g] = M;
        rec[16 + g] = L;
      }
      rec[32 + idx] = O;
    }
  }
}

// Merge of the split records of every (sequence, kv head), launched when
// max_splits > 1; the records come from the previous kernel on the stream.
// A split with no tokens left an empty record (m = -inf), so the merge needs
// neither the lengths nor any other input than the records.  One thread per
// output (head g, dim d) combines the splits in order, 16 at a time: the
// m, l and O of 16 splits are loaded together (split indexes clamped to the
// record array and masked past it), so up to 16 splits cost one round of
// loads.  The kernel arguments are read in one batch on entry.
template <int D>
__global__ __launch_bounds__(256) void attention_merge_kernel(const AttnArgs a) {
  constexpr int CH = 16;
  constexpr int REC = attn_rec(D);
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int G = a.G, tid = threadIdx.x, S = a.max_splits;
  asm volatile("" ::"s"(a.part), "s"(a.out), "s"(a.Hq), "s"(a.Hkv), "s"(a.G), "s"(a.max_splits),
               "s"(a.out_packed));
  const float* rec0 = a.part + ((size_t)b * a.Hkv + kvh) * S * REC;
  for (int idx = tid; idx < G * D; idx += 256) {
    const int g = idx / D;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int c0 = 0; c0 < S; c0 += CH) {
      float m[CH], lv[CH], ov[CH];
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const float* r = rec0 + (size_t)min(c0 + j, S - 1) * REC;
        m[j] = r[g];
        lv[j] = r[16 + g];
        ov[j] = r[32 + idx];
      }
      float Mc = M;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        m[j] = c0 + j < S ? m[j] : -INFINITY;
        Mc = fmaxf(Mc, m[j]);
      }
      const float sc = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mc);
      L *= sc;
      O *= sc;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const bool on = m[j] != -INFINITY;
        const float e = on ? __builtin_amdgcn_exp2f(m[j] - Mc) : 0.f;
        L += on ? e * lv[j] : 0.f;
        O += on ? e * ov[j] : 0.f;
      }
      M = Mc;
    }
    store_out<D>(a, b, kvh, idx, L > 0.f ? O / L : 0.f);
  }
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, int batch, int qmode, hipStream_t st) {
  // kv head fastest: workgroups go to the 8 XCDs round-robin in launch
  // order, so every XCD gets the same mix of sequences and splits (with
  // the split fastest, the XCDs holding the low splits of every sequence
  // would get most of the non-empty workgroups)
  const dim3 grid(a.Hkv, batch, a.max_splits);
  if (a.D != 64 && a.D != 128) return hipErrorInvalidValue;
  if (a.pw != kAttnPW && a.pw != kAttnPWLarge) return hipErrorInvalidValue;
  const bool large = a.pw == kAttnPWLarge;
  const int nt = kAttnWaves * 64;
  if (a.D == 64) {
    if (qmode == kQSplit) {
      if (large) paged_attention_kernel<kQSplit, 64, kAttnPWLarge><<<grid, nt, 0, st>>>(a);
      else paged_attention_kernel<kQSplit, 64, kAttnPW><<<grid, nt, 0, st>>>(a);
    } else {
      if (large) paged_attention_kernel<kQBf16, 64, kAttnPWLarge><<<grid, nt, 0, st>>>(a);
      else paged_attention_kernel<kQBf16, 64, kAttnPW><<<grid, nt, 0, st>>>(a);
    }
  } else {
    if (qmode == kQSplit) {
      if (large) paged_attention_kernel<kQSplit, 128, kAttnPWLarge><<<grid, nt, 0, st>>>(a);
      else paged_attention_kernel<kQSplit, 128, kAttnPW><<<grid, nt, 0, st>>>(a);
    } else {
      if (large) paged_attention_kernel<kQBf16, 128, kAttnPWLarge><<<grid, nt, 0, st>>>(a);
      else paged_attention_kernel<kQBf16, 128, kAttnPW><<<grid, nt, 0, st>>>(a);
    }
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits <= 1) return e;
  if (a.D == 64)
    attention_merge_kernel<64><<<dim3(a.Hkv, batch), 256, 0, st>>>(a);
  else
    attention_merge_kernel<128><<<dim3(a.Hkv, batch), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace pkv
