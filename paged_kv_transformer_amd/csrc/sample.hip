// Sampling of each sequence's next token from its FP32 logits, gfx950.
//
// The decoding step after the LM head ("手写LLM推理引擎" §3.3 logits
// post-processing, §2.4 decoding strategies; llmc 五 plans temperature,
// top-k and top-p after greedy): z = logits / T, p = softmax(z), the
// nucleus = the smallest prefix of the tokens by decreasing p (equal logits:
// lower index first) whose cumulative p reaches top_p, capped at top_k
// tokens, then the first kept token in vocabulary order whose renormalised
// cumulative p exceeds the draw u (an input, so the caller owns the random
// stream).  T <= 0 is greedy.
//
// Nothing is sorted.  The nucleus is found by a radix select on an
// order-preserving 32-bit key of the logit (larger logit, larger key): three
// digits (11, 11, 10 bits), each a histogram of (token count, probability
// mass) over the tokens whose higher digits match the choice so far, then a
// descending scan for the first bucket where the count reaches top_k or the
// mass reaches top_p.  Probability mass is fixed point, p~ = 2^((l - max) T'
// log2 e) * 2^32 as a 64-bit integer, so every sum is an integer sum:
// exact, independent of the order in which workgroups add, and the same on
// every replay.
//
// A batch of B sequences runs on B x W workgroups, each taking one chunk of
// the vocabulary (the logits of a 16-sequence batch are 8 MB, and one
// workgroup per sequence would leave most of the chip idle), until the
// first level has chosen its bucket; each chunk then writes its tokens in
// that bucket (a few thousand per sequence) to its own segment of a
// per-sequence candidate list, and one 1024-thread workgroup per sequence
// finishes from the list.  Workgroups never wait on each other; the four
// launches are:
//   K0 chunk maxima                  (clears the first-level histogram)
//   K1 normaliser + first-level histogram
//   K2 first-level choice; per chunk, the mass above the chosen bucket, and
//      the bucket's tokens written to the chunk's segment of the list
//   K3 per sequence: the second and third levels over the candidates (the
//      threshold key and how many of its ties are kept), each chunk's kept
//      mass, and the draw: the chunk holding u, then the token inside it
// The first-level choice is made by every workgroup of K2 alike and stored
// by workgroup 0 of the sequence for K3.
#include "pkv_dev.h"

namespace pkv {
namespace {

constexpr int kSThreads = 256;
constexpr int kFThreads = 1024;  // the finishing launch: one workgroup per sequence
constexpr int kBuckets = 2048;
constexpr float kLog2eS = 1.4426950408889634f;

// Order-preserving key of an FP32 value (finite or -inf): larger value,
// larger key; -0 takes the key of +0, since the two are equal logits.
__device__ __forceinline__ uint32_t skey(float v) {
  uint32_t u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int digit(uint32_t key, int level) {
  return level == 0 ? (int)(key >> 21) : level == 1 ? (int)((key >> 10) & 2047u) : (int)(key & 1023u);
}

// Key bits a level's digit sits below: a token is a candidate of level L if
// its key agrees with the prefix on the bits of levels 0 .. L-1.
__device__ __forceinline__ bool in_prefix(uint32_t key, int level, uint32_t prefix) {
  return level == 0 || (level == 1 ? (key >> 21) == prefix : (key >> 10) == prefix);
}

struct SArgs {
  const float* logits;
  int32_t B, V;
  const float* temperature;
  const float* top_p;
  const int32_t* top_k;
  const float* u;
  int32_t* tokens;
  SampleWs w;
  int32_t W, chunk;  // workgroups per sequence, logits per workgroup
};

__device__ __forceinline__ float inv_temp(const SArgs& a, int b) {
  const float T = a.temperature[b];
  return T > 0.f ? kLog2eS / T : 0.f;  // greedy: every token mass 1, top_k 1
}

__device__ __forceinline__ uint64_t fixed_mass(float l, float m, float c) {
  // (0, 1]; a -inf logit gives 0 (also when greedy, where -inf * 0 is NaN)
  const float x = (l - m) * c;
  const float e = x == x ? __builtin_amdgcn_exp2f(x) : 0.f;
  // e * 2^32 truncated; below 2^32 one 32-bit conversion does it
  const float f = e * 4294967296.0f;
  return f >= 4294967296.0f ? (1ull << 32) : (uint64_t)(uint32_t)f;
}

// A sequence sampled by top-p alone (temperature > 0, no top-k cap, top_p <
// 1) reaches its mass budget no later than its count budget (all V tokens)
// in every bucket scan, so the first two levels need no token counts: the
// choices are the same without them, and each histogram update is one
// atomic instead of two.  The last level keeps its counts (the ties of the
// threshold key are counted there).
__device__ __forceinline__ bool mass_only(const SArgs& a, int b) {
  const int k = a.top_k[b];
  return a.temperature[b] > 0.f && !(k > 0 && k < a.V) && a.top_p[b] < 1.f;
}

// The chunk of workgroup (b, w): elements [e0, e1) of sequence b.  Passes
// whose result does not depend on order read it coalesced (thread t takes
// e0 + t, e0 + t + 256, ...); the draw, which walks vocabulary order, gives
// thread t the E consecutive elements from e0 + t E.
struct Chunk {
  const float* row;
  int e0, e1, E;
};

template <int NT = kSThreads>
__device__ __forceinline__ Chunk chunk_of(const SArgs& a, int b, int w) {
  Chunk c;
  c.row = a.logits + (size_t)b * a.V;
  c.e0 = w * a.chunk;
  c.e1 = min(a.V, c.e0 + a.chunk);
  c.E = a.chunk / NT;
  return c;
}

// Latency is most of a launch's time here (a chunk is 8-128 KB), so every
// kernel issues its first batch of logits, and the few values its
// decisions need (the chunk maxima, the previous level's histogram, the
// choice records), back to back before it waits for any of them: one round
// trip instead of one per dependent step.  kSBatch logits per thread are in
// flight per batch (a 4096-logit chunk is one batch).
constexpr int kSBatch = 16;

// Thread t's next batch in pass order: e, e + 256, ...; -inf past the chunk.
__device__ __forceinline__ void load_batch(const Chunk& ch, int e, float (&v)[kSBatch]) {
#pragma unroll
  for (int i = 0; i < kSBatch; ++i) {
    const int x = e + i * kSThreads;
    v[i] = x < ch.e1 ? ch.row[x] : -INFINITY;
  }
}

// Clears `n` 32-bit words of `p` with the workgroups of one sequence.
__device__ __forceinline__ void clear_words(uint32_t* p, int n, int w, int W) {
  for (int i = w * kSThreads + (int)threadIdx.x; i < n; i += W * kSThreads) p[i] = 0u;
}

// Inclusive scan over a wave's 64 lanes by data-parallel-primitive moves:
// within each 16-lane row by shifts of 1, 2, 4 and 8 lanes (lanes shifted
// in from outside the row read 0), then lane 15's sum into rows 1 and 3 and
// lane 31's into rows 2 and 3.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_z(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, true);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_z(uint64_t v) {
  const uint32_t lo = dpp_z<CTRL, ROW_MASK>((uint32_t)v);
  const uint32_t hi = dpp_z<CTRL, ROW_MASK>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <typename T>
__device__ __forceinline__ T wave_scan(T v) {
  v += dpp_z<0x111, 0xf>(v);  // row_shr:1
  v += dpp_z<0x112, 0xf>(v);  // row_shr:2
  v += dpp_z<0x114, 0xf>(v);  // row_shr:4
  v += dpp_z<0x118, 0xf>(v);  // row_shr:8
  v += dpp_z<0x142, 0xa>(v);  // row_bcast:15
  v += dpp_z<0x143, 0xc>(v);  // row_bcast:31
  return v;
}
__device__ __forceinline__ uint64_t lane63(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Inclusive scan over the workgroup's threads in thread order: within each
// wave, then the sums of the waves before (one barrier pair).
template <typename T, int NT = kSThreads>
__device__ __forceinline__ T wg_scan(T v) {
  __shared__ T s_wave[NT / 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_scan(v);
  if (lane == 63) s_wave[wv] = v;
  __syncthreads();
  T add = 0;
  for (int i = 0; i < wv; ++i) add += s_wave[i];
  __syncthreads();
  return v + add;
}

// The same for a (count, mass) pair, sharing the barriers.
template <int NT>
__device__ __forceinline__ void wg_scan2(uint32_t& c, uint64_t& m) {
  __shared__ uint32_t s_c[NT / 64];
  __shared__ uint64_t s_m[NT / 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  c = wave_scan(c);
  m = wave_scan(m);
  if (lane == 63) {
    s_c[wv] = c;
    s_m[wv] = m;
  }
  __syncthreads();
  uint32_t ac = 0;
  uint64_t am = 0;
  for (int i = 0; i < wv; ++i) {
    ac += s_c[i];
    am += s_m[i];
  }
  __syncthreads();
  c += ac;
  m += am;
}

// ---- per-sequence choice state, stored between launches
struct Choice {
  uint32_t prefix;    // key bits fixed so far
  uint32_t k_rem;     // tokens still to take, by count
  uint64_t m_rem;     // mass still to reach
  uint64_t m_above;   // mass of the tokens already known to be kept
};
static_assert(sizeof(Choice) == kSampleChoiceBytes, "choice record size");

__device__ __forceinline__ Choice* choices(const SampleWs& w) { return (Choice*)w.choice; }

// The first-level histogram of sequence b.
__device__ __forceinline__ size_t hist_at(int b) { return (size_t)b * kBuckets; }

// A thread's share of a histogram for choose(): the kBuckets / NT buckets
// from top = 2047 - (kBuckets / NT) t downwards, loaded together.
template <int NT>
struct HistPartT {
  static constexpr int P = kBuckets / NT;
  uint32_t cnt[P];
  uint64_t mass[P];
};
using HistPart = HistPartT<kSThreads>;

template <int NT>
__device__ __forceinline__ void load_hist_part(const uint32_t* cnt, const uint64_t* mass, HistPartT<NT>& h) {
  constexpr int P = HistPartT<NT>::P;
  const int top = kBuckets - 1 - P * (int)threadIdx.x;
#pragma unroll
  for (int i = 0; i < P; ++i) {
    h.cnt[i] = cnt[top - i];
    h.mass[i] = mass[top - i];
  }
}

// A choice and the count and mass of the bucket it took.
struct Chosen {
  Choice c;
  uint32_t n;
  uint64_t f;
};

// Scan a histogram from the top bucket down for the first bucket where the
// count reaches k_rem or the mass reaches m_rem; update the choice.  Every
// thread of the workgroup calls it with its HistPart and gets the same
// result.
template <int NT>
__device__ __forceinline__ Chosen choose(const HistPartT<NT>& h, Choice c, int bits) {
  constexpr int kPer = HistPartT<NT>::P;
  __shared__ Chosen s_out;
  const int t = threadIdx.x;
  const int top = kBuckets - 1 - kPer * t;
  if (t == 0) {  // replaced below; kept only if no bucket qualifies
    s_out.c = c;
    s_out.n = 0u;
    s_out.f = 0ull;
  }
  uint32_t lc = 0;
  uint64_t lm = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    lc += h.cnt[i];
    lm += h.mass[i];
  }
  // inclusive scans over threads (thread order = descending buckets)
  uint32_t inc_c = lc;
  uint64_t inc_m = lm;
  wg_scan2<NT>(inc_c, inc_m);
  const uint32_t exc_c = inc_c - lc;
  const uint64_t exc_m = inc_m - lm;
  const bool before = exc_c >= c.k_rem || exc_m >= c.m_rem;
  const bool after = inc_c >= c.k_rem || inc_m >= c.m_rem;
  if (!before && after) {
    // unrolled with constant indices, so the thread's part stays in
    // registers
    uint32_t cc = exc_c;
    uint64_t cm = exc_m;
    bool found = false;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (!found && (cc + h.cnt[i] >= c.k_rem || cm + h.mass[i] >= c.m_rem)) {
        Chosen o;
        o.c.prefix = (c.prefix << bits) | (uint32_t)(top - i);
        o.c.k_rem = c.k_rem - cc;
        o.c.m_rem = c.m_rem - cm;
        o.c.m_above = c.m_above + cm;
        o.n = h.cnt[i];
        o.f = h.mass[i];
        s_out = o;
        found = true;
      }
      cc += h.cnt[i];
      cm += h.mass[i];
    }
  }
  __syncthreads();
  const Chosen o = s_out;
  __syncthreads();
  return o;
}

// The sequence's maximum logit from K0's chunk maxima (W <= 64): wmax_ld is
// thread t's chunk maximum (t < 64), loaded with the first batch.
__device__ __forceinline__ float load_wmax(const SArgs& a, int b) {
  const int t = threadIdx.x;
  return t < 64 && t < a.W ? a.w.wmax[(size_t)b * a.W + t] : -INFINITY;
}
__device__ float seq_max(float wmax_ld) {
  __shared__ float s_res;
  const int t = threadIdx.x;
  if (t < 64) {
    float m = wmax_ld;
    m = wave_max(m);
    if (t == 0) s_res = m;
  }
  __syncthreads();
  return s_res;
}

// The sequence's normaliser from K1's per-chunk parts (W <= 64), part =
// thread t's part (t < 64): an integer sum, the same in any order.
__device__ uint64_t seq_sum(uint64_t part) {
  __shared__ uint64_t s_res;
  const int t = threadIdx.x;
  if (t < 64) {
    uint64_t v = part;
    v = wave_sum(v);
    if (t == 0) s_res = v;
  }
  __syncthreads();
  return s_res;
}

// Histogram of one level over a chunk into LDS, then added to the sequence's
// global histogram (integer atomics: order-independent).  v holds the
// thread's first batch (elements ch.e0 + t + 256 i), already in flight.
__device__ void histogram(const Chunk& ch, float (&v)[kSBatch], int level, uint32_t prefix, float m,
                          float c, bool counts, uint32_t* gcnt, uint64_t* gmass, uint64_t* gsum) {
  __shared__ uint32_t h_cnt[kBuckets];
  __shared__ uint64_t h_mass[kBuckets];
  __shared__ uint64_t h_sum[kSThreads / 64];
  const int t = threadIdx.x;
  for (int i = t; i < kBuckets; i += kSThreads) {
    h_cnt[i] = 0u;
    h_mass[i] = 0ull;
  }
  __syncthreads();
  uint64_t ls = 0;
  for (int e0 = ch.e0 + t;;) {
#pragma unroll
    for (int i = 0; i < kSBatch; ++i) {
      if (e0 + i * kSThreads >= ch.e1) break;
      const float l = v[i];
      const uint32_t key = skey(l);
      const uint64_t f = fixed_mass(l, m, c);
      ls += f;
      if (in_prefix(key, level, prefix)) {
        const int d = digit(key, level);
        if (counts) atomicAdd(&h_cnt[d], 1u);
        atomicAdd((unsigned long long*)&h_mass[d], (unsigned long long)f);
      }
    }
    e0 += kSBatch * kSThreads;
    if (e0 >= ch.e1) break;
    load_batch(ch, e0, v);
  }
  // the chunk's part of the normaliser: a wave sum, then the 4 waves' in
  // order, stored in the chunk's own slot (no atomics on one shared word)
  if (gsum) {
    ls = wave_sum(ls);
    if ((t & 63) == 0) h_sum[t >> 6] = ls;
  }
  __syncthreads();
  for (int i = t; i < kBuckets; i += kSThreads) {
    if (h_cnt[i]) atomicAdd(&gcnt[i], h_cnt[i]);
    if (h_mass[i]) atomicAdd((unsigned long long*)&gmass[i], (unsigned long long)h_mass[i]);
  }
  if (gsum && t == 0) {
    uint64_t v = 0;
    for (int i = 0; i < kSThreads / 64; ++i) v += h_sum[i];
    *gsum = v;
  }
}

__global__ __launch_bounds__(kSThreads) void sample_k0(const SArgs a) {
  __shared__ float red[kSThreads / 64];
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const Chunk ch = chunk_of(a, b, w);
  float m = -INFINITY;
  for (int e0 = ch.e0 + t; e0 < ch.e1; e0 += kSBatch * kSThreads) {
    float v[kSBatch];
    load_batch(ch, e0, v);
#pragma unroll
    for (int i = 0; i < kSBatch; ++i) m = fmaxf(m, v[i]);
  }
  m = wave_max(m);
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  if (t == 0) {
    float r = red[0];
    for (int i = 1; i < kSThreads / 64; ++i) r = fmaxf(r, red[i]);
    a.w.wmax[(size_t)b * a.W + w] = r;
  }
  clear_words(a.w.cnt + hist_at(b), kBuckets, w, a.W);
  clear_words((uint32_t*)(a.w.mass + hist_at(b)), 2 * kBuckets, w, a.W);
}

__global__ __launch_bounds__(kSThreads) void sample_k1(const SArgs a) {
  const int b = blockIdx.y, w = blockIdx.x;
  const Chunk ch = chunk_of(a, b, w);
  float v[kSBatch];
  load_batch(ch, ch.e0 + (int)threadIdx.x, v);
  const float wm = load_wmax(a, b);
  const float c = inv_temp(a, b);
  __builtin_amdgcn_sched_barrier(0);
  const float m = seq_max(wm);
  histogram(ch, v, 0, 0u, m, c, !mass_only(a, b), a.w.cnt + hist_at(b), a.w.mass + hist_at(b),
            a.w.sum + (size_t)b * a.W + w);
}

// The choice before level 0: the count and mass budgets of the nucleus.
// sum: the sequence's normaliser (fixed point).
__device__ Choice initial_choice(const SArgs& a, int b, uint64_t sum) {
  Choice c;
  c.prefix = 0u;
  c.m_above = 0ull;
  const bool greedy = !(a.temperature[b] > 0.f);
  const int k = a.top_k[b];
  c.k_rem = greedy ? 1u : (k > 0 && k < a.V ? (uint32_t)k : (uint32_t)a.V);
  const float p = a.top_p[b];
  if (greedy || p >= 1.f) {
    c.m_rem = ~0ull;
  } else {
    const double target = ceil((double)(p > 0.f ? p : 0.f) * (double)sum);
    c.m_rem = target < 1.0 ? 1ull : (uint64_t)target;
  }
  return c;
}

// The logit an order-preserving key was made from (-0 comes back as +0,
// an equal logit of the same mass).
__device__ __forceinline__ float key_logit(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// K2: the first-level choice; this chunk's mass above the chosen bucket
// and its tokens inside the bucket (its candidates), both stored for K3:
// the candidates in the chunk's own segment of the sequence's list, with
// their number.
__global__ __launch_bounds__(kSThreads) void sample_k2(const SArgs a) {
  __shared__ uint64_t s_m[kSThreads / 64];
  __shared__ uint32_t s_tot;
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const Chunk ch = chunk_of(a, b, w);
  float v[kSBatch];
  load_batch(ch, ch.e0 + t, v);
  const float wm = load_wmax(a, b);
  HistPart hp;
  load_hist_part(a.w.cnt + hist_at(b), a.w.mass + hist_at(b), hp);
  const uint64_t sum_part = t < 64 && t < a.W ? a.w.sum[(size_t)b * a.W + t] : 0ull;
  const float c = inv_temp(a, b);
  __builtin_amdgcn_sched_barrier(0);
  const float m = seq_max(wm);
  const uint64_t sum = seq_sum(sum_part);
  const Choice c1 = choose<kSThreads>(hp, initial_choice(a, b, sum), 11).c;
  if (w == 0 && t == 0) choices(a.w)[b] = c1;
  uint32_t* seg = a.w.cand + 2 * ((size_t)b * a.W + w) * a.chunk;
  uint32_t nseg = 0;
  uint64_t above = 0;
  // batches start at the same element offset in every thread, so every
  // thread takes the same number of trips through the scan's barriers
  for (int base = ch.e0;;) {
    const int e0 = base + t;
    uint32_t mine = 0;  // bit i: element e0 + 256 i is a candidate
#pragma unroll
    for (int i = 0; i < kSBatch; ++i) {
      if (e0 + i * kSThreads < ch.e1) {
        const uint32_t top = skey(v[i]) >> 21;
        if (top > c1.prefix) above += fixed_mass(v[i], m, c);
        mine |= (top == c1.prefix ? 1u : 0u) << i;
      }
    }
    const uint32_t n = (uint32_t)__builtin_popcount(mine);
    const uint32_t inc = wg_scan(n);
    uint32_t slot = nseg + inc - n;
#pragma unroll
    for (int i = 0; i < kSBatch; ++i) {
      if (((mine >> i) & 1u) && slot < (uint32_t)a.chunk) {  // (a chunk's tokens fit its segment)
        *(uint2*)(seg + 2 * (size_t)slot) = make_uint2(skey(v[i]), (uint32_t)(e0 + i * kSThreads));
        ++slot;
      }
    }
    if (t == kSThreads - 1) s_tot = inc;
    __syncthreads();
    nseg += s_tot;
    base += kSBatch * kSThreads;
    if (base >= ch.e1) break;
    __syncthreads();  // s_tot is rewritten by the next batch
    load_batch(ch, base + t, v);
  }
  above = wave_sum(above);
  if ((t & 63) == 0) s_m[t >> 6] = above;
  __syncthreads();
  if (t == 0) {
    uint64_t sm = 0;
    for (int i = 0; i < kSThreads / 64; ++i) sm += s_m[i];
    a.w.wmass[(size_t)b * a.W + w] = sm;
    a.w.ncand[(size_t)b * a.W + w] = min(nseg, (uint32_t)a.chunk);
  }
}

// The nucleus, final: every token with key > tau, and the first `ties`
// tokens (vocabulary order) with key == tau, each of mass f_tau.
struct Nucleus {
  uint32_t tau, ties;
  uint64_t f_tau, m_above;
};

// The last level's choice (hp: the thread's part of the last level's
// histogram, prev: the choice before it) as the final nucleus.
template <int NT>
__device__ __forceinline__ Nucleus nucleus(const HistPartT<NT>& hp, const Choice& prev) {
  const Chosen ch3 = choose<NT>(hp, prev, 10);
  const Choice& c3 = ch3.c;
  const uint32_t n = ch3.n;
  const uint64_t f = n ? ch3.f / n : 0ull;  // equal keys, equal masses
  uint32_t t = c3.k_rem;
  if (f > 0 && c3.m_rem <= ch3.f) {
    const uint64_t need = (c3.m_rem + f - 1) / f;
    t = need < t ? (uint32_t)need : t;
  }
  Nucleus r;
  r.tau = c3.prefix;
  r.ties = t < n ? t : n;
  r.f_tau = f;
  r.m_above = c3.m_above;
  return r;
}

// A sequence's candidates as K3 sees them: the list is the chunks'
// segments one after another (entry j lies in the segment s with off[s] <=
// j < off[s + 1]).  Thread t holds the q consecutive entries from j0 = t q
// in registers, loaded once; a list longer than 256 kCandRegs entries has
// its remainder read again, in batches, by every pass that walks it.
constexpr int kCandRegs = 8;
struct CandList {
  const uint32_t* p;    // the sequence's segments, [W][chunk][2] (key, index)
  const uint32_t* off;  // LDS: segment starts, off[W] = n
  int W, chunk;
  uint32_t n, q, j0;
  uint32_t key[kCandRegs], idx[kCandRegs];
};

// The segment holding entry j < n: the last s with off[s] <= j.
__device__ __forceinline__ int seg_of(const CandList& L, uint32_t j) {
  int s = 0;
#pragma unroll
  for (int step = 32; step > 0; step >>= 1)
    if (s + step < L.W && L.off[s + step] <= j) s += step;
  return s;
}

__device__ __forceinline__ uint2 cand_entry(const CandList& L, int s, uint32_t j) {
  return *(const uint2*)(L.p + 2 * ((size_t)s * L.chunk + (j - L.off[s])));
}

__device__ __forceinline__ void load_cands(CandList& L) {
  const uint32_t t = threadIdx.x;
  L.q = (L.n + kFThreads - 1) / kFThreads;
  if (L.q > (uint32_t)kCandRegs) L.q = kCandRegs;
  L.j0 = t * L.q;
  int s = L.j0 < L.n ? seg_of(L, L.j0) : 0;
  uint32_t next = L.off[s + 1];  // where segment s ends
#pragma unroll
  for (int i = 0; i < kCandRegs; ++i) {
    const uint32_t j = L.j0 + (uint32_t)i;
    L.key[i] = 0u;
    L.idx[i] = 0u;
    if ((uint32_t)i < L.q && j < L.n) {
      while (next <= j) next = L.off[++s + 1];  // skips empty segments
      const uint2 e = cand_entry(L, s, j);
      L.key[i] = e.x;
      L.idx[i] = e.y;
    }
  }
}

// The chunk of vocabulary index idx (chunks of `chunk` logits; inv =
// 1 / chunk): a double-precision estimate, off by at most one, corrected.
__device__ __forceinline__ int chunk_index(uint32_t idx, uint32_t chunk, double inv) {
  int w = (int)((double)idx * inv);
  if ((uint32_t)(w + 1) * chunk <= idx)
    ++w;
  else if ((uint32_t)w * chunk > idx)
    --w;
  return w;
}

// Calls f(key, index) for each of this thread's candidates.
template <typename F>
__device__ __forceinline__ void each_cand(const CandList& L, F f) {
  const uint32_t t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kCandRegs; ++i)
    if ((uint32_t)i < L.q && L.j0 + (uint32_t)i < L.n) f(L.key[i], L.idx[i]);
  for (uint32_t b0 = (uint32_t)kCandRegs * kFThreads; b0 < L.n; b0 += (uint32_t)kSBatch * kFThreads) {
    uint2 e[kSBatch];
#pragma unroll
    for (int i = 0; i < kSBatch; ++i) {
      const uint32_t j = b0 + t + (uint32_t)i * kFThreads;
      e[i] = j < L.n ? cand_entry(L, seg_of(L, j), j) : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < kSBatch; ++i)
      if (b0 + t + (uint32_t)i * kFThreads < L.n) f(e[i].x, e[i].y);
  }
}

// A histogram of one level over the candidates whose key agrees with
// `prefix` above the level's digit, in LDS (zeroed by the caller), then the
// thread's part of it for choose().
__device__ __forceinline__ void cand_level(const CandList& L, int level, uint32_t prefix, float m, float c, bool counts,
                           uint32_t* h_cnt, uint64_t* h_mass, HistPartT<kFThreads>& hp) {
  each_cand(L, [&](uint32_t key, uint32_t) {
    if (in_prefix(key, level, prefix)) {
      const int d = digit(key, level);
      if (counts) atomicAdd(&h_cnt[d], 1u);
      atomicAdd((unsigned long long*)&h_mass[d], (unsigned long long)fixed_mass(key_logit(key), m, c));
    }
  });
  __syncthreads();
  load_hist_part(h_cnt, h_mass, hp);
}

__device__ __forceinline__ void zero_hist(uint32_t* h_cnt, uint64_t* h_mass) {
  for (int i = threadIdx.x; i < kBuckets; i += kFThreads) {
    h_cnt[i] = 0u;
    h_mass[i] = 0ull;
  }
}

// Thread t's E consecutive elements of the chunk from e0 + t E, when E <=
// kSBatch: 16-byte loads where the row is 16-byte aligned (the first is a
// multiple of 4: chunks are multiples of 1024 and E of 4); otherwise, and
// for the vocabulary's last partial quad, element by element.
__device__ __forceinline__ void load_run(const Chunk& ch, float (&v)[kSBatch]) {
  const int base = ch.e0 + (int)threadIdx.x * ch.E;
  const int end = min(base + ch.E, ch.e1);
  const bool vec = ((uintptr_t)ch.row & 15u) == 0;
#pragma unroll
  for (int i = 0; i < kSBatch; i += 4) {
    if (vec && base + i + 3 < end) {
      const float4 q = *(const float4*)(ch.row + base + i);
      v[i] = q.x;
      v[i + 1] = q.y;
      v[i + 2] = q.z;
      v[i + 3] = q.w;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[i + j] = base + i + j < end ? ch.row[base + i + j] : -INFINITY;
    }
  }
}

// The draw inside chunk ch of sequence b, which holds it: r in [before,
// before + the chunk's kept mass); ties_before = ties (key == tau) in the
// chunks before; v = load_run(ch) when E <= kSBatch.  The chunk's kept
// tokens are walked in vocabulary order, thread by thread (thread t takes
// the E consecutive elements from e0 + t E), then element by element, until
// their cumulative mass exceeds r.
__device__ __forceinline__ void draw_in_chunk(const SArgs& a, int b, const Chunk& ch, const Nucleus& nu, uint64_t before,
                              uint32_t ties_before, uint64_t r, float m, float c, const float (&v)[kSBatch]) {
  const int t = threadIdx.x;
  const int base = ch.e0 + t * ch.E;
  const int end = min(base + ch.E, ch.e1);
  const bool in_regs = ch.E <= kSBatch;
  // element j of this thread (vocabulary order), from registers or reloaded
  auto elem = [&](int j) -> float {
    if (in_regs) {
      float x = -INFINITY;
#pragma unroll
      for (int i = 0; i < kSBatch; ++i) x = i == j ? v[i] : x;
      return x;
    }
    return ch.row[base + j];
  };
  const int n_el = end - base;  // may be <= 0 past the vocabulary
  // this thread's ties (key == tau), scanned over the threads in vocabulary
  // order: which of them are kept depends on the ties before it
  uint32_t lt = 0;
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kSBatch; ++i) lt += i < n_el && skey(v[i]) == nu.tau;
  } else {
    for (int j = 0; j < n_el; ++j) lt += skey(ch.row[base + j]) == nu.tau;
  }
  const uint32_t lt_inc = wg_scan<uint32_t, kFThreads>(lt);
  const uint32_t tb = ties_before + lt_inc - lt;
  // mass of element l (in vocabulary order within the thread): kept ties
  // are counted by tk
  auto kept_mass = [&](float l, uint32_t& tk) -> uint64_t {
    const uint32_t key = skey(l);
    if (key == nu.tau) return (tb + tk++ < nu.ties) ? nu.f_tau : 0ull;
    return key > nu.tau ? fixed_mass(l, m, c) : 0ull;
  };
  uint64_t km = 0;
  uint32_t tk = 0;
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kSBatch; ++i)
      if (i < n_el) km += kept_mass(v[i], tk);
  } else {
    for (int j = 0; j < n_el; ++j) km += kept_mass(ch.row[base + j], tk);
  }
  const uint64_t excl = before + wg_scan<uint64_t, kFThreads>(km) - km;
  if (!(r >= excl && r < excl + km)) return;
  uint64_t acc = excl;
  tk = 0;
  for (int j = 0; j < n_el; ++j) {
    acc += kept_mass(elem(j), tk);
    if (acc > r) {
      a.tokens[b] = base + j;
      return;
    }
  }
}

// K3, one workgroup per sequence: the second and third levels over the
// candidates, the nucleus, each chunk's kept mass (K2's mass above the
// bucket, the candidates above the threshold key, its kept ties in chunk
// order), then r = floor(u * S_kept) and the draw in the chunk holding r.
__global__ __launch_bounds__(kFThreads) void sample_k3(const SArgs a) {
  __shared__ uint32_t h_cnt[kBuckets];
  __shared__ uint64_t h_mass[kBuckets];
  __shared__ uint32_t s_off[65];
  __shared__ uint64_t s_km[64];  // per chunk: candidates' mass above tau, then the chunk's kept mass
  __shared__ uint32_t s_kt[64];  // per chunk: ties (key == tau)
  const int b = blockIdx.x, t = threadIdx.x;
  const uint32_t n_seg = t < a.W ? a.w.ncand[(size_t)b * a.W + t] : 0u;
  const Choice c1 = choices(a.w)[b];
  const float wm = load_wmax(a, b);
  const uint64_t above = t < 64 && t < a.W ? a.w.wmass[(size_t)b * a.W + t] : 0ull;
  const float c = inv_temp(a, b);
  __builtin_amdgcn_sched_barrier(0);
  zero_hist(h_cnt, h_mass);
  if (t < 64) {
    // the segment starts: an inclusive scan of the counts over wave 0
    s_off[t + 1] = wave_scan(n_seg);
    if (t == 0) s_off[0] = 0u;
    s_km[t] = 0ull;
    s_kt[t] = 0u;
  }
  const float m = seq_max(wm);  // (its barrier also publishes the LDS above)
  CandList L;
  L.p = a.w.cand + 2 * (size_t)b * a.W * a.chunk;
  L.off = s_off;
  L.W = a.W;
  L.chunk = a.chunk;
  L.n = s_off[a.W];
  load_cands(L);
  HistPartT<kFThreads> hp;
  cand_level(L, 1, c1.prefix, m, c, !mass_only(a, b), h_cnt, h_mass, hp);
  const Choice c2 = choose<kFThreads>(hp, c1, 11).c;  // (its barriers end every thread's reads of hp)
  zero_hist(h_cnt, h_mass);
  __syncthreads();
  cand_level(L, 2, c2.prefix, m, c, true, h_cnt, h_mass, hp);
  const Nucleus nu = nucleus<kFThreads>(hp, c2);
  // the candidates' share of each chunk's kept mass, and each chunk's ties:
  // a thread's entries run through few segments, so it adds per run
  const double inv_chunk = 1.0 / (double)a.chunk;
  int cur = -1;
  uint64_t run_m = 0;
  uint32_t run_t = 0;
  auto flush = [&]() {
    if (cur >= 0) {
      if (run_m) atomicAdd((unsigned long long*)&s_km[cur], (unsigned long long)run_m);
      if (run_t) atomicAdd(&s_kt[cur], run_t);
    }
  };
  each_cand(L, [&](uint32_t key, uint32_t idx) {
    const int w = chunk_index(idx, (uint32_t)a.chunk, inv_chunk);
    if (w != cur) {
      flush();
      cur = w;
      run_m = 0;
      run_t = 0;
    }
    if (key > nu.tau)
      run_m += fixed_mass(key_logit(key), m, c);
    else if (key == nu.tau)
      ++run_t;
  });
  flush();
  __syncthreads();
  // wave 0, lane i = chunk i: the chunk's kept mass (it keeps its ties
  // while the ties of the chunks before it number fewer than nu.ties),
  // inclusive scans over the chunks, r = floor(u * S_kept), and the chunk
  // holding r
  __shared__ int s_draw;
  __shared__ uint64_t s_before, s_r;
  __shared__ uint32_t s_ties_before;
  if (t < 64) {
    const uint32_t ti = t < a.W ? s_kt[t] : 0u;
    const uint32_t texc = wave_scan(ti) - ti;
    const uint32_t kt = texc >= nu.ties ? 0u : min(ti, nu.ties - texc);
    const uint64_t km = (t < a.W ? s_km[t] + above : 0ull) + (uint64_t)kt * nu.f_tau;
    const uint64_t kinc = wave_scan(km);
    const uint64_t total = lane63(kinc);
    const float uu = fminf(fmaxf(a.u[b], 0.f), 1.f);
    uint64_t r = (uint64_t)floor((double)uu * (double)total);
    if (r >= total) r = total - 1;
    const uint64_t kexc = kinc - km;
    const bool here = r >= kexc && r < kinc;  // at most one lane
    const uint64_t hit = __ballot(here);
    if (t == 0) s_draw = hit ? __builtin_ctzll(hit) : -1;
    if (here) {
      s_before = kexc;
      s_ties_before = texc;
    }
    if (t == 0) s_r = r;
  }
  __syncthreads();
  const int wd = s_draw;
  if (wd < 0) return;  // nothing kept (every logit -inf): no draw
  const Chunk ch = chunk_of<kFThreads>(a, b, wd);
  float v[kSBatch];
  if (ch.E <= kSBatch) load_run(ch, v);
  draw_in_chunk(a, b, ch, nu, s_before, s_ties_before, s_r, m, c, v);
}

}  // namespace

SampleWs sample_ws_carve(void* base, int B, int W, int chunk) {
  SampleWs w{};
  const uintptr_t p = (uintptr_t)base;
  size_t off = kWsHeaderBytes;  // the header every workspace keeps
  auto take = [&](size_t bytes) { const size_t at = off; off = align256(off + bytes); return (void*)(p + at); };
  w.cnt = (uint32_t*)take(sizeof(uint32_t) * (size_t)B * kBuckets);
  w.mass = (uint64_t*)take(sizeof(uint64_t) * (size_t)B * kBuckets);
  w.sum = (uint64_t*)take(sizeof(uint64_t) * (size_t)B * W);
  w.choice = (void*)take((size_t)kSampleChoiceBytes * B);
  w.wmax = (float*)take(sizeof(float) * (size_t)B * W);
  w.wmass = (uint64_t*)take(sizeof(uint64_t) * (size_t)B * W);
  w.ncand = (uint32_t*)take(sizeof(uint32_t) * (size_t)B * W);
  w.cand = (uint32_t*)take(2 * sizeof(uint32_t) * (size_t)B * W * chunk);
  w.bytes = off;
  return w;
}

int sample_chunks(int B, int V, int* chunk) {
  int W = (512 + B - 1) / B;
  if (W > 64) W = 64;
  if (W < 1) W = 1;
  int ch = (V + W - 1) / W;
  ch = (ch + 1023) / 1024 * 1024;
  *chunk = ch;
  return (V + ch - 1) / ch;
}

hipError_t launch_sample(const float* logits, int B, int V, const float* temperature,
                         const float* top_p, const int32_t* top_k, const float* u, int32_t* tokens,
                         const SampleWs& ws, int W, int chunk, hipStream_t st) {
  SArgs a{};
  a.logits = logits;
  a.B = B;
  a.V = V;
  a.temperature = temperature;
  a.top_p = top_p;
  a.top_k = top_k;
  a.u = u;
  a.tokens = tokens;
  a.w = ws;
  a.W = W;
  a.chunk = chunk;
  const dim3 grid(W, B);
  sample_k0<<<grid, kSThreads, 0, st>>>(a);
  sample_k1<<<grid, kSThreads, 0, st>>>(a);
  sample_k2<<<grid, kSThreads, 0, st>>>(a);
  sample_k3<<<B, kFThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace pkv
