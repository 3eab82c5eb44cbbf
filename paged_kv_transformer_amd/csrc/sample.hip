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
// workgroup per sequence would leave most of the chip idle).  Workgroups
// never wait on each other; the six launches are:
//   K0 chunk maxima                       (and clears the level-1 sums)
//   K1 normaliser + level-1 histogram     (clears level 2)
//   K2 level-1 choice + level-2 histogram (clears level 3)
//   K3 level-2 choice + level-3 histogram
//   K4 level-3 choice (threshold key, ties kept) + per-chunk kept mass
//   K5 the draw: the chunk holding u, then the token inside it
// Each choice is made by every workgroup alike and stored by workgroup 0 of
// the sequence for the next launch.
#include "pkv_dev.h"

namespace pkv {
namespace {

constexpr int kSThreads = 256;
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

__device__ __forceinline__ Chunk chunk_of(const SArgs& a, int b, int w) {
  Chunk c;
  c.row = a.logits + (size_t)b * a.V;
  c.e0 = w * a.chunk;
  c.e1 = min(a.V, c.e0 + a.chunk);
  c.E = a.chunk / kSThreads;
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

// Inclusive scan over the workgroup's threads in thread order: within a
// wave by shuffles, then the sums of the waves before (one barrier pair).
template <typename T>
__device__ __forceinline__ T wg_scan(T v) {
  __shared__ T s_wave[kSThreads / 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  if (lane == 63) s_wave[wv] = v;
  __syncthreads();
  T add = 0;
  for (int i = 0; i < wv; ++i) add += s_wave[i];
  __syncthreads();
  return v + add;
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

// Level L's global histogram of sequence b.
__device__ __forceinline__ size_t hist_at(int b, int level) { return ((size_t)b * 3 + level) * kBuckets; }

// A thread's share of a histogram for choose(): the 8 buckets from
// top = 2047 - 8t downwards, loaded together.
constexpr int kPer = kBuckets / kSThreads;
struct HistPart {
  uint32_t cnt[kPer];
  uint64_t mass[kPer];
};

__device__ __forceinline__ void load_hist_part(const uint32_t* cnt, const uint64_t* mass, HistPart& h) {
  const int top = kBuckets - 1 - kPer * (int)threadIdx.x;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
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
__device__ Chosen choose(const HistPart& h, Choice c, int bits) {
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
  const uint32_t inc_c = wg_scan(lc);
  const uint64_t inc_m = wg_scan(lm);
  const uint32_t exc_c = inc_c - lc;
  const uint64_t exc_m = inc_m - lm;
  const bool before = exc_c >= c.k_rem || exc_m >= c.m_rem;
  const bool after = inc_c >= c.k_rem || inc_m >= c.m_rem;
  if (!before && after) {
    uint32_t cc = exc_c;
    uint64_t cm = exc_m;
    for (int i = 0; i < kPer; ++i) {
      if (cc + h.cnt[i] >= c.k_rem || cm + h.mass[i] >= c.m_rem) {
        Chosen o;
        o.c.prefix = (c.prefix << bits) | (uint32_t)(top - i);
        o.c.k_rem = c.k_rem - cc;
        o.c.m_rem = c.m_rem - cm;
        o.c.m_above = c.m_above + cm;
        o.n = h.cnt[i];
        o.f = h.mass[i];
        s_out = o;
        break;
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
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
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
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
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
    for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
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
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((t & 63) == 0) red[t >> 6] = m;
  __syncthreads();
  if (t == 0) {
    float r = red[0];
    for (int i = 1; i < kSThreads / 64; ++i) r = fmaxf(r, red[i]);
    a.w.wmax[(size_t)b * a.W + w] = r;
  }
  clear_words((uint32_t*)(a.w.cnt + hist_at(b, 0)), kBuckets, w, a.W);
  clear_words((uint32_t*)(a.w.mass + hist_at(b, 0)), 2 * kBuckets, w, a.W);
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
  histogram(ch, v, 0, 0u, m, c, !mass_only(a, b), a.w.cnt + hist_at(b, 0), a.w.mass + hist_at(b, 0),
            a.w.sum + (size_t)b * a.W + w);
  clear_words((uint32_t*)(a.w.cnt + hist_at(b, 1)), kBuckets, w, a.W);
  clear_words((uint32_t*)(a.w.mass + hist_at(b, 1)), 2 * kBuckets, w, a.W);
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

__global__ __launch_bounds__(kSThreads) void sample_k2(const SArgs a) {
  const int b = blockIdx.y, w = blockIdx.x;
  const Chunk ch = chunk_of(a, b, w);
  float v[kSBatch];
  load_batch(ch, ch.e0 + (int)threadIdx.x, v);
  const float wm = load_wmax(a, b);
  HistPart hp;
  load_hist_part(a.w.cnt + hist_at(b, 0), a.w.mass + hist_at(b, 0), hp);
  const int t = threadIdx.x;
  const uint64_t sum_part = t < 64 && t < a.W ? a.w.sum[(size_t)b * a.W + t] : 0ull;
  const float c = inv_temp(a, b);
  __builtin_amdgcn_sched_barrier(0);
  const float m = seq_max(wm);
  const uint64_t sum = seq_sum(sum_part);
  const Choice c1 = choose(hp, initial_choice(a, b, sum), 11).c;
  if (w == 0 && threadIdx.x == 0) choices(a.w)[b] = c1;
  histogram(ch, v, 1, c1.prefix, m, c, !mass_only(a, b), a.w.cnt + hist_at(b, 1),
            a.w.mass + hist_at(b, 1), nullptr);
  clear_words((uint32_t*)(a.w.cnt + hist_at(b, 2)), kBuckets, w, a.W);
  clear_words((uint32_t*)(a.w.mass + hist_at(b, 2)), 2 * kBuckets, w, a.W);
}

__global__ __launch_bounds__(kSThreads) void sample_k3(const SArgs a) {
  const int b = blockIdx.y, w = blockIdx.x;
  const Chunk ch = chunk_of(a, b, w);
  float v[kSBatch];
  load_batch(ch, ch.e0 + (int)threadIdx.x, v);
  const float wm = load_wmax(a, b);
  HistPart hp;
  load_hist_part(a.w.cnt + hist_at(b, 1), a.w.mass + hist_at(b, 1), hp);
  const Choice prev = choices(a.w)[b];
  const float c = inv_temp(a, b);
  __builtin_amdgcn_sched_barrier(0);
  const float m = seq_max(wm);
  const Choice c2 = choose(hp, prev, 11).c;
  if (w == 0 && threadIdx.x == 0) choices(a.w)[a.B + b] = c2;
  histogram(ch, v, 2, c2.prefix, m, c, true, a.w.cnt + hist_at(b, 2),
            a.w.mass + hist_at(b, 2), nullptr);
}

// The nucleus, final: every token with key > tau, and the first `ties`
// tokens (vocabulary order) with key == tau, each of mass f_tau.
struct Nucleus {
  uint32_t tau, ties;
  uint64_t f_tau, m_above;
};
static_assert(sizeof(Nucleus) <= kSampleChoiceBytes, "nucleus record size");

// K4 stores each sequence's nucleus for K5, in the third third of the
// choice records ([3][B] records of kSampleChoiceBytes).
__device__ __forceinline__ Nucleus* nuclei(const SampleWs& w, int B) {
  return (Nucleus*)((char*)w.choice + (size_t)2 * B * kSampleChoiceBytes);
}

// The level-3 choice (hp: the thread's part of the level-3 histogram,
// prev: the choice after level 2) as the final nucleus.
__device__ Nucleus nucleus(const HistPart& hp, const Choice& prev) {
  const Chosen ch3 = choose(hp, prev, 10);
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

// K4: per chunk, the mass of its tokens above tau and its count of ties.
__global__ __launch_bounds__(kSThreads) void sample_k4(const SArgs a) {
  __shared__ uint64_t s_m[kSThreads / 64];
  __shared__ uint32_t s_t[kSThreads / 64];
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const Chunk ch = chunk_of(a, b, w);
  float v[kSBatch];
  load_batch(ch, ch.e0 + t, v);
  const float wm = load_wmax(a, b);
  HistPart hp;
  load_hist_part(a.w.cnt + hist_at(b, 2), a.w.mass + hist_at(b, 2), hp);
  const Choice prev = choices(a.w)[a.B + b];
  const float c = inv_temp(a, b);
  __builtin_amdgcn_sched_barrier(0);
  const float m = seq_max(wm);
  const Nucleus nu = nucleus(hp, prev);
  if (w == 0 && t == 0) nuclei(a.w, a.B)[b] = nu;
  uint64_t mg = 0;
  uint32_t ties = 0;
  for (int e0 = ch.e0 + t;;) {
#pragma unroll
    for (int i = 0; i < kSBatch; ++i) {
      if (e0 + i * kSThreads >= ch.e1) break;
      const uint32_t key = skey(v[i]);
      if (key > nu.tau) mg += fixed_mass(v[i], m, c);
      ties += key == nu.tau;
    }
    e0 += kSBatch * kSThreads;
    if (e0 >= ch.e1) break;
    load_batch(ch, e0, v);
  }
  for (int o = 32; o > 0; o >>= 1) {
    mg += __shfl_xor(mg, o);
    ties += __shfl_xor(ties, o);
  }
  if ((t & 63) == 0) {
    s_m[t >> 6] = mg;
    s_t[t >> 6] = ties;
  }
  __syncthreads();
  if (t == 0) {
    uint64_t sm = 0;
    uint32_t st = 0;
    for (int i = 0; i < kSThreads / 64; ++i) {
      sm += s_m[i];
      st += s_t[i];
    }
    a.w.wmass[(size_t)b * a.W + w] = sm;
    a.w.wties[(size_t)b * a.W + w] = st;
  }
}

// K5: the draw.  r = floor(u * S_kept); the kept tokens in vocabulary order
// are walked chunk by chunk, then thread by thread, then element by element
// until their cumulative mass exceeds r.  Every workgroup loads its own
// elements with the per-chunk records (most of them then find that the draw
// is elsewhere and exit), so the one that holds the draw has its data in
// registers when it learns so.
__global__ __launch_bounds__(kSThreads) void sample_k5(const SArgs a) {
  const int b = blockIdx.y, w = blockIdx.x, t = threadIdx.x;
  const Chunk ch = chunk_of(a, b, w);
  // this thread's elements in vocabulary order: [base, end)
  const int base = ch.e0 + t * ch.E;
  const int end = min(base + ch.E, ch.e1);
  const bool in_regs = ch.E <= kSBatch;
  float v[kSBatch];
  if (in_regs) {
    // 16-byte loads where the row is 16-byte aligned (base is a multiple
    // of 4: chunks are multiples of 1024 and E of 4); otherwise, and for
    // the vocabulary's last partial quad, element by element
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
  const Nucleus nu = nuclei(a.w, a.B)[b];
  const float wm = load_wmax(a, b);
  const float c = inv_temp(a, b);
  // kept mass of every chunk (chunk i keeps its ties while the ties of
  // chunks before it number fewer than nu.ties), and where this chunk's
  // starts; the per-chunk records come in with one load per thread
  __shared__ uint64_t s_wm[64];
  __shared__ uint32_t s_wt[64];
  if (t < 64) {
    s_wm[t] = t < a.W ? a.w.wmass[(size_t)b * a.W + t] : 0ull;
    s_wt[t] = t < a.W ? a.w.wties[(size_t)b * a.W + t] : 0u;
  }
  __builtin_amdgcn_sched_barrier(0);
  const float m = seq_max(wm);  // (its barrier also publishes s_wm, s_wt)
  uint64_t total = 0, before = 0, mine = 0;
  uint32_t ties_before = 0, tie_acc = 0;
  for (int i = 0; i < a.W; ++i) {
    const uint32_t ti = s_wt[i];
    const uint32_t kt = tie_acc >= nu.ties ? 0u : min(ti, nu.ties - tie_acc);
    const uint64_t km = s_wm[i] + (uint64_t)kt * nu.f_tau;
    if (i < w) {
      before += km;
      ties_before += ti;
    }
    if (i == w) mine = km;
    total += km;
    tie_acc += ti;
  }
  const float uu = fminf(fmaxf(a.u[b], 0.f), 1.f);
  uint64_t r = (uint64_t)floor((double)uu * (double)total);
  if (r >= total) r = total - 1;
  if (!(r >= before && r < before + mine)) return;  // the draw is not in this chunk
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
  const uint32_t lt_inc = wg_scan(lt);
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
  const uint64_t excl = before + wg_scan(km) - km;
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

}  // namespace

SampleWs sample_ws_carve(void* base, int B, int W) {
  SampleWs w{};
  const uintptr_t p = (uintptr_t)base;
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off = align256(off + bytes); return (void*)(p + at); };
  w.cnt = (uint32_t*)take(sizeof(uint32_t) * (size_t)B * 3 * kBuckets);
  w.mass = (uint64_t*)take(sizeof(uint64_t) * (size_t)B * 3 * kBuckets);
  w.sum = (uint64_t*)take(sizeof(uint64_t) * (size_t)B * W);
  w.choice = (void*)take((size_t)kSampleChoiceBytes * B * 3);
  w.wmax = (float*)take(sizeof(float) * (size_t)B * W);
  w.wmass = (uint64_t*)take(sizeof(uint64_t) * (size_t)B * W);
  w.wties = (uint32_t*)take(sizeof(uint32_t) * (size_t)B * W);
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
  sample_k3<<<grid, kSThreads, 0, st>>>(a);
  sample_k4<<<grid, kSThreads, 0, st>>>(a);
  sample_k5<<<grid, kSThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace pkv
