// One decoder layer of a single sequence (batch 1) in one launch, gfx950.
//
// The operation is decoder_layer_decode's (the layer op list of the
// "Inference from Scratch" summary: RMSNorm, QKV, RoPE at the token's
// absolute position, the append into the page, direct paged attention, the
// output projection and residual, RMSNorm, SwiGLU, the down projection and
// residual).  The engine-building article ("手写LLM推理引擎", section 4.2)
// counts the launches of such a layer as overhead of their own; at batch 1
// a layer's weights (30 MB for the Qwen2.5-0.5B shape) stream in a few
// microseconds, so six dependent launches, each paying its launch gap and
// the latency of its first bytes, cost several times the data.
//
// Here the whole layer is one launch of one workgroup per compute unit,
// all resident at once (the LDS each workgroup holds allows one per unit):
//   * Every projection is cut into units (a 16-row group of its packed
//     weights; for gate/up, 8 interleaved gate and up rows together with
//     the down projection's 8 matching columns) dealt round-robin over the
//     workgroups, each phase from its own first workgroup so that the
//     phases' units spread over the chip.
//   * A workgroup has kFusedWaves worker waves and as many loader waves.
//     At kernel start each loader wave issues every weight block of its
//     worker's share of all the workgroup's units, of all phases, as direct
//     global -> LDS copies (1 KiB per instruction, non-temporal), a few in
//     flight at a time, and publishes in LDS how many have landed; the
//     layer's weights thus stream from HBM at once while the phases that
//     need them still wait for their inputs.  The workers wait only for
//     the count of the blocks they are about to use and meet at a barrier
//     of their own (an LDS arrival counter), never at one that includes the
//     loaders.
//   * The phases (QKV with the norm, RoPE and the append; attention; O with
//     the residual; gate/up with SwiGLU and the down-projection partials;
//     the reduction of those partials with the residual) hand each other
//     only small vectors (q and the new K/V row, the attention records, h1,
//     the per-workgroup partials of the layer output), as 8-byte words
//     holding a value and the launch's epoch, stored and loaded at device
//     scope.  A consumer polls the words it needs until each carries the
//     current epoch: the data are their own flag, so no barrier, fence or
//     counter is needed between phases, and no word can be mistaken for an
//     older launch's or for another call's (the epoch is a tagged pattern no
//     other stored value has).
//   * Each workgroup keeps its own launch counter in the workspace's
//     header; all workgroups run every launch, so the counters stay equal.
//     Every wait is bounded in time: a poll that outlives its deadline sets
//     PKV_DEVERR_SYNC and lets the workgroup run on, so every wave exits.
//   * Products run on the matrix cores with the input vector as BF16 hi and
//     lo halves (FP32-like precision, as the multi-launch path); the
//     attention is the paged attention kernel's tile code on K/V tiles
//     that the loader waves copy into LDS first.  The down projection is
//     folded into the gate/up units: each multiplies its 8 SwiGLU outputs
//     by its 8 columns of the down weights into a partial of the whole
//     output row, and the reduction phase adds the partials of every
//     workgroup in a fixed order.
// Results are deterministic: every sum runs in a fixed order.
#include <type_traits>

#include "pkv_dev.h"

namespace pkv {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSc1 = 16;                 // device-scope cache policy of a buffer load
constexpr uint64_t kSpinTicks = 500000;  // 5 ms of the 100 MHz real-time counter
constexpr int kPollBatch = 12;           // 16-byte chunks per lane and poll round

__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i32x4 rsrc_words(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  return (i32x4){(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// One global -> LDS copy of 1 KiB by a wave (lane l's 16 bytes land at LDS
// byte address lds + 16 l); non-temporal: every weight block is read once.
// M0 carries the LDS address; the statement sets it itself.  The copy is
// counted by vmcnt and waited for explicitly (wait_vm).
__device__ __forceinline__ void lds_copy16_nt(uint32_t lds, uint32_t voff, i32x4 rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void ll_store(uint64_t* p, float v, uint32_t e) {
  __hip_atomic_store(p, ((uint64_t)e << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until the exchange words of `nch` 16-byte chunks (two words each)
// carry epoch e and copies their values to LDS: map(c, word, dst) gives
// chunk c's word offset in the exchange region r and its two destination
// floats.  The lanes li = 0 .. nl-1 of the calling waves share the chunks
// and issue all of their loads at once (at most kPollBatch per lane and
// round), so one round trip serves the whole gather; a lane reloads only
// its chunks not yet current.  Past the deadline the lane sets ERR_SYNC and
// writes zeros.
template <class F>
__device__ __forceinline__ void ll_gather(__amdgpu_buffer_rsrc_t r, int nch, F map, uint32_t e, int li, int nl,
                                          uint32_t* err) {
  for (int c0 = 0; c0 < nch; c0 += kPollBatch * nl) {
    u32x4 v[kPollBatch];
    int off[kPollBatch];
    float* dst[kPollBatch];
    bool need[kPollBatch];
#pragma unroll
    for (int k = 0; k < kPollBatch; ++k) {
      const int c = c0 + li + k * nl;
      need[k] = c < nch;
      int word = 0;
      map(need[k] ? c : 0, word, dst[k]);
      off[k] = word * 8;
      // only the lane's own chunks: a load whose result is never read
      // would make the compiler wait for every memory operation in flight
      // before it reuses the register
      if (need[k]) v[k] = __builtin_amdgcn_raw_buffer_load_b128(r, off[k], 0, kSc1);
    }
    uint64_t t0 = 0;
    for (int it = 0;; ++it) {
      bool all = true;
#pragma unroll
      for (int k = 0; k < kPollBatch; ++k) {
        if (!need[k]) continue;
        if (v[k].y == e && v[k].w == e) {
          dst[k][0] = __uint_as_float(v[k].x);
          dst[k][1] = __uint_as_float(v[k].z);
          need[k] = false;
        } else {
          all = false;
        }
      }
      if (all) break;
      const uint64_t now = __builtin_amdgcn_s_memrealtime();
      if (it == 0) {
        t0 = now;
      } else if (now - t0 > kSpinTicks) {
        set_error(err, ERR_SYNC);
#pragma unroll
        for (int k = 0; k < kPollBatch; ++k) {
          if (!need[k]) continue;
          dst[k][0] = 0.f;
          dst[k][1] = 0.f;
        }
        break;
      }
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int k = 0; k < kPollBatch; ++k)
        if (need[k]) v[k] = __builtin_amdgcn_raw_buffer_load_b128(r, off[k], 0, kSc1);
    }
  }
}

// Eight values as the B operand of a product: BF16 hi halves, then lo
// halves (x = hi + lo keeps ~16 significant bits), 32 bytes at chunk c of X.
__device__ __forceinline__ void put_chunk(float* X, int c, const float (&v)[8]) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const uint16_t h0 = to_bf16_bits(v[2 * x]), h1 = to_bf16_bits(v[2 * x + 1]);
    hw[x] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    lw[x] = (uint32_t)to_bf16_bits(v[2 * x] - bf16_lo(h0)) | ((uint32_t)to_bf16_bits(v[2 * x + 1] - bf16_lo(h1)) << 16);
  }
  u32x4* q = (u32x4*)X;
  q[2 * c] = (u32x4){hw[0], hw[1], hw[2], hw[3]};
  q[2 * c + 1] = (u32x4){lw[0], lw[1], lw[2], lw[3]};
}

// Keep the first `nv` of the four BF16 values in v (the rest -> +0).
__device__ __forceinline__ u32x2 keep_first(u32x2 v, int nv) {
  if (nv >= 4) return v;
  u32x2 r;
  r.x = nv >= 2 ? v.x : (nv == 1 ? (v.x & 0xffffu) : 0u);
  r.y = nv == 3 ? (v.y & 0xffffu) : 0u;
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return (uint32_t)to_bf16_bits(a) | ((uint32_t)to_bf16_bits(b) << 16);
}

// Barrier of the worker waves only (the loader waves never wait): an LDS
// arrival counter that only grows; `gen` counts this wave's barriers times
// the number of workers.
__device__ __forceinline__ void worker_barrier(uint32_t* cnt, uint32_t& gen) {
  gen += kFusedWaves;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < gen) __builtin_amdgcn_s_sleep(1);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// A loader wave publishes how many of its copies have landed; a worker
// waits for the count it needs.
__device__ __forceinline__ void publish(uint32_t* landed, int v) {
  __hip_atomic_store(landed, (uint32_t)v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void wait_landed(const uint32_t* landed, int need) {
  while ((int)__hip_atomic_load(landed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < need)
    __builtin_amdgcn_s_sleep(1);
}

// Copies a loader wave keeps in flight: after each copy past this many it
// waits for the oldest and publishes the count that has landed.
constexpr int kLoadDepth = 4;
template <int K>
__device__ __forceinline__ void drain(uint32_t* landed, int issued) {
  if constexpr (K >= 0) {
    wait_vm<K>();
    publish(landed, issued - K);
    drain<K - 1>(landed, issued);
  }
}

template <int D>
__global__ __launch_bounds__(kFusedThreads) void fused_layer_kernel(const FusedArgs a) {
  constexpr int NW = kFusedWaves;
  constexpr int NT = NW * 64;  // worker threads
  constexpr int NH = D / 32, NC = D / 16;
  constexpr int PW = 2;        // attention tiles per wave
  constexpr int KS = NH;       // 1 KiB slots of one K tile
  constexpr int TS = NH + D / 32;  // slots of one tile (K, then V)
  constexpr int MAXT = kFusedMaxHidden / 64 / NW;  // output rows per lane in the down partial
  __shared__ u32x4 wsl[NW][kFusedCap][64];
  __shared__ __align__(16) float X[kFusedX];
  __shared__ float red[2][NW][kFusedMaxUnits][16];  // by phase parity
  __shared__ float ssqp[2][NW];
  __shared__ float aval[kFusedMaxUnits][8];
  __shared__ float hrow[kFusedMaxUnits][kFusedRedRows];
  __shared__ uint32_t landed[NW];
  __shared__ uint32_t wbar;

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x, nwg = a.nwg;
  const int H = a.H, Hq = a.Hq, Hkv = a.Hkv, I = a.I, G = a.G, ns = a.ns;

  FusedGeo geo[FP_COUNT];
  int k0[FP_COUNT], cnt[FP_COUNT];
#pragma unroll
  for (int P = 0; P < FP_COUNT; ++P) {
    geo[P] = fused_geo(P, H, Hq, Hkv, D, I, ns);
    k0[P] = fused_first_unit(wg, a.first[P], nwg);
    cnt[P] = min(fused_unit_count(geo[P].n, k0[P], nwg), kFusedMaxUnits);
  }
  auto unit = [&](int P, int k) { return k0[P] + k * nwg; };
  const bool has_att = cnt[FP_ATT] > 0;
  const int ua = has_att ? unit(FP_ATT, 0) : 0;
  const int kvh = ua / ns, split = ua - (ua / ns) * ns;

  // the layer input and the attention norm, issued by the workers before
  // the loaders start: worker lane l loads chunk l & 3 (8 values) of its
  // wave's K step w + NW (l / 4) of the hidden vector
  const int wsh = fused_wave_slots(H / 32, w);  // this wave's 32-wide steps of H
  const bool hv = w < NW && l < 4 * wsh;
  const int hk = 32 * (w + NW * (l >> 2)) + 8 * (l & 3);  // first element of the lane's chunk
  float4 xq0 = {0.f, 0.f, 0.f, 0.f}, xq1 = xq0;
  u32x4 nq = {0u, 0u, 0u, 0u};
  if (hv && cnt[FP_QKV] > 0) {
    xq0 = *(const float4*)(a.hidden + hk);
    xq1 = *(const float4*)(a.hidden + hk + 4);
    nq = *(const u32x4*)(a.attn_norm + hk);
  }
  if (tid < NW) landed[tid] = 0u;
  if (tid == 0) wbar = 0u;
  __syncthreads();  // the only barrier of all waves

  // ===================================================== loader waves ===
  // Loader w - NW copies the slots of worker w - NW: the attention unit's K
  // and V tiles first (wave-local tiles split * 8 + 4 i + worker), then, in
  // phase order, slots j = worker, worker + NW, ... of every unit (for a
  // gate/up unit, its K steps, then its down-projection slots).
  if (w >= NW) {
    const int lw = w - NW;
    uint32_t* lnd = &landed[lw];
    const uint32_t base = (uint32_t)(uintptr_t)&wsl[lw][0][0];
    int issued = 0;
    auto copy = [&](uint32_t voff, i32x4 r) {
      lds_copy16_nt(base + (uint32_t)issued * 1024u, voff, r);
      ++issued;
      if (issued > kLoadDepth) {
        wait_vm<kLoadDepth>();
        publish(lnd, issued - kLoadDepth);
      }
    };
    if (has_att) {
      const int p = a.pos[0];
      const int sh = a.pv.pt_shift, PT = kTile << sh;
      const bool bad_len = p < 0 || (int64_t)(p + 1) > (int64_t)a.bt_stride * PT;
      const int ntiles = bad_len ? 0 : (p + 1 + kTile - 1) / kTile;
#pragma unroll
      for (int i = 0; i < PW; ++i) {
        const int lp = split * kFusedAttnTiles + NW * i + lw;
        int page = a.bt[min(lp >> sh, a.bt_stride - 1)];
        const bool ok = lp < ntiles && (unsigned)page < (unsigned)a.pv.num_pages;
        page = ok ? page : 0;
        const int sub = (lp & ((1 << sh) - 1)) * kTile;
        const i32x4 kr = rsrc_words(a.pv.k + pv_k_elem(a.pv, page, kvh, sub, 0, D), 32u * D);
        const i32x4 vr = rsrc_words(a.pv.v + pv_v_index(a.pv, page, kvh, 0, sub, D), 32u * D);
#pragma unroll
        for (int h = 0; h < KS; ++h) copy(h * 1024 + 16 * l, kr);
#pragma unroll
        for (int h = 0; h < TS - KS; ++h) copy(h * 1024 + 16 * l, vr);
      }
    }
    const uint16_t* mats[FP_COUNT] = {a.w_qkv, nullptr, a.w_o, a.w_gu, nullptr};
#pragma unroll
    for (int P = 0; P < FP_COUNT; ++P) {
      if (mats[P] == nullptr || cnt[P] == 0) continue;
      const FusedGeo g = geo[P];
      const i32x4 r = rsrc_words(mats[P], (uint32_t)g.n * (uint32_t)g.slots * 1024u);
      const int SI = I / 32;  // K steps of the down projection
      const i32x4 rd = rsrc_words(a.w_down, (uint32_t)(H / 16) * (uint32_t)SI * 1024u);
      for (int k = 0; k < cnt[P]; ++k) {
        const int u = unit(P, k);
        for (int j = lw; j < g.slots; j += NW) copy(((uint32_t)u * g.slots + (uint32_t)j) * 1024u + 16u * l, r);
        // gate/up unit u: columns 8 u .. 8 u + 7 of the down projection are
        // the 16-byte chunk (u % 4) of K step u / 4 of every 16-row group;
        // slot t holds row groups 4 t .. 4 t + 3 (lane l: group 4 t + l / 16)
        for (int t = lw; t < g.extra; t += NW) {
          const uint32_t grp_row = 4u * t + (l >> 4);
          copy(((grp_row * SI + (uint32_t)(u >> 2)) * 64u + 16u * (u & 3) + (l & 15)) * 16u, rd);
        }
      }
    }
    drain<kLoadDepth>(lnd, issued);
    return;
  }

  // ===================================================== worker waves ===
  uint32_t* err = a.err;
  uint32_t gen = 0;
  // the copy of the h1 words this workgroup reads: the consumers of each
  // copy are a fixed eighth of the grid
  const int copy = wg % kFusedCopies;
  const uint64_t* ll0 = a.q;  // the exchange region starts at q
  const uint32_t llw = (uint32_t)(a.ypart + (size_t)H * nwg - a.q);
  const uint32_t launch_no = a.epoch[wg] + 1u;  // this launch's number
  const uint32_t e = fused_epoch_tag(launch_no);  // the epoch its words carry
  const int p = a.pos[0];
  const int psh = 4 + a.pv.pt_shift, PT = 1 << psh;
  const int half = D / 2;
  // slots of this worker before each phase's first (its loader's order)
  int first_slot[FP_COUNT];
  {
    int at = has_att ? PW * TS : 0;
#pragma unroll
    for (int P = 0; P < FP_COUNT; ++P) {
      first_slot[P] = at;
      at += cnt[P] * (fused_wave_slots(geo[P].slots, w) + fused_wave_slots(geo[P].extra, w));
    }
  }

  // ---- prefetch: everything else that does not depend on another phase
  // the MLP norm for the lane's chunk of h1 (same chunks as the input's)
  u32x4 ng = {0u, 0u, 0u, 0u};
  if (hv && cnt[FP_GU] > 0) ng = *(const u32x4*)(a.mlp_norm + hk);
  // QKV epilogue: lane idx = 8 k + i (pair i of unit k): RoPE cos/sin, the page
  float pf_cs = 1.f, pf_sn = 0.f;
  int pf_page = -1;
  const bool p_rope = p >= 0 && p < a.max_pos;
  const bool p_tab = p >= 0 && (p >> psh) < a.bt_stride;
  if (tid < 8 * cnt[FP_QKV]) {
    const int u = unit(FP_QKV, tid >> 3), gph = D / 16, hd = u / gph, j = 8 * (u - hd * gph) + (tid & 7);
    if (p_rope && hd < Hq + Hkv) {
      pf_cs = a.rcos[(size_t)p * half + j];
      pf_sn = a.rsin[(size_t)p * half + j];
    }
    if (hd >= Hq && p_tab) pf_page = a.bt[p >> psh];
  }
  // attention: this wave's tiles' table entries
  int att_page[2] = {0, 0};
  if (has_att) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int lp = split * kFusedAttnTiles + NW * i + w;
      att_page[i] = a.bt[min(lp >> a.pv.pt_shift, a.bt_stride - 1)];
    }
  }
  // O epilogue: lane idx = 16 k + m holds the residual x[16 u + m]
  float pf_x = 0.f;
  if (tid < 16 * cnt[FP_O]) pf_x = a.hidden[16 * unit(FP_O, tid >> 4) + (tid & 15)];

  const __amdgpu_buffer_rsrc_t llr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t*>(ll0), (short)0, (int)(llw * 8u), 0x00020000);
  auto word = [&](const uint64_t* q) { return (int)(q - ll0); };

  // Products of this wave's slots j (= w, w + NW, ...) of every unit of
  // phase P with the input chunks in X (hi/lo BF16, put_chunk), on the
  // matrix cores: the 1 KiB slot is the A operand as packed, the input
  // chunks of K step j the B operand (the same in every column), so column 0
  // of the result holds the unit's 16 row sums over this wave's K steps.
  auto products = [&](int P, int par) {
    const FusedGeo g = geo[P];
    const int ws = fused_wave_slots(g.slots, w), we = fused_wave_slots(g.extra, w);
    wait_landed(&landed[w], first_slot[P] + cnt[P] * (ws + we));
    const u32x4* Xc = (const u32x4*)X;
    const int col = l & 15, ch = l >> 4;
    // the units' products interleaved (independent accumulators, the hi
    // and lo halves of the input in separate ones): no MFMA waits for the
    // previous one's result
    const int s0 = first_slot[P], su = ws + we;
    // KU units at once (a compile-time count, so that every operand read of
    // a K step is issued before its products), from unit k0u on
    auto run = [&](auto KC, int k0u) {
      constexpr int KU = decltype(KC)::value;
      f32x4 ah[KU], al[KU];
#pragma unroll
      for (int k = 0; k < KU; ++k) ah[k] = al[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
      for (int jj = 0; jj < ws; ++jj) {
        const int c = 4 * (w + jj * NW) + ch;
        const u32x4 bh = Xc[2 * c], bl = Xc[2 * c + 1];
        u32x4 av[KU];
#pragma unroll
        for (int k = 0; k < KU; ++k) av[k] = wsl[w][s0 + (k0u + k) * su + jj][l];
#pragma unroll
        for (int k = 0; k < KU; ++k) {
          ah[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[k]),
                                                         __builtin_bit_cast(bf16x8, bh), ah[k], 0, 0, 0);
          al[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[k]),
                                                         __builtin_bit_cast(bf16x8, bl), al[k], 0, 0, 0);
        }
      }
      if (col == 0) {
#pragma unroll
        for (int k = 0; k < KU; ++k)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[par][w][k0u + k][4 * ch + r] = ah[k][r] + al[k][r];
      }
    };
    // the phase's units in groups of at most four
    for (int k0u = 0; k0u < cnt[P]; k0u += 4) {
      switch (min(cnt[P] - k0u, 4)) {
        case 1: run(std::integral_constant<int, 1>{}, k0u); break;
        case 2: run(std::integral_constant<int, 2>{}, k0u); break;
        case 3: run(std::integral_constant<int, 3>{}, k0u); break;
        default: run(std::integral_constant<int, 4>{}, k0u); break;
      }
    }
  };
  // Input chunks of this wave's K steps (w + NW j) from values already in X
  // (floats), converted in place (put_chunk).
  auto convert_runs = [&](int steps) {
    for (int c = l; c < 4 * fused_wave_slots(steps, w); c += 64) {
      const int cc = 4 * (w + NW * (c >> 2)) + (c & 3);
      const float4 v0 = *(const float4*)(X + 8 * cc), v1 = *(const float4*)(X + 8 * cc + 4);
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      put_chunk(X, cc, v);
    }
  };
  int par = 0;

  // ================= QKV: products on RMSNorm's input, RoPE, the append
  if (cnt[FP_QKV] > 0) {
    float ssq = 0.f;
    if (hv) {
      float v[8] = {xq0.x, xq0.y, xq0.z, xq0.w, xq1.x, xq1.y, xq1.z, xq1.w};
      const uint32_t nw[4] = {nq.x, nq.y, nq.z, nq.w};
#pragma unroll
      for (int x = 0; x < 8; ++x) ssq += v[x] * v[x];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        v[2 * x] *= bf16_lo(nw[x]);
        v[2 * x + 1] *= bf16_hi(nw[x]);
      }
      put_chunk(X, hk / 8, v);
    }
    ssq = wave_sum(ssq);
    if (l == 0) ssqp[par][w] = ssq;
    products(FP_QKV, par);
    worker_barrier(&wbar, gen);
    if (tid < 8 * cnt[FP_QKV]) {
      float tot = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) tot += ssqp[par][ww];
      const float rs = 1.0f / sqrtf(tot / (float)H + a.eps);
      const int k = tid >> 3, i = tid & 7;
      const int u = unit(FP_QKV, k), gph = D / 16, hd = u / gph, j = 8 * (u - hd * gph) + i;
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        x0 += red[par][ww][k][i];
        x1 += red[par][ww][k][8 + i];
      }
      x0 *= rs;
      x1 *= rs;
      const bool is_q = hd < Hq, is_k = !is_q && hd < Hq + Hkv;
      float y0 = x0, y1 = x1;
      if (is_q || is_k) {
        if (!p_rope) {
          set_error(err, ERR_ROPE);
        } else {
          y0 = __fsub_rn(__fmul_rn(x0, pf_cs), __fmul_rn(x1, pf_sn));
          y1 = __fadd_rn(__fmul_rn(x0, pf_sn), __fmul_rn(x1, pf_cs));
        }
      }
      if (is_q) {
        ll_store(a.q + (size_t)hd * D + j, y0, e);
        ll_store(a.q + (size_t)hd * D + j + half, y1, e);
      } else {
        const int h = is_k ? hd - Hq : hd - Hq - Hkv;
        const uint16_t b0 = to_bf16_bits(y0), b1 = to_bf16_bits(y1);
        uint64_t* dst = is_k ? a.kn : a.vn;
        ll_store(dst + (size_t)h * D + j, bf16_lo(b0), e);
        ll_store(dst + (size_t)h * D + j + half, bf16_lo(b1), e);
        if (!p_tab) {
          set_error(err, ERR_LENGTH);
        } else if ((unsigned)pf_page >= (unsigned)a.pv.num_pages) {
          set_error(err, ERR_PAGE);
        } else {
          const int slot = p & (PT - 1);
          if (is_k) {
            a.pv.k[pv_k_elem(a.pv, pf_page, h, slot, j, D)] = b0;
            a.pv.k[pv_k_elem(a.pv, pf_page, h, slot, j + half, D)] = b1;
          } else {
            uint16_t* vp = a.pv.v + pv_v_index(a.pv, pf_page, h, 0, slot, D);
            vp[j * kTile] = b0;
            vp[(j + half) * kTile] = b1;
          }
        }
      }
    }
    par ^= 1;
  }

  // ================= attention of one (kv head, 128-token split)
  const int RL = fused_rec_len(G, D);
  if (has_att) {
    // staging in X: q (G rows of D + 4 floats: rows 16 bytes apart in the
    // banks), the new K row, the new V row, then the waves' m, l and O
    constexpr int QST = D + 4;
    const int XQ = 0, XK = G * QST, XV = XK + D, XS = XV + D;
    const int nq_ch = G * D / 2, nk_ch = D / 2;
    ll_gather(llr, nq_ch + 2 * nk_ch, [&](int c, int& wd, float*& dst) {
      if (c < nq_ch) {
        wd = word(a.q) + kvh * G * D + 2 * c;
        dst = X + XQ + (2 * c / D) * QST + (2 * c) % D;
      } else if (c < nq_ch + nk_ch) {
        wd = word(a.kn) + kvh * D + 2 * (c - nq_ch);
        dst = X + XK + 2 * (c - nq_ch);
      } else {
        wd = word(a.vn) + kvh * D + 2 * (c - nq_ch - nk_ch);
        dst = X + XV + 2 * (c - nq_ch - nk_ch);
      }
    }, e, tid, NT, err);
    worker_barrier(&wbar, gen);
    const int n = p + 1;
    const bool bad_len = p < 0 || (int64_t)n > (int64_t)a.bt_stride * PT;
    const int ntiles = bad_len ? 0 : (n + kTile - 1) / kTile;
    const int col = l & 15, grp = l >> 4;
    int lpv[PW];
    bool bad_page = false;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int lp = split * kFusedAttnTiles + NW * i + w;
      const int page = att_page[i];
      const bool live = lp < ntiles, ok = (unsigned)page < (unsigned)a.pv.num_pages;
      bad_page |= live && !ok;
      lpv[i] = live && ok ? lp : -1;
    }
    wait_landed(&landed[w], PW * TS);
    u32x4 kr[PW][NH];
    u32x2 vr[PW][NC];
#pragma unroll
    for (int i = 0; i < PW; ++i) {
#pragma unroll
      for (int h = 0; h < NH; ++h) kr[i][h] = wsl[w][i * TS + h][l];
      const char* vb = (const char*)&wsl[w][i * TS + KS][0];
#pragma unroll
      for (int c = 0; c < NC; ++c)
        vr[i][c] = *(const u32x2*)(vb + (c >> 1) * 1024 + (c & 1) * 512 + 32 * col + 8 * grp);
    }
    const int pt = p & 15, ptile = p >> 4;
    // q^T operand (head g = col, dims 8 grp + e + 32 h) as BF16 hi + lo
    const int gq = col < G ? col : 0;
    bf16x8 qh[NH], ql[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const float4 v0 = *(const float4*)(X + XQ + gq * QST + 32 * h + 8 * grp);
      const float4 v1 = *(const float4*)(X + XQ + gq * QST + 32 * h + 8 * grp + 4);
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const uint16_t h0 = to_bf16_bits(v[2 * x]), h1 = to_bf16_bits(v[2 * x + 1]);
        hw[x] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        lw[x] = (uint32_t)to_bf16_bits(v[2 * x] - bf16_lo(h0)) |
                ((uint32_t)to_bf16_bits(v[2 * x + 1] - bf16_lo(h1)) << 16);
      }
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 hv4 = {hw[0], hw[1], hw[2], hw[3]}, lv4 = {lw[0], lw[1], lw[2], lw[3]};
      qh[h] = __builtin_bit_cast(bf16x8, col < G ? hv4 : z);
      ql[h] = __builtin_bit_cast(bf16x8, col < G ? lv4 : z);
    }
    // the new token: its K and V from the QKV phase, not from the page
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      if (lpv[i] != ptile) continue;
      if (col == pt) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const float* kv = X + XK + 32 * h + 8 * grp;
          kr[i][h] = (u32x4){pack_bf16(kv[0], kv[1]), pack_bf16(kv[2], kv[3]), pack_bf16(kv[4], kv[5]),
                             pack_bf16(kv[6], kv[7])};
        }
      }
      if ((pt >> 2) == grp) {
        const int r = pt & 3;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const uint32_t b = to_bf16_bits(X[XV + col + 16 * c]);
          const uint32_t wd = r < 2 ? vr[i][c].x : vr[i][c].y;
          const uint32_t nw = (r & 1) ? ((wd & 0xffffu) | (b << 16)) : ((wd & 0xffff0000u) | b);
          if (r < 2)
            vr[i][c].x = nw;
          else
            vr[i][c].y = nw;
        }
      }
    }
    if (bad_page && l == 0) set_error(err, ERR_PAGE);
    if (bad_len && split == 0 && w == 0 && l == 0) set_error(err, ERR_LENGTH);
    const float c2 = a.scale * kLog2e;
    bool full[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i) full[i] = lpv[i] >= 0 && (lpv[i] + 1) * kTile <= n;
    f32x4 sc[PW];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        acc = mfma_k32(kr[i][h], qh[h], acc);
        acc = mfma_k32(kr[i][h], ql[h], acc);
      }
      if (!full[i]) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = lpv[i] * kTile + 4 * grp + r;
          acc[r] = lpv[i] >= 0 && t < n ? acc[r] : -INFINITY;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, acc[r]);
      sc[i] = acc;
    }
    mx = rows_max4(mx);
    const float msub = mx == -INFINITY ? 0.f : mx;
    const float m2 = mx == -INFINITY ? -INFINITY : mx * c2;
    float lsum = 0.f;
    s16x4 ph[PW], pl[PW];
#pragma unroll
    for (int i = 0; i < PW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = (sc[i][r] - msub) * c2;
        if (!full[i]) x = sc[i][r] == -INFINITY ? -INFINITY : x;
        const float pv = __builtin_amdgcn_exp2f(x);
        lsum += pv;
        const __bf16 hi = (__bf16)pv;
        ph[i][r] = __builtin_bit_cast(short, hi);
        pl[i][r] = __builtin_bit_cast(short, (__bf16)(pv - (float)hi));
      }
    lsum = rows_sum4(lsum);
    f32x4 o[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) o[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int nv = full[i] ? 4 : (lpv[i] < 0 ? 0 : n - (lpv[i] * kTile + 4 * grp));
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const s16x4 vb = __builtin_bit_cast(s16x4, keep_first(vr[i][c], nv));
        o[c] = mfma_k16(ph[i], vb, o[c]);
        o[c] = mfma_k16(pl[i], vb, o[c]);
      }
    }
    // the wave's (m, l, O): O as [wave][d][head], heads padded to GP, so
    // that a lane's four heads of one column are one 16-byte write
    const int GP = G <= 4 ? 4 : (G <= 8 ? 8 : 16);
    float* sm_m = X + XS;
    float* sm_l = X + XS + NW * 16;
    float* sm_o = X + XS + 2 * NW * 16;
    if (grp == 0) {
      sm_m[w * 16 + col] = m2;
      sm_l[w * 16 + col] = lsum;
    }
    if (4 * grp < GP) {
#pragma unroll
      for (int c = 0; c < NC; ++c) *(f32x4*)&sm_o[(w * D + col + 16 * c) * GP + 4 * grp] = o[c];
    }
    worker_barrier(&wbar, gen);
    // the four waves merged in order: with one split per kv head the
    // attention output itself (o = O / L at o index kvh G D + idx),
    // otherwise this split's (m, l, O) record
    uint64_t* rec = a.rec + (size_t)(kvh * ns + split) * RL;
    for (int idx = tid; idx < G * D; idx += NT) {
      const int gg = idx / D, d = idx - gg * D;
      float M = sm_m[gg];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sm_m[ww * 16 + gg]);
      float L = 0.f, O = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float mw = sm_m[ww * 16 + gg];
        const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L += f * sm_l[ww * 16 + gg];
        O += f * sm_o[(ww * D + d) * GP + gg];
      }
      if (ns == 1) {
        ll_store(a.rec + (size_t)kvh * G * D + idx, L > 0.f ? O / L : 0.f, e);
      } else {
        if (d == 0) {
          ll_store(rec + gg, M, e);
          ll_store(rec + G + gg, L, e);
        }
        ll_store(rec + 2 * G + idx, O, e);
      }
    }
    worker_barrier(&wbar, gen);  // X is reused below
  }

  // ================= O: products on the attention output, the residual
  if (cnt[FP_O] > 0) {
    const int QD = Hq * D, nr = fused_wave_slots(QD / 32, w);
    if (ns == 1) {
      // this wave's runs of o, straight from the attention's words
      ll_gather(llr, 16 * nr, [&](int c, int& wd, float*& dst) {
        const int j = w + NW * (c >> 4), at = 32 * j + 2 * (c & 15);
        wd = word(a.rec) + at;
        dst = X + at;
      }, e, l, 64, err);
    } else {
      // every split's record, merged by the whole workgroup into o
      ll_gather(llr, Hkv * ns * RL / 2, [&](int c, int& wd, float*& dst) {
        wd = word(a.rec) + 2 * c;
        dst = X + QD + 2 * c;
      }, e, tid, NT, err);
      worker_barrier(&wbar, gen);
      for (int idx = tid; idx < QD; idx += NT) {
        const int h = idx / (G * D), rem = idx - h * (G * D), gg = rem / D;
        const float* r0 = X + QD + (size_t)h * ns * RL;
        float M = -INFINITY;
        for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, r0[sp * RL + gg]);
        float L = 0.f, O = 0.f;
        for (int sp = 0; sp < ns; ++sp) {
          const float ms = r0[sp * RL + gg];
          const float f = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
          L += f * r0[sp * RL + G + gg];
          O += f * r0[sp * RL + 2 * G + rem];
        }
        X[idx] = L > 0.f ? O / L : 0.f;
      }
      worker_barrier(&wbar, gen);
    }
    convert_runs(Hq * D / 32);
    products(FP_O, par);
    worker_barrier(&wbar, gen);
    if (tid < 16 * cnt[FP_O]) {
      const int k = tid >> 4, m = tid & 15;
      float y = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) y += red[par][ww][k][m];
      const float v = pf_x + y;
#pragma unroll
      for (int c = 0; c < kFusedCopies; ++c) ll_store(a.h1 + (size_t)c * H + 16 * unit(FP_O, k) + m, v, e);
    }
    par ^= 1;
  }

  // ================= gate/up: products on h1 times the MLP norm, SwiGLU,
  // then the down projection's columns of these units
  float ypart[MAXT];
#pragma unroll
  for (int t = 0; t < MAXT; ++t) ypart[t] = 0.f;
  if (cnt[FP_GU] > 0) {
    const uint64_t* h1c = a.h1 + (size_t)copy * H;
    ll_gather(llr, 16 * wsh, [&](int c, int& wd, float*& dst) {
      const int at = 32 * (w + NW * (c >> 4)) + 2 * (c & 15);
      wd = word(h1c) + at;
      dst = X + at;
    }, e, l, 64, err);
    // the lane's chunk hk of h1 is the one its prefetched norm chunk covers
    float ssq = 0.f;
    if (hv) {
      const float4 v0 = *(const float4*)(X + hk), v1 = *(const float4*)(X + hk + 4);
      float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      const uint32_t nw[4] = {ng.x, ng.y, ng.z, ng.w};
#pragma unroll
      for (int x = 0; x < 8; ++x) ssq += v[x] * v[x];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        v[2 * x] *= bf16_lo(nw[x]);
        v[2 * x + 1] *= bf16_hi(nw[x]);
      }
      put_chunk(X, hk / 8, v);
    }
    ssq = wave_sum(ssq);
    if (l == 0) ssqp[par][w] = ssq;
    products(FP_GU, par);
    worker_barrier(&wbar, gen);
    if (tid < 8 * cnt[FP_GU]) {
      float tot = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) tot += ssqp[par][ww];
      const float rs = 1.0f / sqrtf(tot / (float)H + a.eps);
      const int k = tid >> 3, i = tid & 7;
      float gv = 0.f, uv = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        gv += red[par][ww][k][i];
        uv += red[par][ww][k][8 + i];
      }
      gv *= rs;
      uv *= rs;
      aval[k][i] = gv / (1.0f + expf(-gv)) * uv;
    }
    worker_barrier(&wbar, gen);
    // down-projection slots t = w, w + NW, ..: lane l holds row 64 t + l,
    // columns 8 u .. 8 u + 7; the lane sums every unit of the workgroup
    const FusedGeo g = geo[FP_GU];
    const int ws = fused_wave_slots(g.slots, w), we = fused_wave_slots(g.extra, w);
    for (int k = 0; k < cnt[FP_GU]; ++k) {
      const float4 a0 = *(const float4*)&aval[k][0], a1 = *(const float4*)&aval[k][4];
      const int slot0 = first_slot[FP_GU] + k * (ws + we) + ws;
#pragma unroll
      for (int t = 0; t < MAXT; ++t) {
        if (t >= we) break;
        const u32x4 wv = wsl[w][slot0 + t][l];
        float y = ypart[t];
        y = fmaf(bf16_lo(wv.x), a0.x, y);
        y = fmaf(bf16_hi(wv.x), a0.y, y);
        y = fmaf(bf16_lo(wv.y), a0.z, y);
        y = fmaf(bf16_hi(wv.y), a0.w, y);
        y = fmaf(bf16_lo(wv.z), a1.x, y);
        y = fmaf(bf16_hi(wv.z), a1.y, y);
        y = fmaf(bf16_lo(wv.w), a1.z, y);
        y = fmaf(bf16_hi(wv.w), a1.w, y);
        ypart[t] = y;
      }
    }
    par ^= 1;
  }
  // every workgroup's partial of the layer output, zero if it has no
  // gate/up unit: row r at word ((r / 4) nwg + wg) 4 + r % 4
  {
    const int wt = fused_wave_slots(H / 64, w);
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      if (t >= wt) break;
      const int r = 64 * (w + NW * t) + l;
      ll_store(a.ypart + ((size_t)(r >> 2) * nwg + wg) * 4 + (r & 3), ypart[t], e);
    }
  }

  // ================= the layer output: h1 + the partials, in workgroup order
  if (cnt[FP_RED] > 0) {
    const uint64_t* h1c = a.h1 + (size_t)copy * H;
    const int per = 2 * nwg;  // chunks of one unit's partials
    ll_gather(llr, cnt[FP_RED] * (per + 2), [&](int c, int& wd, float*& dst) {
      const int k = c / (per + 2), t = c - k * (per + 2), u = unit(FP_RED, k);
      if (t < per) {
        wd = word(a.ypart) + u * 4 * nwg + 2 * t;
        dst = X + k * 4 * nwg + 2 * t;
      } else {
        wd = word(h1c) + kFusedRedRows * u + 2 * (t - per);
        dst = &hrow[k][2 * (t - per)];
      }
    }, e, tid, NT, err);
    worker_barrier(&wbar, gen);
    // wave w: row 4 u + w of every unit; lane l sums workgroups l, l + 64, ..
    for (int k = 0; k < cnt[FP_RED]; ++k) {
      float y = 0.f;
      for (int s2 = l; s2 < nwg; s2 += 64) y += X[k * 4 * nwg + 4 * s2 + w];
      y = wave_sum(y);
      if (l == 0) {
        const int r = kFusedRedRows * unit(FP_RED, k) + w;
        const float v = hrow[k][w] + y;
        a.hidden[r] = v;
        if (a.hidden_packed) a.hidden_packed[packed_act_index(0, r, H)] = v;
      }
    }
  }
  if (tid == 0) a.epoch[wg] = launch_no;
}

}  // namespace

// ------------------------------------------------------------------ host ---

bool plan_fused_layer(int H, int Hq, int Hkv, int D, int I, int64_t max_tiles, int nwg, FusedArgs* a) {
  if (nwg < 1 || nwg > kFusedMaxWgs || (D != 64 && D != 128)) return false;
  if (H > kFusedMaxHidden || H % 64 != 0 || I % 32 != 0) return false;
  const int G = Hq / Hkv;
  if (G < 1 || G > kMaxGroup) return false;
  const int ns = fused_splits(max_tiles);
  if (ns < 1 || (int64_t)Hkv * ns > nwg) return false;  // one attention unit per workgroup at most
  // the phase-input buffer: input vectors, the split records beside o, the
  // attention staging, the partials of the output rows a workgroup adds
  const int RL = fused_rec_len(G, D);
  const int64_t need_o = (int64_t)Hq * D + (ns > 1 ? (int64_t)Hkv * ns * RL : 0);
  const int GP = G <= 4 ? 4 : (G <= 8 ? 8 : 16);
  const int64_t need_att = (int64_t)G * (D + 4) + 2 * D + 2 * kFusedWaves * 16 + (int64_t)kFusedWaves * D * GP;
  const int red_units = (H / kFusedRedRows + nwg - 1) / nwg;
  const int64_t need_red = (int64_t)red_units * kFusedRedRows * nwg;
  if (need_o > kFusedX || need_att > kFusedX || need_red > kFusedX || H > kFusedX) return false;
  FusedGeo geo[FP_COUNT];
  for (int P = 0; P < FP_COUNT; ++P) geo[P] = fused_geo(P, H, Hq, Hkv, D, I, ns);
  // gate/up from workgroup 0; QKV, O and attention from the first workgroup
  // with one gate/up unit fewer; the reduction from workgroup 0
  int first[FP_COUNT];
  first[FP_GU] = 0;
  first[FP_QKV] = geo[FP_GU].n % nwg;
  first[FP_O] = (first[FP_QKV] + geo[FP_QKV].n) % nwg;
  first[FP_ATT] = (first[FP_O] + geo[FP_O].n) % nwg;
  first[FP_RED] = 0;
  for (int wg = 0; wg < nwg; ++wg) {
    for (int w = 0; w < kFusedWaves; ++w) {
      int slots = 0;
      for (int P = 0; P < FP_COUNT; ++P) {
        const int c = fused_unit_count(geo[P].n, fused_first_unit(wg, first[P], nwg), nwg);
        if (c > kFusedMaxUnits || (P == FP_ATT && c > 1)) return false;
        // an attention unit's K and V tiles: 2 per wave of D / 16 slots each
        slots += P == FP_ATT ? c * 2 * (D / 16)
                             : c * (fused_wave_slots(geo[P].slots, w) + fused_wave_slots(geo[P].extra, w));
      }
      if (slots > kFusedCap) return false;
    }
  }
  a->H = H;
  a->Hq = Hq;
  a->Hkv = Hkv;
  a->D = D;
  a->I = I;
  a->G = G;
  a->nwg = nwg;
  a->ns = ns;
  for (int P = 0; P < FP_COUNT; ++P) a->first[P] = first[P];
  return true;
}

int fused_device_wgs() {
  static int cache[64];  // per device: 0 unknown, -1 unsupported, else compute units
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  if (cache[dev] != 0) return cache[dev];
  int cus = 0, blocks = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fused_layer_kernel<64>, kFusedThreads, 0) !=
          hipSuccess ||
      blocks < 1 || cus < 1 || cus > kFusedMaxWgs) {
    (void)hipGetLastError();
    cache[dev] = -1;
    return -1;
  }
  cache[dev] = cus;
  return cus;
}

hipError_t launch_fused_layer(const FusedArgs& a, hipStream_t st) {
  if (a.D == 64)
    fused_layer_kernel<64><<<a.nwg, kFusedThreads, 0, st>>>(a);
  else if (a.D == 128)
    fused_layer_kernel<128><<<a.nwg, kFusedThreads, 0, st>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkv
