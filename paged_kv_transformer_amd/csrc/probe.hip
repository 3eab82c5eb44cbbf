// Measurement kernels: what the memory system and the launch path give
// without any of the method's arithmetic, so that a kernel's time can be
// read against them.
//   probe_read_kernel        streams a buffer once (16-byte non-temporal
//                            loads, several in flight per lane) and keeps
//                            nothing: the practical read ceiling of one
//                            launch of that size.
//   probe_paged_read_kernel  reads exactly the K and V tiles one paged
//                            attention call reads (same grid, same block
//                            table walk, same loads) and does no arithmetic
//                            on them: the ceiling of that call's data phase
//                            in one launch.
//   probe_empty_kernel       does nothing: the cost of a launch.
// None of them writes memory except through a store that the data cannot
// trigger (a sum compared with a value no finite sum of these loads takes
// exactly in practice), which keeps the compiler from dropping the loads.
#include "pkv_dev.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr unsigned kNever = 0x7f7fffffu;  // FLT_MAX's bits: the sink guard

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* p, int64_t n16, float* sink) {
  constexpr int U = 8;  // loads in flight per lane
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned acc = 0u;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == kNever) sink[0] = __uint_as_float(acc);
}

// Grid and loads of paged_attention_kernel<kQBf16, D, PW>: workgroup (kv
// head, sequence, split of kAttnWaves * PW tiles); each wave loads its
// tiles' K (16 tokens x D) and V (D x 16 tokens) of that kv head, all loads
// issued back to back (tiles past the sequence read page 0 and are masked,
// as in the attention kernel).
template <int D, int PW>
__global__ __launch_bounds__(kAttnWaves * 64) void probe_paged_read_kernel(const AttnArgs a, float* sink) {
  constexpr int NW = kAttnWaves, CP = NW * PW;
  constexpr int NH = D / 32, NC = D / 16;
  const int kvh = blockIdx.x, b = blockIdx.y, split = a.max_splits - 1 - (int)blockIdx.z;
  const int l = threadIdx.x & 63, col = l & 15, grp = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sh = a.pv.pt_shift;
  const int32_t* btrow = a.bt + (size_t)b * a.bt_row;
  int page[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) page[i] = btrow[min((split * CP + NW * i + wu) >> sh, a.bt_stride - 1)];
  const int n = a.lens[b];
  const int tiles = n > 0 ? (n + kTile - 1) / kTile : 0;
  if (split * CP >= tiles) return;
  bool live[PW];
  int sub[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int lp = split * CP + NW * i + wu;
    live[i] = lp < tiles && (unsigned)page[i] < (unsigned)a.pv.num_pages;
    page[i] = live[i] ? page[i] : 0;
    sub[i] = (lp & ((1 << sh) - 1)) * kTile;
  }
  u32x4 kr[PW][NH];
  u32x2 vr[PW][NC];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
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
  unsigned acc = 0u;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    unsigned t = 0u;
#pragma unroll
    for (int h = 0; h < NH; ++h) t ^= kr[i][h].x ^ kr[i][h].y ^ kr[i][h].z ^ kr[i][h].w;
#pragma unroll
    for (int c = 0; c < NC; ++c) t ^= vr[i][c].x ^ vr[i][c].y;
    acc ^= live[i] ? t : 0u;
  }
  if (acc == kNever) sink[0] = __uint_as_float(acc);
}

__global__ void probe_empty_kernel() {}

}  // namespace

hipError_t launch_probe_read(const void* buf, int64_t bytes, int workgroups, float* sink, hipStream_t st) {
  probe_read_kernel<<<workgroups, 256, 0, st>>>((const u32x4*)buf, bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_paged_read(const AttnArgs& a, int batch, float* sink, hipStream_t st) {
  const dim3 grid(a.Hkv, batch, a.max_splits);
  const int nt = kAttnWaves * 64;
  const bool large = a.pw == kAttnPWLarge;
  if (a.pw != kAttnPW && !large) return hipErrorInvalidValue;
  if (a.D == 64) {
    if (large) probe_paged_read_kernel<64, kAttnPWLarge><<<grid, nt, 0, st>>>(a, sink);
    else probe_paged_read_kernel<64, kAttnPW><<<grid, nt, 0, st>>>(a, sink);
  } else if (a.D == 128) {
    if (large) probe_paged_read_kernel<128, kAttnPWLarge><<<grid, nt, 0, st>>>(a, sink);
    else probe_paged_read_kernel<128, kAttnPW><<<grid, nt, 0, st>>>(a, sink);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_probe_empty(int launches, int workgroups, hipStream_t st) {
  for (int i = 0; i < launches; ++i) {
    probe_empty_kernel<<<workgroups, 64, 0, st>>>();
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pkv
