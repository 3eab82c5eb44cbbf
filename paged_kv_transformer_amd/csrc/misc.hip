// Small kernels of the decode path: the standalone KV append, the embedding
// gather, the weight packing, the RoPE cos/sin table and a workspace fill.
#include "pkv_dev.h"

namespace pkv {
namespace {

// One workgroup per sequence: copy the new token's K and V ([Hkv][D] each)
// into its slot of the page's K and V tiles.
// The engine's decode appends one token per sequence at its absolute
// position: logical page pos / 16, slot pos % 16.  A position outside the
// table or a table entry outside the pool writes nothing and sets its bit
// in the caller's error word (if any); the workgroup then exits.
__global__ void kv_append_kernel(const PoolView pv, const int32_t* bt, int32_t bt_stride,
                                 const int32_t* pos, const uint16_t* k, const uint16_t* v, int Hkv,
                                 int D, uint32_t* err) {
  const int b = blockIdx.x;
  const int p = pos[b];
  const int psh = 4 + pv.pt_shift;  // log2 of the page's tokens
  if (p < 0 || (p >> psh) >= bt_stride) {
    if (err && threadIdx.x == 0) set_error(err, ERR_LENGTH);
    return;
  }
  const int page = bt[(size_t)b * bt_stride + (p >> psh)];
  if ((unsigned)page >= (unsigned)pv.num_pages) {
    if (err && threadIdx.x == 0) set_error(err, ERR_PAGE);
    return;
  }
  const int slot = p & ((1 << psh) - 1);
  const uint16_t* kb = k + (size_t)b * Hkv * D;
  const uint16_t* vb = v + (size_t)b * Hkv * D;
  for (int i = threadIdx.x; i < Hkv * D; i += blockDim.x) {
    const int h = i / D, d = i % D;
    pv.k[pv_k_elem(pv, page, h, slot, d, D)] = kb[i];
    pv.v[pv_v_index(pv, page, h, d, slot, D)] = vb[i];
  }
}

// x[b] = E[token[b]] widened from BF16 to FP32 (the engine's embedding
// gather), read from the packed embedding (which is also the tied LM head)
// and written plain and, if xp is given, packed (the first projection's
// input).  One thread per 8 consecutive elements (H is a multiple of 64):
// one 16-byte load, no loop.
__global__ void embed_kernel(const uint16_t* E, int V, int H, const int32_t* tok, float* x,
                             float* xp, uint32_t* err) {
  const int b = blockIdx.y;
  const int k = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (k >= H) return;
  const int t = tok[b];
  float4* xr = (float4*)(x + (size_t)b * H + k);
  float4 lo = make_float4(0.f, 0.f, 0.f, 0.f), hi = lo;
  if ((unsigned)t >= (unsigned)V) {
    if (k == 0) set_error(err, ERR_TOKEN);
  } else {
    // packed block (group t / 16, step k / 32), lane 16 ((k % 32) / 8) + t % 16
    const int64_t e = ((((int64_t)(t >> 4) * (H >> 5) + (k >> 5)) * 64 + ((k & 31) >> 3) * 16 + (t & 15)) << 3);
    const uint4 w = *(const uint4*)(E + e);
    lo = make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
    hi = make_float4(bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w));
  }
  xr[0] = lo;
  xr[1] = hi;
  if (xp) {
    float4* xq = (float4*)(xp + packed_act_index(b, k, H));
    xq[0] = lo;
    xq[1] = hi;
  }
}

// Packs a row-major [rows][cols] BF16 matrix (cols a multiple of 32): one
// thread per 16-byte lane chunk of a 1 KiB block (group G, step s, lane l).
__global__ void pack_weight_kernel(const uint16_t* src, int rows, int cols, int kind,
                                   uint16_t* dst, int64_t chunks) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= chunks) return;
  const int S = cols >> 5;
  const int l = (int)(c & 63);
  const int64_t gs = c >> 6;
  const int s = (int)(gs % S);
  const int G = (int)(gs / S);
  const int r = packed_row(kind, rows, G, l & 15);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (r >= 0) v = *(const uint4*)(src + (size_t)r * cols + 32 * s + 8 * (l >> 4));
  *(uint4*)(dst + (c << 3)) = v;
}

// cos/sin of p * theta^(-2j/D) in double, rounded to FP32.
__global__ void rope_table_kernel(double theta, int D, int max_pos, float* c, float* s) {
  const int half = D / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)max_pos * half) return;
  const int p = (int)(idx / half), j = (int)(idx % half);
  const double inv_freq = pow(theta, -2.0 * (double)j / (double)D);
  const double ang = (double)p * inv_freq;
  c[idx] = (float)cos(ang);
  s[idx] = (float)sin(ang);
}

__global__ void fill_zero_kernel(uint4* p, size_t n16, unsigned char* tail, size_t ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_kv_append(const PoolView& pv, const int32_t* bt, int32_t bt_stride,
                            const int32_t* pos, const uint16_t* k, const uint16_t* v, int batch,
                            int Hkv, int D, uint32_t* err, hipStream_t st) {
  kv_append_kernel<<<batch, 256, 0, st>>>(pv, bt, bt_stride, pos, k, v, Hkv, D, err);
  return hipGetLastError();
}

hipError_t launch_embed(const uint16_t* E_packed, int V, int H, const int32_t* tok, float* x,
                        float* x_packed, int batch, uint32_t* err, hipStream_t st) {
  const dim3 grid((H / 8 + 255) / 256, batch);
  embed_kernel<<<grid, 256, 0, st>>>(E_packed, V, H, tok, x, x_packed, err);
  return hipGetLastError();
}

hipError_t launch_pack_weight(const uint16_t* src, int rows, int cols, int kind, uint16_t* dst,
                              hipStream_t st) {
  const int64_t chunks = packed_weight_elems(rows, cols, kind) / 8;
  pack_weight_kernel<<<(unsigned)((chunks + 255) / 256), 256, 0, st>>>(src, rows, cols, kind, dst,
                                                                       chunks);
  return hipGetLastError();
}

hipError_t launch_rope_table(double theta, int D, int max_pos, float* c, float* s,
                             hipStream_t st) {
  const int64_t n = (int64_t)max_pos * (D / 2);
  const int blocks = (int)((n + 255) / 256);
  rope_table_kernel<<<blocks, 256, 0, st>>>(theta, D, max_pos, c, s);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const size_t ntail = bytes % 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  fill_zero_kernel<<<(unsigned)blocks, 256, 0, st>>>((uint4*)p, n16, (unsigned char*)p + n16 * 16,
                                                     ntail);
  return hipGetLastError();
}

}  // namespace pkv
