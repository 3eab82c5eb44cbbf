// Small kernels of the decode path: the standalone KV append, the embedding
// gather, the RoPE cos/sin table and a workspace fill.
#include "pkv_dev.h"

namespace pkv {
namespace {

// One workgroup per sequence: copy the new token's K ([Hkv][D], into the
// K block at [head][slot][d]) and V (into the V block at [head][d][slot]).
// The engine's decode appends one token per sequence at its absolute
// position: logical page pos / 16, slot pos % 16.
__global__ void kv_append_kernel(uint16_t* pool, int64_t page_elems, int32_t num_pages,
                                 const int32_t* bt, int32_t bt_stride, const int32_t* pos,
                                 const uint16_t* k, const uint16_t* v, int Hkv) {
  const int b = blockIdx.x;
  const int p = pos[b];
  if (p < 0 || p / kPageTokens >= bt_stride) return;
  const int page = bt[(size_t)b * bt_stride + p / kPageTokens];
  if ((unsigned)page >= (unsigned)num_pages) return;
  const int slot = p % kPageTokens;
  uint16_t* pg = pool + (int64_t)page * page_elems;
  uint16_t* vblk = pg + (int64_t)Hkv * kPageTokens * kHeadDim;
  const uint16_t* kb = k + (size_t)b * Hkv * kHeadDim;
  const uint16_t* vb = v + (size_t)b * Hkv * kHeadDim;
  for (int i = threadIdx.x; i < Hkv * kHeadDim; i += blockDim.x) {
    const int h = i / kHeadDim, d = i % kHeadDim;
    pg[((int64_t)h * kPageTokens + slot) * kHeadDim + d] = kb[i];
    vblk[((int64_t)h * kHeadDim + d) * kPageTokens + slot] = vb[i];
  }
}

// x[b] = E[token[b]] widened from BF16 to FP32 (the engine's embedding gather).
__global__ void embed_kernel(const uint16_t* E, int V, int H, const int32_t* tok, float* x,
                             uint32_t* err) {
  const int b = blockIdx.x;
  const int t = tok[b];
  float* xr = x + (size_t)b * H;
  if ((unsigned)t >= (unsigned)V) {
    if (threadIdx.x == 0) set_error(err, ERR_TOKEN);
    for (int i = threadIdx.x; i < H; i += blockDim.x) xr[i] = 0.f;
    return;
  }
  const uint16_t* er = E + (size_t)t * H;
  for (int i = threadIdx.x; i < H; i += blockDim.x) xr[i] = __uint_as_float((uint32_t)er[i] << 16);
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

hipError_t launch_kv_append(uint16_t* pool, int64_t page_elems, int32_t num_pages,
                            const int32_t* bt, int32_t bt_stride, const int32_t* pos,
                            const uint16_t* k, const uint16_t* v, int batch, int Hkv,
                            hipStream_t st) {
  kv_append_kernel<<<batch, 256, 0, st>>>(pool, page_elems, num_pages, bt, bt_stride, pos, k, v,
                                          Hkv);
  return hipGetLastError();
}

hipError_t launch_embed(const uint16_t* E, int V, int H, const int32_t* tok, float* x, int batch,
                        uint32_t* err, hipStream_t st) {
  embed_kernel<<<batch, 256, 0, st>>>(E, V, H, tok, x, err);
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
