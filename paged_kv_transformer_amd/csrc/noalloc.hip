// paged_gqa_decode_noalloc: the paged decode attention for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc).  It runs exactly the kernels of
// paged_gqa_decode; the only difference is where their scratch lives.  The
// split records that the attention kernel leaves for its merge kernel are
// kept in a file-scope device array, `scratch`, of a fixed size that every
// GPU the library runs on holds until the process ends; nothing is
// allocated or freed by the call, and the device-error bits go to a word the
// caller passes.
//
// In host code the name `scratch` is a host-side stand-in, not a device
// address: the array's device address is looked up once per device with
// hipGetSymbolAddress (with that device current, on the first call there)
// and only that address is ever handed to a kernel.
//
// Every call on one GPU shares that GPU's array, which keeps the last call's
// records: calls that overlap on one GPU (different streams, or different
// host threads without ordering) race on it.  Nothing in it has to start at
// zero (every record the merge reads is written by the same call first).
#include <errno.h>
#include <mutex>

#include "pkv.h"
#include "pkv_dev.h"

using namespace pkv;

static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on the
// first call there; nullptr if the runtime cannot say.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" int paged_gqa_decode_noalloc(const pkv_pool* pool, const uint16_t* q, int32_t num_q_heads,
                                        const int32_t* block_table, int32_t max_pages,
                                        const int32_t* context_lens, int32_t batch, float scale,
                                        float* out, uint32_t* dev_error, void* stream) {
  AttnArgs a{};
  int rc = prepare_attention_call(pool, q, num_q_heads, block_table, max_pages, context_lens, batch,
                                  scale, out, &a);
  if (rc || batch == 0) return rc;
  if (!dev_error || !aligned(dev_error, 4)) return -EINVAL;
  if (attention_record_bytes(a, batch) > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return -ENOSPC;
  void* sp = scratch_address();
  if (!sp) return -EIO;
  a.part = (float*)sp;
  a.err = dev_error;
  if (launch_attention(a, batch, kQBf16, (hipStream_t)stream) == hipSuccess) return 0;
  (void)hipGetLastError();
  return -EIO;
}
