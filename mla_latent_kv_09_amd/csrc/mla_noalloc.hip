// mla_attend_noalloc: split-KV decode plus log-sum-exp merge (mla_decode_paged followed
// by mla_combine) with the split partials in library-owned static device memory, for
// callers that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  It calls no allocating routine: the partials live in
// `scratch`, a file-scope device array of MLA_NOALLOC_SCRATCH_BYTES that every device the
// library runs on holds until the process ends.
#include <stdint.h>

#include <atomic>

#include "mla_internal.h"
#include "mla_kv.h"

namespace {

static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device.  The array's name is a host-side
// stand-in, never a device address: host code uses only what hipGetSymbolAddress returns,
// looked up once per device (ids below 64; higher ids look it up on every call) with that
// device current.
int scratch_address(char** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<char*> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MLA_ERR_LAUNCH;
  if (dev < kMaxDevices) {
    char* p = cached[dev].load(std::memory_order_acquire);
    if (p != nullptr) {
      *out = p;
      return MLA_OK;
    }
  }
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_ERR_LAUNCH;
  if (dev < kMaxDevices) cached[dev].store(static_cast<char*>(p), std::memory_order_release);
  *out = static_cast<char*>(p);
  return MLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int mla_attend_noalloc(const void* q_abs, const void* q_r, const void* kv_cache,
                                  const int32_t* page_table, const int32_t* seq_lens,
                                  const int32_t* cu_q, const float* rope_cos, const float* rope_sin,
                                  int rope_max_pos, void* o_latent, float* lse_out, int batch,
                                  int total_q, int max_pages_per_seq, int num_pool_pages, int heads,
                                  int groups, int d_hc, int d_c, int d_R, int page_size,
                                  int num_splits, int pages_per_split, float softmax_scale,
                                  int causal, int dtype, void* stream) {
  // Every argument is checked on the host before the device is touched: the decode's own
  // validation (without partial buffers), the merge's outputs, then the capacity.
  mla::DecodeArgs a{};
  bool bf16 = false;
  int st = mla::decode_validate(q_abs, q_r, kv_cache, page_table, seq_lens, cu_q, rope_cos,
                                rope_sin, rope_max_pos, nullptr, nullptr, batch, total_q,
                                max_pages_per_seq, num_pool_pages, heads, groups, d_hc, d_c, d_R,
                                page_size, num_splits, pages_per_split, softmax_scale, causal,
                                dtype, false, &a, &bf16);
  if (st != MLA_OK || total_q == 0) return st;
  if (!o_latent) return MLA_ERR_NULL;
  if (!aligned16(o_latent) || (lse_out && !aligned16(lse_out))) return MLA_ERR_ALIGN;
  const size_t rows = static_cast<size_t>(total_q) * heads * num_splits;
  const size_t o_bytes = rows * static_cast<size_t>(d_c / groups) * (bf16 ? 2 : 4);
  const size_t lse_off = (o_bytes + 255) & ~static_cast<size_t>(255);
  if (lse_off + rows * sizeof(float) > MLA_NOALLOC_SCRATCH_BYTES) return MLA_ERR_UNSUPPORTED;
  char* base = nullptr;
  if ((st = scratch_address(&base)) != MLA_OK) return st;
  a.o_part = base;
  a.lse_part = reinterpret_cast<float*>(base + lse_off);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = mla::decode_launch(a, bf16, s)) != MLA_OK) return st;
  return mla_combine(a.o_part, a.lse_part, o_latent, lse_out, total_q, heads, groups, d_c,
                     num_splits, dtype, stream);
}
