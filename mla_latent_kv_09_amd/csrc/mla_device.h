// Device-side helpers shared by the HIP kernels of the MLA decode library:
// bf16 <-> fp32 conversion, element load/store by storage type, the
// token -> sequence lookup and the split plan of the paged decode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float load_elem(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float load_elem(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ void store_elem(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
__device__ __forceinline__ void store_elem(float* p, size_t i, float v) { p[i] = v; }

// Sequence owning packed query row t: the largest b with cu_q[b] <= t.
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ cu_q, int batch, int t) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Where query row t sits and which keys split s of its sequence covers.
struct QueryWork {
  int b;       // sequence
  int L;       // keys of the sequence (clamped to the page-table capacity)
  int pos;     // absolute position of the query
  int k0, k1;  // key range [k0, k1) of this split, already clipped to the visible keys
};

__device__ __forceinline__ QueryWork query_work(const int32_t* __restrict__ cu_q,
                                                const int32_t* __restrict__ seq_lens, int batch,
                                                int t, int split, int num_splits,
                                                int pages_per_split, int page_size,
                                                int max_pages, int causal) {
  QueryWork w;
  w.b = find_seq(cu_q, batch, t);
  const int q0 = cu_q[w.b];
  const int q_len = cu_q[w.b + 1] - q0;
  int L = seq_lens[w.b];
  const int cap = max_pages * page_size;
  L = L < 0 ? 0 : (L > cap ? cap : L);
  w.L = L;
  w.pos = L - q_len + (t - q0);
  int n_vis = causal ? min(L, w.pos + 1) : L;
  if (n_vis < 0) n_vis = 0;
  const int n_pages = (L + page_size - 1) / page_size;
  const int per_split = pages_per_split > 0 ? pages_per_split
                                            : (n_pages + num_splits - 1) / num_splits;
  w.k0 = split * per_split * page_size;
  w.k1 = split == num_splits - 1 ? n_vis : min((split + 1) * per_split * page_size, n_vis);
  return w;
}

__device__ __forceinline__ int clamp_page(int32_t p, int num_pool_pages) {
  return p < 0 ? 0 : (p >= num_pool_pages ? num_pool_pages - 1 : p);
}

}  // namespace mla
