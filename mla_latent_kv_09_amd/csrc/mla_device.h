// Device-side helpers shared by the HIP kernels of the MLA decode library:
// bf16 <-> fp32 conversion, element load/store by storage type, the
// token -> sequence lookup and the split plan of the paged decode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_index.h"

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

__device__ __forceinline__ QueryWork query_work(const int32_t* __restrict__ cu_q,
                                                const int32_t* __restrict__ seq_lens, int batch,
                                                int t, int split, int num_splits,
                                                int pages_per_split, int page_size,
                                                int max_pages, int causal) {
  const int b = find_seq(cu_q, batch, t);
  const int q0 = cu_q[b];
  return split_work(b, q0, cu_q[b + 1] - q0, seq_lens[b], t, split, num_splits, pages_per_split,
                    page_size, max_pages, causal);
}

// The batch's sequence table spread over one wave: for batch <= 64, lane l holds the end
// offset cu_q[l + 1] and the length seq_lens[l] of sequence l, fetched in one round trip
// at the start of a kernel, and a lookup is a ballot and a lane read instead of the
// binary search's chain of dependent loads.  Larger batches fall back to those loads.
// Every lane of the wave must be active when it is loaded and queried.
struct SeqIndex {
  const int32_t* cu_q;
  const int32_t* seq_lens;
  int batch;
  int end, len, first;

  __device__ __forceinline__ bool wide() const { return batch <= 64; }
  __device__ __forceinline__ void load(const int32_t* __restrict__ cu, const int32_t* __restrict__ lens,
                                       int n) {
    cu_q = cu;
    seq_lens = lens;
    batch = n;
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const bool in = wide() && lane < n;
    end = in ? cu[lane + 1] : 0;
    len = in ? lens[lane] : 0;
    first = cu[0];
  }
  // The largest b with cu_q[b] <= t (cu_q non-decreasing): the number of sequences
  // 1 .. batch-1 that start at or before row t.
  __device__ __forceinline__ int find(int t) const {
    if (!wide()) return find_seq(cu_q, batch, t);
    const int lane = static_cast<int>(threadIdx.x) & 63;
    return __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < batch - 1 && end <= t));
  }
  __device__ __forceinline__ int start(int b) const {
    if (!wide()) return cu_q[b];
    return b > 0 ? __builtin_amdgcn_readlane(end, b - 1) : first;
  }
  __device__ __forceinline__ int stop(int b) const {
    return wide() ? __builtin_amdgcn_readlane(end, b) : cu_q[b + 1];
  }
  __device__ __forceinline__ int length(int b) const {
    return wide() ? __builtin_amdgcn_readlane(len, b) : seq_lens[b];
  }
};

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  const int lane = static_cast<int>(threadIdx.x) & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// unit_active_first (mla_index.h) for workgroup L, the sequences taken 64 at a time
// (lane l holds sequence c + l of chunk c): per pass, a prefix sum of the units each
// sequence contributes locates L's sequence, and unit_in_sequence places it there.
__device__ __forceinline__ Unit unit_active_first_wave(int L, int S, int pages_per_split, int page_size,
                                                       int max_pages, const int32_t* __restrict__ cu_q,
                                                       const int32_t* __restrict__ seq_lens, int batch) {
  const int lane = static_cast<int>(threadIdx.x) & 63;
  int base = 0;
  for (int pass = 0; pass < 2; ++pass)
    for (int c = 0; c < batch; c += 64) {
      const int b = c + lane;
      int q0 = 0, nq = 0, a = 0;
      if (b < batch) {
        q0 = cu_q[b];
        nq = cu_q[b + 1] - q0;
        a = active_splits(seq_lens[b], S, pages_per_split, page_size, max_pages);
      }
      const int lo = pass == 0 ? 0 : a, cnt = pass == 0 ? a : S - a;
      const int units = nq * cnt;
      const int incl = wave_inclusive_sum(units);
      const int total = __builtin_amdgcn_readlane(incl, 63);
      if (L < base + total) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(b < batch && L < base + incl);
        const int lb = static_cast<int>(__builtin_ctzll(m));
        const int before = __builtin_amdgcn_readlane(incl - units, lb);
        return unit_in_sequence(L - base - before, __builtin_amdgcn_readlane(q0, lb),
                                __builtin_amdgcn_readlane(nq, lb), __builtin_amdgcn_readlane(lo, lb),
                                __builtin_amdgcn_readlane(cnt, lb));
      }
      base += total;
    }
  return unit_split_fastest(L, S);
}

__device__ __forceinline__ QueryWork query_work(const SeqIndex& ix, int t, int split, int num_splits,
                                                int pages_per_split, int page_size, int max_pages,
                                                int causal) {
  const int b = ix.find(t);
  const int q0 = ix.start(b);
  return split_work(b, q0, ix.stop(b) - q0, ix.length(b), t, split, num_splits, pages_per_split,
                    page_size, max_pages, causal);
}

__device__ __forceinline__ int clamp_page(int32_t p, int num_pool_pages) {
  return p < 0 ? 0 : (p >= num_pool_pages ? num_pool_pages - 1 : p);
}

}  // namespace mla
