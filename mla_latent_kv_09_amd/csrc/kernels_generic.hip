// Shape-generic HIP kernels of the MLA decode step.
//
// These handle any supported dimensions in either storage type with plain
// fp32 FMA arithmetic.  They are the path for small or unusual shapes (the
// 16-head fp32 tiny workload among them); the production shapes (d_cg 512 or
// 256, d_R 64, bf16) go to the MFMA kernels.  Both produce the same results up
// to fp32 rounding order.
//
// Sources: www.nxmr.cn/news/151634 §1 (latent row = c_KV | k_R), §4 (absorbed
// score q_abs . c_KV + q_R . k_R, scale 1/sqrt(d_hc + d_R)), §3/§4 (RoPE in
// fp32); m.xxqk.cn/news/443191 §2.4 (up-projection back to the value space)
// and §2.5 (softmax attention).
#include <math.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerPass = 16;  // query rows handled per pass of the projection kernels

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// q_abs[t,h,c] = sum_d q_c[t,h,d] * w_uk[h,d,c].  Block: one head, 256 latent columns.
template <typename T>
__global__ void __launch_bounds__(kThreads)
absorb_generic_kernel(const T* __restrict__ q_c, const T* __restrict__ w_uk, T* __restrict__ q_abs,
                      int Tq, int H, int d_hc, int d_cg) {
  extern __shared__ float q_s[];  // [kRowsPerPass][d_hc]
  const int h = blockIdx.y;
  const int c = blockIdx.x * kThreads + threadIdx.x;
  const T* w = w_uk + static_cast<size_t>(h) * d_hc * d_cg;
  for (int t0 = 0; t0 < Tq; t0 += kRowsPerPass) {
    const int nt = min(kRowsPerPass, Tq - t0);
    __syncthreads();
    for (int e = threadIdx.x; e < kRowsPerPass * d_hc; e += kThreads) {
      const int i = e / d_hc, d = e - i * d_hc;
      q_s[e] = i < nt ? load_elem(q_c, (static_cast<size_t>(t0 + i) * H + h) * d_hc + d) : 0.f;
    }
    __syncthreads();
    if (c < d_cg) {
      float acc[kRowsPerPass];
#pragma unroll
      for (int i = 0; i < kRowsPerPass; ++i) acc[i] = 0.f;
      for (int d = 0; d < d_hc; ++d) {
        const float wv = load_elem(w, static_cast<size_t>(d) * d_cg + c);
#pragma unroll
        for (int i = 0; i < kRowsPerPass; ++i) acc[i] = fmaf(q_s[i * d_hc + d], wv, acc[i]);
      }
      for (int i = 0; i < nt; ++i)
        store_elem(q_abs, (static_cast<size_t>(t0 + i) * H + h) * d_cg + c, acc[i]);
    }
  }
}

// out[t,h,d] = sum_c w_uv[h,d,c] * o[t,h,c].  Block: one head, 16 output dims (4 per wave).
template <typename T>
__global__ void __launch_bounds__(kThreads)
up_v_generic_kernel(const T* __restrict__ o_lat, const T* __restrict__ w_uv, T* __restrict__ out,
                    int Tq, int H, int d_hc, int d_cg) {
  extern __shared__ float o_s[];  // [kRowsPerPass][d_cg]
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const T* w = w_uv + static_cast<size_t>(h) * d_hc * d_cg;
  for (int t0 = 0; t0 < Tq; t0 += kRowsPerPass) {
    const int nt = min(kRowsPerPass, Tq - t0);
    __syncthreads();
    for (int e = threadIdx.x; e < kRowsPerPass * d_cg; e += kThreads) {
      const int i = e / d_cg, c = e - i * d_cg;
      o_s[e] = i < nt ? load_elem(o_lat, (static_cast<size_t>(t0 + i) * H + h) * d_cg + c) : 0.f;
    }
    __syncthreads();
    for (int k = 0; k < 4; ++k) {
      const int d = blockIdx.x * 16 + wave * 4 + k;
      if (d >= d_hc) break;
      float acc[kRowsPerPass];
#pragma unroll
      for (int i = 0; i < kRowsPerPass; ++i) acc[i] = 0.f;
      for (int c = lane; c < d_cg; c += 64) {
        const float wv = load_elem(w, static_cast<size_t>(d) * d_cg + c);
#pragma unroll
        for (int i = 0; i < kRowsPerPass; ++i) acc[i] = fmaf(o_s[i * d_cg + c], wv, acc[i]);
      }
      for (int i = 0; i < nt; ++i) {
        const float v = wave_sum(acc[i]);
        if (lane == 0) store_elem(out, (static_cast<size_t>(t0 + i) * H + h) * d_hc + d, v);
      }
    }
  }
}

// One block per (query row t, split s, head h): online softmax over the split's
// keys, one page (<= 64 keys) at a time.
template <typename T>
__global__ void __launch_bounds__(kThreads) decode_generic_kernel(DecodeArgs a) {
  constexpr int kMaxCols = 1024, kMaxRope = 256, kTile = 64;
  __shared__ float q_s[kMaxCols];
  __shared__ float qr_s[kMaxRope];
  __shared__ float s_s[kTile];
  const int t = blockIdx.x, split = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.heads, S = a.num_splits, d_cg = a.d_c / a.groups, d_R = a.d_R;
  const int width = a.d_c + a.d_R;
  const int g = h / (H / a.groups);
  const QueryWork w = query_work(a.cu_q, a.seq_lens, a.batch, t, split, S,
                                 a.pages_per_split, a.page_size, a.max_pages, a.causal);
  const size_t row = (static_cast<size_t>(t) * H + h) * S + split;
  T* o_out = static_cast<T*>(a.o_part) + row * d_cg;
  if (w.k0 >= w.k1) {  // empty split: only the LSE is written
    if (tid == 0) a.lse_part[row] = -INFINITY;
    return;
  }
  const T* q = static_cast<const T*>(a.q_abs) + (static_cast<size_t>(t) * H + h) * d_cg;
  for (int c = tid; c < d_cg; c += kThreads) q_s[c] = load_elem(q, c);
  const T* qr = static_cast<const T*>(a.q_r) + (static_cast<size_t>(t) * H + h) * d_R;
  const int half = d_R / 2;
  for (int k = tid; k < half; k += kThreads) {
    const float x0 = load_elem(qr, 2 * k), x1 = load_elem(qr, 2 * k + 1);
    if (a.rope_cos != nullptr) {
      const int p = min(max(w.pos, 0), a.rope_max_pos - 1);
      const float cs = a.rope_cos[static_cast<size_t>(p) * half + k];
      const float sn = a.rope_sin[static_cast<size_t>(p) * half + k];
      qr_s[2 * k] = fmaf(x0, cs, -x1 * sn);
      qr_s[2 * k + 1] = fmaf(x0, sn, x1 * cs);
    } else {
      qr_s[2 * k] = x0;
      qr_s[2 * k + 1] = x1;
    }
  }
  __syncthreads();

  const float scale_log2 = a.scale * kLog2e;
  constexpr int kColsPerThread = kMaxCols / kThreads;
  float acc[kColsPerThread];
#pragma unroll
  for (int k = 0; k < kColsPerThread; ++k) acc[k] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int j0 = w.k0; j0 < w.k1; j0 += a.page_size) {
    const int n = min(a.page_size, w.k1 - j0);
    const int page = clamp_page(a.page_table[static_cast<size_t>(w.b) * a.max_pages + j0 / a.page_size],
                                a.num_pool_pages);
    const T* kv = static_cast<const T*>(a.kv) + static_cast<size_t>(page) * a.page_size * width;
    for (int jj = wave; jj < n; jj += kThreads / 64) {
      const T* r = kv + static_cast<size_t>(jj) * width;
      float part = 0.f;
      for (int c = lane; c < d_cg; c += 64) part = fmaf(q_s[c], load_elem(r, g * d_cg + c), part);
      for (int c = lane; c < d_R; c += 64) part = fmaf(qr_s[c], load_elem(r, a.d_c + c), part);
      part = wave_sum(part);
      if (lane == 0) s_s[jj] = part * scale_log2;
    }
    __syncthreads();
    float tmax = -INFINITY;
    for (int jj = 0; jj < n; ++jj) tmax = fmaxf(tmax, s_s[jj]);
    const float m_new = fmaxf(m, tmax);
    const float alpha = exp2f(m - m_new);
    l *= alpha;
#pragma unroll
    for (int k = 0; k < kColsPerThread; ++k) acc[k] *= alpha;
    for (int jj = 0; jj < n; ++jj) {
      const float p = exp2f(s_s[jj] - m_new);
      l += p;
      const T* r = kv + static_cast<size_t>(jj) * width + g * d_cg;
#pragma unroll
      for (int k = 0; k < kColsPerThread; ++k) {
        const int c = tid + k * kThreads;
        if (c < d_cg) acc[k] = fmaf(p, load_elem(r, c), acc[k]);
      }
    }
    m = m_new;
    __syncthreads();
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int k = 0; k < kColsPerThread; ++k) {
    const int c = tid + k * kThreads;
    if (c < d_cg) store_elem(o_out, c, acc[k] * inv);
  }
  if (tid == 0) a.lse_part[row] = (m + log2f(l)) * kLn2;
}

// One block per (t, h): merge num_splits partials by their log-sum-exp.
template <typename T>
__global__ void __launch_bounds__(kThreads)
combine_kernel(const T* __restrict__ o_part, const float* __restrict__ lse_part,
               T* __restrict__ o_lat, float* __restrict__ lse_out, int d_cg, int S) {
  constexpr int kMaxSplits = 256;
  __shared__ float w_s[kMaxSplits];
  __shared__ float red_s[kThreads / 64];
  __shared__ float stat_s[2];
  const size_t r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float v = tid < S ? lse_part[r * S + tid] : -INFINITY;
  float mx = v;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) red_s[wave] = mx;
  __syncthreads();
  if (tid == 0) {
    float M = red_s[0];
    for (int i = 1; i < kThreads / 64; ++i) M = fmaxf(M, red_s[i]);
    stat_s[0] = M;
  }
  __syncthreads();
  const float M = stat_s[0];
  const float wt = (tid < S && M != -INFINITY) ? expf(v - M) : 0.f;
  if (tid < S) w_s[tid] = wt;
  const float ws = wave_sum(wt);
  __syncthreads();
  if (lane == 0) red_s[wave] = ws;
  __syncthreads();
  if (tid == 0) {
    float sum = 0.f;
    for (int i = 0; i < kThreads / 64; ++i) sum += red_s[i];
    stat_s[1] = sum;
  }
  __syncthreads();
  const float sum = stat_s[1];
  const float inv = M == -INFINITY ? 0.f : 1.f / sum;
  for (int c = tid; c < d_cg; c += kThreads) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) {
      const float ww = w_s[s];
      if (ww != 0.f) acc = fmaf(ww, load_elem(o_part, (r * S + s) * d_cg + c), acc);
    }
    store_elem(o_lat, r * d_cg + c, acc * inv);
  }
  if (tid == 0 && lse_out != nullptr) lse_out[r] = M == -INFINITY ? -INFINITY : M + logf(sum);
}

// Vectorised combine for d_cg in {256, 512}: one wave per (t, h) row; lane l owns
// columns kE l .. kE l + kE - 1 (kE = d_cg / 64), read as kW 32-bit words per split
// (16 B for bf16 rows of 512).  The partials of up to kChunk splits (at most 128 words
// per lane) are requested together, before the log-sum-exp reduction, so a row of up
// to kChunk splits costs about one memory round trip; the launch picks the smallest
// chunk that covers the split count, which keeps the register count, and so the
// number of rows in flight per CU, as high as the split count allows.  Splits with LSE = -inf (no keys)
// get weight 0 and their partials -- never written -- are not used.
template <typename T, int kW>
__device__ __forceinline__ void load_words(const T* p, uint32_t (&x)[kW]) {
  static_assert(kW == 2 || kW % 4 == 0, "8- or 16-byte pieces");
  if constexpr (kW == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    x[0] = v.x;
    x[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < kW / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      x[4 * i] = v.x;
      x[4 * i + 1] = v.y;
      x[4 * i + 2] = v.z;
      x[4 * i + 3] = v.w;
    }
  }
}
// Element e of a lane's piece, widened to float.
template <typename T>
__device__ __forceinline__ float word_elem(const uint32_t* x, int e) {
  if constexpr (sizeof(T) == 2)
    return __uint_as_float((e & 1) ? (x[e >> 1] & 0xffff0000u) : (x[e >> 1] << 16));
  else
    return __uint_as_float(x[e]);
}

template <typename T, int kDcg>
constexpr int combine_max_chunk() { return 128 / (kDcg / 64 * static_cast<int>(sizeof(T)) / 4); }

template <typename T, int kDcg, int kChunk>
__global__ void __launch_bounds__(kThreads)
combine_vec_kernel(const T* __restrict__ o_part, const float* __restrict__ lse_part,
                   T* __restrict__ o_lat, float* __restrict__ lse_out, int rows, int S) {
  constexpr int kE = kDcg / 64;                                  // columns per lane
  constexpr int kW = kE * static_cast<int>(sizeof(T)) / 4;       // words per lane and split
  static_assert(kChunk * kW <= 128, "at most 128 words of partials per lane");
  const int lane = threadIdx.x & 63;
  const size_t r = static_cast<size_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= static_cast<size_t>(rows)) return;
  const float* lse = lse_part + r * S;
  const T* base = o_part + r * S * kDcg + kE * lane;
  // Lane s holds the LSE of split s (s < 64): loaded before the partials so that its
  // wait does not also wait for them, and broadcast with readlane below.
  const float l_lane = lane < S ? lse[lane] : -INFINITY;
  uint32_t x[kChunk][kW];
  auto load_chunk = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      if (s0 + u < S) load_words<T, kW>(base + static_cast<size_t>(s0 + u) * kDcg, x[u]);
  };
  load_chunk(0);
  float mx = l_lane;
  for (int s = lane + 64; s < S; s += 64) mx = fmaxf(mx, lse[s]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  float acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
  float sum = 0.f;
  for (int s0 = 0; s0 < S; s0 += kChunk) {
    if (s0 > 0) load_chunk(s0);
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int s = s0 + u;
      float l = -INFINITY;
      if (s < S) l = s < 64 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_lane), s)) : lse[s];
      const float wt = (l == -INFINITY || mx == -INFINITY) ? 0.f : expf(l - mx);
      sum += wt;
      if (wt != 0.f) {
#pragma unroll
        for (int e = 0; e < kE; ++e) acc[e] += wt * word_elem<T>(x[u], e);
      }
    }
  }
  const float inv = mx == -INFINITY ? 0.f : 1.f / sum;
  uint32_t y[kW];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int w = 0; w < kW; ++w)
      y[w] = static_cast<uint32_t>(f32_to_bf16(acc[2 * w] * inv)) |
             (static_cast<uint32_t>(f32_to_bf16(acc[2 * w + 1] * inv)) << 16);
  } else {
#pragma unroll
    for (int w = 0; w < kW; ++w) y[w] = __float_as_uint(acc[w] * inv);
  }
  T* dst = o_lat + r * kDcg + kE * lane;
  if constexpr (kW == 2) {
    *reinterpret_cast<uint2*>(dst) = uint2{y[0], y[1]};
  } else {
#pragma unroll
    for (int i = 0; i < kW / 4; ++i)
      reinterpret_cast<uint4*>(dst)[i] = uint4{y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]};
  }
  if (lane == 0 && lse_out != nullptr) lse_out[r] = mx == -INFINITY ? -INFINITY : mx + logf(sum);
}

__global__ void __launch_bounds__(kThreads)
rope_table_kernel(float* __restrict__ cos_out, float* __restrict__ sin_out, int max_pos, int half,
                  double base) {
  const size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= static_cast<size_t>(max_pos) * half) return;
  const int p = static_cast<int>(i / half), k = static_cast<int>(i % half);
  const double theta = pow(base, -2.0 * k / (2.0 * half));
  const double ang = static_cast<double>(p) * theta;
  cos_out[i] = static_cast<float>(cos(ang));
  sin_out[i] = static_cast<float>(sin(ang));
}

}  // namespace

hipError_t launch_absorb_generic(const void* q_c, const void* w_uk, void* q_abs, int T, int H,
                                 int d_hc, int d_cg, bool bf16, hipStream_t s) {
  const dim3 grid((d_cg + kThreads - 1) / kThreads, H);
  const size_t lds = sizeof(float) * kRowsPerPass * d_hc;
  if (bf16)
    absorb_generic_kernel<uint16_t><<<grid, kThreads, lds, s>>>(
        static_cast<const uint16_t*>(q_c), static_cast<const uint16_t*>(w_uk),
        static_cast<uint16_t*>(q_abs), T, H, d_hc, d_cg);
  else
    absorb_generic_kernel<float><<<grid, kThreads, lds, s>>>(
        static_cast<const float*>(q_c), static_cast<const float*>(w_uk), static_cast<float*>(q_abs),
        T, H, d_hc, d_cg);
  return hipGetLastError();
}

hipError_t launch_up_v_generic(const void* o_lat, const void* w_uv, void* out, int T, int H,
                               int d_hc, int d_cg, bool bf16, hipStream_t s) {
  const dim3 grid((d_hc + 15) / 16, H);
  const size_t lds = sizeof(float) * kRowsPerPass * d_cg;
  if (bf16)
    up_v_generic_kernel<uint16_t><<<grid, kThreads, lds, s>>>(
        static_cast<const uint16_t*>(o_lat), static_cast<const uint16_t*>(w_uv),
        static_cast<uint16_t*>(out), T, H, d_hc, d_cg);
  else
    up_v_generic_kernel<float><<<grid, kThreads, lds, s>>>(
        static_cast<const float*>(o_lat), static_cast<const float*>(w_uv), static_cast<float*>(out),
        T, H, d_hc, d_cg);
  return hipGetLastError();
}

hipError_t launch_decode_generic(const DecodeArgs& a, bool bf16, hipStream_t s) {
  const dim3 grid(a.total_q, a.num_splits, a.heads);
  if (bf16)
    decode_generic_kernel<uint16_t><<<grid, kThreads, 0, s>>>(a);
  else
    decode_generic_kernel<float><<<grid, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

// Many-row form of the same merge, for launches whose partial bytes dominate (thousands
// of rows).  Each wave walks `rpw` consecutive rows.  A row's LSEs are requested while
// the previous row's partials are in flight, and only the partials of splits that hold
// keys (LSE > -inf) are read.  Splits past a short sequence's end are never written, so
// a batch of unequal lengths reads just the written partials, still at one memory round
// trip per row.  Needs S <= kChunk (all splits of a row in one request).
template <typename T, int kDcg, int kChunk>
__global__ void __launch_bounds__(kThreads)
combine_rows_kernel(const T* __restrict__ o_part, const float* __restrict__ lse_part,
                    T* __restrict__ o_lat, float* __restrict__ lse_out, int rows, int S, int rpw) {
  constexpr int kE = kDcg / 64;
  constexpr int kW = kE * static_cast<int>(sizeof(T)) / 4;
  static_assert(kChunk * kW <= 128 && kChunk <= 64, "one request of at most 128 words per lane");
  const int lane = threadIdx.x & 63;
  const size_t wv = static_cast<size_t>(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
  size_t r = wv * static_cast<size_t>(rpw);
  if (r >= static_cast<size_t>(rows)) return;
  const size_t r_end = r + rpw < static_cast<size_t>(rows) ? r + rpw : static_cast<size_t>(rows);
  float l_next = lane < S ? lse_part[r * S + lane] : -INFINITY;
  for (; r < r_end; ++r) {
    const float l_lane = l_next;
    // Splits with keys, as a wave-uniform bit mask (lanes >= S hold -inf).
    const uint64_t live = __builtin_amdgcn_ballot_w64(l_lane != -INFINITY);
    const T* base = o_part + r * S * kDcg + kE * lane;
    uint32_t x[kChunk][kW];
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      if ((live >> u) & 1) load_words<T, kW>(base + static_cast<size_t>(u) * kDcg, x[u]);
    if (r + 1 < r_end) l_next = lane < S ? lse_part[(r + 1) * S + lane] : -INFINITY;
    float mx = l_lane;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    float acc[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] = 0.f;
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      if ((live >> u) & 1) {
        const float l = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_lane), u));
        const float wt = expf(l - mx);
        sum += wt;
#pragma unroll
        for (int e = 0; e < kE; ++e) acc[e] += wt * word_elem<T>(x[u], e);
      }
    }
    const float inv = live == 0 ? 0.f : 1.f / sum;
    uint32_t y[kW];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < kW; ++w)
        y[w] = static_cast<uint32_t>(f32_to_bf16(acc[2 * w] * inv)) |
               (static_cast<uint32_t>(f32_to_bf16(acc[2 * w + 1] * inv)) << 16);
    } else {
#pragma unroll
      for (int w = 0; w < kW; ++w) y[w] = __float_as_uint(acc[w] * inv);
    }
    T* dst = o_lat + r * kDcg + kE * lane;
    if constexpr (kW == 2) {
      *reinterpret_cast<uint2*>(dst) = uint2{y[0], y[1]};
    } else {
#pragma unroll
      for (int i = 0; i < kW / 4; ++i)
        reinterpret_cast<uint4*>(dst)[i] = uint4{y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]};
    }
    if (lane == 0 && lse_out != nullptr) lse_out[r] = live == 0 ? -INFINITY : mx + logf(sum);
  }
}

// Waves per SIMD that a many-row combine keeps resident, from its partial registers per
// lane (64 words: about 105 VGPRs; 96: about 140; 128: about 170).
constexpr int combine_rows_occupancy(int words) { return words <= 64 ? 4 : (words <= 96 ? 3 : 2); }

// The many-row form, when the rows outnumber the waves the chip keeps resident (its
// 1024 SIMDs times the occupancy above): then each wave takes rpw >= 2 rows.  Returns
// false (nothing launched) when one round of waves covers the rows.
template <typename T, int kDcg, int kChunk>
bool launch_combine_rows(const T* o_part, const float* lse_part, T* o_lat, float* lse_out, int rows,
                         int S, hipStream_t s) {
  constexpr int kWords = kChunk * (kDcg / 64) * static_cast<int>(sizeof(T)) / 4;
  constexpr int kResident = 1024 * combine_rows_occupancy(kWords);
  if (rows <= kResident) return false;
  const int rpw = (rows + kResident - 1) / kResident;
  const int waves = (rows + rpw - 1) / rpw;
  const dim3 grid((waves + 3) / 4);
  combine_rows_kernel<T, kDcg, kChunk><<<grid, kThreads, 0, s>>>(o_part, lse_part, o_lat, lse_out, rows, S, rpw);
  return true;
}

template <typename T, int kDcg>
hipError_t launch_combine_vec(const T* o_part, const float* lse_part, T* o_lat, float* lse_out,
                              int rows, int S, hipStream_t s) {
  constexpr int kMax = combine_max_chunk<T, kDcg>();
  bool done = false;
  if (S <= 8)
    done = launch_combine_rows<T, kDcg, 8>(o_part, lse_part, o_lat, lse_out, rows, S, s);
  else if (S <= 16 && kMax >= 16)
    done = launch_combine_rows<T, kDcg, 16>(o_part, lse_part, o_lat, lse_out, rows, S, s);
  else if (S <= 24 && kMax >= 24)
    done = launch_combine_rows<T, kDcg, (kMax >= 24 ? 24 : 8)>(o_part, lse_part, o_lat, lse_out, rows, S, s);
  else if (S <= 32 && kMax >= 32)
    done = launch_combine_rows<T, kDcg, (kMax >= 32 ? 32 : 8)>(o_part, lse_part, o_lat, lse_out, rows, S, s);
  if (done) return hipGetLastError();
  const dim3 grid((rows + 3) / 4);
  if (S <= 8)
    combine_vec_kernel<T, kDcg, 8><<<grid, kThreads, 0, s>>>(o_part, lse_part, o_lat, lse_out, rows, S);
  else if (S <= 16 || kMax == 16)
    combine_vec_kernel<T, kDcg, 16><<<grid, kThreads, 0, s>>>(o_part, lse_part, o_lat, lse_out, rows, S);
  else
    combine_vec_kernel<T, kDcg, kMax><<<grid, kThreads, 0, s>>>(o_part, lse_part, o_lat, lse_out, rows, S);
  return hipGetLastError();
}

hipError_t launch_combine(const void* o_part_v, const float* lse_part, void* o_lat, float* lse_out,
                          int T, int H, int d_cg, int S, bool bf16, hipStream_t s) {
  const int rows = T * H;
  const auto* op16 = static_cast<const uint16_t*>(o_part_v);
  const auto* op32 = static_cast<const float*>(o_part_v);
  if (d_cg == 512 || d_cg == 256) {
    if (bf16) {
      auto* o = static_cast<uint16_t*>(o_lat);
      return d_cg == 512 ? launch_combine_vec<uint16_t, 512>(op16, lse_part, o, lse_out, rows, S, s)
                         : launch_combine_vec<uint16_t, 256>(op16, lse_part, o, lse_out, rows, S, s);
    }
    auto* o = static_cast<float*>(o_lat);
    return d_cg == 512 ? launch_combine_vec<float, 512>(op32, lse_part, o, lse_out, rows, S, s)
                       : launch_combine_vec<float, 256>(op32, lse_part, o, lse_out, rows, S, s);
  }
  const dim3 grid(static_cast<unsigned>(T) * H);
  if (bf16)
    combine_kernel<uint16_t><<<grid, kThreads, 0, s>>>(op16, lse_part, static_cast<uint16_t*>(o_lat),
                                                       lse_out, d_cg, S);
  else
    combine_kernel<float><<<grid, kThreads, 0, s>>>(op32, lse_part, static_cast<float*>(o_lat),
                                                    lse_out, d_cg, S);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* cos_out, float* sin_out, int max_pos, int d_R, double base,
                             hipStream_t s) {
  const int half = d_R / 2;
  const size_t n = static_cast<size_t>(max_pos) * half;
  const dim3 grid(static_cast<unsigned>((n + kThreads - 1) / kThreads));
  rope_table_kernel<<<grid, kThreads, 0, s>>>(cos_out, sin_out, max_pos, half, base);
  return hipGetLastError();
}

}  // namespace mla
