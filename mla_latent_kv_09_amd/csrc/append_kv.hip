// Latent-cache append: writes the cache row of every new token of a decode step into
// its page (www.nxmr.cn/news/151634 §1: what a token stores per layer is its latent
// c_KV followed by its decoupled RoPE key k_R, the part that carries its position; §3:
// 64-token pages of bf16 rows, RoPE computed in fp32; §4: the fp32 table applied with
// fp32 multiply-adds).
//
// New token i of sequence b (packed row cu_q[b] + i) sits at position
// pos = seq_lens[b] - q_len_b + i, the position its query is rotated at, and goes to
// slot pos % 64 of physical page page_table[b][pos / 64].  The row written is
// [c_KV | RoPE(k_R, pos)]: the latent unchanged, the key's interleaved pairs
// (x0, x1) = (k[2k], k[2k+1]) rotated by the table angle of (pos, k):
//     y0 = x0 cos - x1 sin,  y1 = x0 sin + x1 cos   (fp32, rounded once to the storage type)
// which is the same arithmetic the decode applies to q_R, so scores see the relative
// rotation of query and key.
//
// Work: one wave per row, handled as 16-byte pieces (8 bf16 or 4 fp32 elements);
// consecutive lanes take consecutive pieces, so every load and store of a wave is one
// contiguous run.  The launcher requires d_c and d_R to be multiples of the piece
// length, so a piece is either all latent or all RoPE key and its pairs never
// straddle it.
#include <type_traits>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

__device__ __forceinline__ void rotate_pairs(float* x, int n, const float* cs, const float* sn) {
#pragma unroll
  for (int i = 0; i < n / 2; ++i) {
    const float x0 = x[2 * i], x1 = x[2 * i + 1];
    x[2 * i] = fmaf(x0, cs[i], -x1 * sn[i]);
    x[2 * i + 1] = fmaf(x0, sn[i], x1 * cs[i]);
  }
}

constexpr int kBlock = 256;  // 4 waves, one row each

// One wave per row.  The row's pieces are loaded first (lane l takes pieces l and
// 64 + l: the 72 pieces of a 576-element bf16 row in one pass), then the wave-uniform
// chain that places the row (query offsets, length, page id) runs on scalar loads,
// which the pieces' vector loads do not wait behind, then the RoPE pieces read their
// table row, rotate, and every piece is stored.
template <bool kBf16>
__global__ void __launch_bounds__(kBlock) append_kv_kernel(
    const typename std::conditional<kBf16, uint16_t, float>::type* __restrict__ c_new,
    const typename std::conditional<kBf16, uint16_t, float>::type* __restrict__ k_new,
    typename std::conditional<kBf16, uint16_t, float>::type* __restrict__ kv,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, int rope_max_pos, int batch, int total_q, int max_pages,
    int num_pool_pages, int d_c, int d_R, int page_size) {
  using T = typename std::conditional<kBf16, uint16_t, float>::type;
  constexpr int kE = 16 / sizeof(T);  // elements per 16-byte piece
  const int row_elems = d_c + d_R;
  const int pieces = row_elems / kE;
  const int c_pieces = d_c / kE;
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * (kBlock / 64) +
                                               static_cast<int>(threadIdx.x >> 6));
  if (t >= total_q) return;

  for (int base = 0; base < pieces; base += 128) {
    const int p0 = base + lane, p1 = base + 64 + lane;
    auto src = [&](int pc) {
      return pc < c_pieces ? c_new + static_cast<size_t>(t) * d_c + pc * kE
                           : k_new + static_cast<size_t>(t) * d_R + (pc - c_pieces) * kE;
    };
    uint4 v0{}, v1{};
    if (p0 < pieces) v0 = *reinterpret_cast<const uint4*>(src(p0));
    if (p1 < pieces) v1 = *reinterpret_cast<const uint4*>(src(p1));

    // Where the row goes (wave-uniform).
    const int b = find_seq(cu_q, batch, t);
    const int q0 = cu_q[b];
    const int q_len = cu_q[b + 1] - q0;
    const int cap = max_pages * page_size;
    int L = seq_lens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int pos = L - q_len + (t - q0);
    if (pos < 0 || pos >= cap) return;  // lengths shorter than q_len: nothing to write
    const int page = clamp_page(page_table[static_cast<size_t>(b) * max_pages + pos / page_size],
                                num_pool_pages);
    T* dst = kv + (static_cast<size_t>(page) * page_size + pos % page_size) * row_elems;

    auto put = [&](int pc, const uint4& v) {
      if (pc >= pieces) return;
      if (pc < c_pieces) {  // latent piece: copied as stored
        *reinterpret_cast<uint4*>(dst + pc * kE) = v;
        return;
      }
      float x[kE];
      const T* xs = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int e = 0; e < kE; ++e) x[e] = load_elem(xs, e);
      if (rope_cos != nullptr) {
        const int p = min(pos, rope_max_pos - 1);
        const size_t off = static_cast<size_t>(p) * (d_R / 2) + (pc - c_pieces) * (kE / 2);
        float cs[kE / 2], sn[kE / 2];
#pragma unroll
        for (int i = 0; i < kE / 2; ++i) {
          cs[i] = rope_cos[off + i];
          sn[i] = rope_sin[off + i];
        }
        rotate_pairs(x, kE, cs, sn);
      }
      uint4 o;
      T* os = reinterpret_cast<T*>(&o);
#pragma unroll
      for (int e = 0; e < kE; ++e) store_elem(os, e, x[e]);
      *reinterpret_cast<uint4*>(dst + pc * kE) = o;
    };
    put(p0, v0);
    put(p1, v1);
  }
}

// Nearest E4M3 code to x, ties to the even code, magnitudes at or past 448 saturating to
// 448, NaN to 0x7F, the sign bit taken from x (E4M3: 1 sign, 4 exponent bits with bias
// 7, 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6).
__device__ __forceinline__ uint32_t e4m3_from_f32(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;          // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;  // |x| >= 448, infinities included
  if (a < 0x3c800000u) {                      // |x| < 2^-6: steps of 2^-9, 8 steps = 2^-6 = 0x08
    return sign | static_cast<uint32_t>(rintf(__uint_as_float(a) * 512.f));
  }
  uint32_t e = (a >> 23) - 120u;              // biased E4M3 exponent: (E - 127) + 7
  uint32_t m = (a >> 20) & 7u;                // top 3 of the 23 mantissa bits
  const uint32_t rest = a & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ++m;
  if (m == 8u) {
    m = 0;
    ++e;
  }
  const uint32_t code = (e << 3) | m;
  return sign | (code > 0x7eu ? 0x7eu : code);
}

// FP8 cache append: one wave per new token row.  The page holds the latent codes
// [64][d_c] (E4M3), then k_R [64][d_R] (bf16), then one float32 scale per token; the
// row's latent gets scale = 2^e, e the smallest integer with amax <= 448 * 2^e clamped to
// [-124, 117] (e = 0 for an all-zero row), and code_i = e4m3(x_i * 2^-e), an exact
// product; k_R is rotated at the token's position as in the bf16 append.  With amax in
// [2^k, 2^(k+1)) (k from its exponent field) e is k - 8 when amax <= 1.75 * 2^k = 448 * 2^(k-8)
// and k - 7 otherwise; a subnormal amax takes the lower clamp.  Lane l takes latent elements 8l .. 8l+7 and
// k_R elements 8l .. 8l+7 (the launcher requires d_c <= 512, d_R <= 512, both multiples
// of 8).
__global__ void __launch_bounds__(kBlock) append_kv_fp8_kernel(
    const uint16_t* __restrict__ c_new, const uint16_t* __restrict__ k_new, uint8_t* __restrict__ kv,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, int rope_max_pos, int batch, int total_q, int max_pages,
    int num_pool_pages, int d_c, int d_R, int page_size) {
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * (kBlock / 64) +
                                               static_cast<int>(threadIdx.x >> 6));
  if (t >= total_q) return;
  const bool has_c = lane < d_c / 8, has_k = lane < d_R / 8;
  uint4 cv{}, kvv{};
  if (has_c) cv = *reinterpret_cast<const uint4*>(c_new + static_cast<size_t>(t) * d_c + 8 * lane);
  if (has_k) kvv = *reinterpret_cast<const uint4*>(k_new + static_cast<size_t>(t) * d_R + 8 * lane);

  const int b = find_seq(cu_q, batch, t);
  const int q0 = cu_q[b];
  const int q_len = cu_q[b + 1] - q0;
  const int cap = max_pages * page_size;
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int pos = L - q_len + (t - q0);
  if (pos < 0 || pos >= cap) return;
  const int page = clamp_page(page_table[static_cast<size_t>(b) * max_pages + pos / page_size],
                              num_pool_pages);
  const int slot = pos % page_size;
  uint8_t* pg = kv + static_cast<size_t>(page) * page_size * (d_c + 2 * d_R + 4);

  // Latent: row maximum over the wave, then the codes.
  float x[8];
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(&cv);
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = bf16_to_f32(xs[e]);
    amax = fmaxf(amax, fabsf(x[e]));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  int sexp = 0;  // e of scale = 2^e
  if (amax > 0.f) {
    const int E = static_cast<int>(__float_as_uint(amax) >> 23);  // amax >= 0: no sign bit
    if (E == 0) {
      sexp = -124;
    } else {
      const float lim = __uint_as_float(static_cast<uint32_t>(E) << 23) * 1.75f;  // 1.75 * 2^k, exact
      sexp = amax <= lim ? E - 127 - 8 : E - 127 - 7;
      sexp = sexp < -124 ? -124 : (sexp > 117 ? 117 : sexp);
    }
  }
  const float scale = __uint_as_float(static_cast<uint32_t>(127 + sexp) << 23);
  const float inv = __uint_as_float(static_cast<uint32_t>(127 - sexp) << 23);
  if (has_c) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w0 |= e4m3_from_f32(x[e] * inv) << (8 * e);
      w1 |= e4m3_from_f32(x[4 + e] * inv) << (8 * e);
    }
    *reinterpret_cast<uint2*>(pg + static_cast<size_t>(slot) * d_c + 8 * lane) = uint2{w0, w1};
  }
  if (has_k) {
    float k[8];
    const uint16_t* ks = reinterpret_cast<const uint16_t*>(&kvv);
#pragma unroll
    for (int e = 0; e < 8; ++e) k[e] = bf16_to_f32(ks[e]);
    if (rope_cos != nullptr) {
      const int p = min(pos, rope_max_pos - 1);
      const size_t off = static_cast<size_t>(p) * (d_R / 2) + 4 * lane;
      float cs[4], sn[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cs[i] = rope_cos[off + i];
        sn[i] = rope_sin[off + i];
      }
      rotate_pairs(k, 8, cs, sn);
    }
    uint4 o;
    uint16_t* os = reinterpret_cast<uint16_t*>(&o);
#pragma unroll
    for (int e = 0; e < 8; ++e) os[e] = f32_to_bf16(k[e]);
    *reinterpret_cast<uint4*>(pg + static_cast<size_t>(page_size) * d_c +
                              (static_cast<size_t>(slot) * d_R + 8 * lane) * 2) = o;
  }
  if (lane == 0)
    *reinterpret_cast<float*>(pg + static_cast<size_t>(page_size) * (d_c + 2 * d_R) + 4 * slot) = scale;
}

// Nearest E2M1 code to the magnitude m (ties to the even code, past 6 saturating to 6):
// the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0 .. 7) and the midpoints between
// neighbours 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5; a midpoint goes to the even code, so
// the comparison is inclusive below an even code and strict below an odd one.
__device__ __forceinline__ uint32_t e2m1_magnitude_code(float m) {
  return static_cast<uint32_t>(m > 0.25f) + static_cast<uint32_t>(m >= 0.75f) +
         static_cast<uint32_t>(m > 1.25f) + static_cast<uint32_t>(m >= 1.75f) +
         static_cast<uint32_t>(m > 2.5f) + static_cast<uint32_t>(m >= 3.5f) +
         static_cast<uint32_t>(m > 5.0f);
}

// MXFP4 cache append (the OCP microscaling 4-bit format): one wave per new token row.
// The page holds the packed codes [64][d_c / 2] (byte j: element 2j in the low nibble,
// 2j + 1 in the high one), then k_R [64][d_R] (bf16), then the scale bytes [64][d_c / 32]
// (E8M0, one per 32 latent elements).  Lane l takes latent elements 8l .. 8l+7, so lanes
// 4k .. 4k+3 hold block k.  Its shared exponent is e = floor(log2 amax) - 2 (2: the
// exponent of E2M1's largest value, 6 = 1.5 * 2^2), at least -126, and its scale byte
// e + 127 = max(E - 2, 1) with E the float32 exponent field of amax (0 for a zero or
// subnormal amax).  Each code is the E2M1 value nearest to x * 2^-e, an exact product,
// with x's sign.  k_R is rotated at the token's position as in the bf16 append.  The
// launcher requires d_c a multiple of 32 and d_R of 8, both at most 512.
__global__ void __launch_bounds__(kBlock) append_kv_mxfp4_kernel(
    const uint16_t* __restrict__ c_new, const uint16_t* __restrict__ k_new, uint8_t* __restrict__ kv,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ cu_q, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, int rope_max_pos, int batch, int total_q, int max_pages,
    int num_pool_pages, int d_c, int d_R, int page_size) {
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * (kBlock / 64) +
                                               static_cast<int>(threadIdx.x >> 6));
  if (t >= total_q) return;
  const bool has_c = lane < d_c / 8, has_k = lane < d_R / 8;
  uint4 cv{}, kvv{};
  if (has_c) cv = *reinterpret_cast<const uint4*>(c_new + static_cast<size_t>(t) * d_c + 8 * lane);
  if (has_k) kvv = *reinterpret_cast<const uint4*>(k_new + static_cast<size_t>(t) * d_R + 8 * lane);

  const int b = find_seq(cu_q, batch, t);
  const int q0 = cu_q[b];
  const int q_len = cu_q[b + 1] - q0;
  const int cap = max_pages * page_size;
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int pos = L - q_len + (t - q0);
  if (pos < 0 || pos >= cap) return;
  const int page = clamp_page(page_table[static_cast<size_t>(b) * max_pages + pos / page_size],
                              num_pool_pages);
  const int slot = pos % page_size;
  const size_t row_codes = static_cast<size_t>(d_c) / 2, row_scales = static_cast<size_t>(d_c) / 32;
  uint8_t* pg = kv + static_cast<size_t>(page) * page_size * (row_codes + 2 * d_R + row_scales);

  // Latent: the block maximum over lanes 4k .. 4k+3, then the codes.
  float x[8];
  const uint16_t* xs = reinterpret_cast<const uint16_t*>(&cv);
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    x[e] = bf16_to_f32(xs[e]);
    amax = fmaxf(amax, fabsf(x[e]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int E = static_cast<int>(__float_as_uint(amax) >> 23);  // amax >= 0: no sign bit
  const int sbyte = E - 2 > 1 ? E - 2 : 1;                        // e + 127, e >= -126
  const float inv = __uint_as_float(static_cast<uint32_t>(254 - sbyte) << 23);  // 2^-e
  if (has_c) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float y = x[e] * inv;  // exact: a power of two, |y| < 8
      const uint32_t code = e2m1_magnitude_code(fabsf(y)) | ((__float_as_uint(y) >> 28) & 8u);
      w |= code << (4 * e);
    }
    *reinterpret_cast<uint32_t*>(pg + static_cast<size_t>(slot) * row_codes + 4 * lane) = w;
    if ((lane & 3) == 0)
      pg[static_cast<size_t>(page_size) * (row_codes + 2 * d_R) + slot * row_scales + (lane >> 2)] =
          static_cast<uint8_t>(sbyte);
  }
  if (has_k) {
    float k[8];
    const uint16_t* ks = reinterpret_cast<const uint16_t*>(&kvv);
#pragma unroll
    for (int e = 0; e < 8; ++e) k[e] = bf16_to_f32(ks[e]);
    if (rope_cos != nullptr) {
      const int p = min(pos, rope_max_pos - 1);
      const size_t off = static_cast<size_t>(p) * (d_R / 2) + 4 * lane;
      float cs[4], sn[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cs[i] = rope_cos[off + i];
        sn[i] = rope_sin[off + i];
      }
      rotate_pairs(k, 8, cs, sn);
    }
    uint4 o;
    uint16_t* os = reinterpret_cast<uint16_t*>(&o);
#pragma unroll
    for (int e = 0; e < 8; ++e) os[e] = f32_to_bf16(k[e]);
    *reinterpret_cast<uint4*>(pg + static_cast<size_t>(page_size) * row_codes +
                              (static_cast<size_t>(slot) * d_R + 8 * lane) * 2) = o;
  }
}

}  // namespace

hipError_t launch_append_kv_fp8(const AppendArgs& a, hipStream_t s) {
  const long long rows_per_block = kBlock / 64;
  const dim3 grid(static_cast<unsigned>((a.total_q + rows_per_block - 1) / rows_per_block));
  append_kv_fp8_kernel<<<grid, kBlock, 0, s>>>(
      static_cast<const uint16_t*>(a.c_new), static_cast<const uint16_t*>(a.k_new),
      static_cast<uint8_t*>(a.kv), a.page_table, a.seq_lens, a.cu_q, a.rope_cos, a.rope_sin,
      a.rope_max_pos, a.batch, a.total_q, a.max_pages, a.num_pool_pages, a.d_c, a.d_R,
      a.page_size);
  return hipGetLastError();
}

hipError_t launch_append_kv_mxfp4(const AppendArgs& a, hipStream_t s) {
  const long long rows_per_block = kBlock / 64;
  const dim3 grid(static_cast<unsigned>((a.total_q + rows_per_block - 1) / rows_per_block));
  append_kv_mxfp4_kernel<<<grid, kBlock, 0, s>>>(
      static_cast<const uint16_t*>(a.c_new), static_cast<const uint16_t*>(a.k_new),
      static_cast<uint8_t*>(a.kv), a.page_table, a.seq_lens, a.cu_q, a.rope_cos, a.rope_sin,
      a.rope_max_pos, a.batch, a.total_q, a.max_pages, a.num_pool_pages, a.d_c, a.d_R,
      a.page_size);
  return hipGetLastError();
}

hipError_t launch_append_kv(const AppendArgs& a, bool bf16, hipStream_t s) {
  const long long rows_per_block = kBlock / 64;
  const dim3 grid(static_cast<unsigned>((a.total_q + rows_per_block - 1) / rows_per_block));
  if (bf16)
    append_kv_kernel<true><<<grid, kBlock, 0, s>>>(
        static_cast<const uint16_t*>(a.c_new), static_cast<const uint16_t*>(a.k_new),
        static_cast<uint16_t*>(a.kv), a.page_table, a.seq_lens, a.cu_q, a.rope_cos, a.rope_sin,
        a.rope_max_pos, a.batch, a.total_q, a.max_pages, a.num_pool_pages, a.d_c, a.d_R,
        a.page_size);
  else
    append_kv_kernel<false><<<grid, kBlock, 0, s>>>(
        static_cast<const float*>(a.c_new), static_cast<const float*>(a.k_new),
        static_cast<float*>(a.kv), a.page_table, a.seq_lens, a.cu_q, a.rope_cos, a.rope_sin,
        a.rope_max_pos, a.batch, a.total_q, a.max_pages, a.num_pool_pages, a.d_c, a.d_R,
        a.page_size);
  return hipGetLastError();
}

}  // namespace mla
