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

}  // namespace

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
