// The two per-head projections of the absorbed MLA decode step on bf16 MFMA (gfx950):
//
//   absorb  q_abs[t,h,:] = q_c[t,h,:] . W_UK[h]      W_UK [H, d_hc, d_cg]
//           (nxmr.cn/news/151634 §1, §4 path B: fold W_UK into the query so scores are
//           taken against the cached latent and K is never re-expanded)
//   up_v    out[t,h,:]   = W_UV[h] . o_latent[t,h,:]  W_UV [H, d_hc, d_cg]
//           (m.xxqk.cn/news/443191 §2.4: the latent is mapped back up to the value space)
//
// Both are batched GEMMs with small M (the T query rows) and read each weight
// element exactly once, so they are bound by streaming the 2*H*d_hc*d_cg bytes of
// weights.  Tiles use v_mfma_f32_16x16x32_bf16 (M = 16 query rows per block),
// fp32 accumulation, one rounding to bf16 on the way out.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// Workgroup -> (x, head) for a 1-D launch of nx * n_heads workgroups.  The dispatcher
// deals workgroups to the 8 XCDs of the chip in turn (id mod 8), and every XCD has its
// own L2; the nx workgroups of one head read the same activation rows, so they are
// placed on one XCD (ids with the same residue mod 8, consecutive in that XCD's order)
// and the rows come from HBM once instead of once per XCD.  Head counts that are not a
// multiple of 8 keep the plain order.
struct HeadTile { int x, head; };
__device__ __forceinline__ HeadTile head_tile(int nx, int n_heads) {
  const int L = blockIdx.x;
  if (n_heads % 8 != 0) return {L % nx, L / nx};
  const int r = L >> 3;
  return {r % nx, (r / nx) * 8 + (L & 7)};
}

// ---------------------------------------------------------------- up_v
// Two forms.  up_v_lds_kernel (below) shares each block of activation rows across a
// workgroup through LDS and is used whenever d_hc is a multiple of 64; this one, for the
// other shapes, loads its rows itself.
// One wave per (head h, 16 output dims d0..d0+15).  B operand = W_UV[h][d][c]:
// lane (n = d0 + l%16, k = 8*(l/16) + e) reads 16 contiguous bytes of row d, so
// the wave's 16 x d_cg weight slice goes straight from HBM into registers (once).
// A operand = o_latent[t][h][c], 16 bytes per lane, one M-block of 16 rows at a time.
// All loads of an M-block (the wave's weight slice and the block's activation rows)
// are issued before the first MFMA, so the kernel costs one memory round trip per
// block rather than one per K-step.
template <int kSteps>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ base, size_t row_stride,
                                          int row, int n_rows, bf16x8 (&a)[kSteps]) {
  const bool ok = row < n_rows;
  const uint16_t* p = base + static_cast<size_t>(ok ? row : 0) * row_stride;
#pragma unroll
  for (int k = 0; k < kSteps; ++k) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p + 32 * k);
    a[k] = ok ? v : bf16x8{};
  }
}

template <int kSteps>  // d_cg / 32
__global__ void __launch_bounds__(64)
up_v_mfma_kernel(const uint16_t* __restrict__ o_lat, const uint16_t* __restrict__ w_uv,
                 uint16_t* __restrict__ out, int T, int H, int d_hc) {
  constexpr int d_cg = kSteps * 32;
  const HeadTile ht = head_tile(d_hc / 16, H);
  const int h = ht.head;
  const int d0 = ht.x * 16;
  const int lane = threadIdx.x, g = lane >> 4, j = lane & 15;
  // A operand rows t0 + j of o_latent[t][h][:]; lane holds columns 32k + 8g .. +7.
  const uint16_t* abase = o_lat + static_cast<size_t>(h) * d_cg + 8 * g;
  const size_t astride = static_cast<size_t>(H) * d_cg;
  bf16x8 a[kSteps];
  load_rows<kSteps>(abase, astride, j, T, a);
  const uint16_t* wrow = w_uv + (static_cast<size_t>(h) * d_hc + d0 + j) * d_cg + 8 * g;
  bf16x8 b[kSteps];
#pragma unroll
  for (int k = 0; k < kSteps; ++k) b[k] = *reinterpret_cast<const bf16x8*>(wrow + 32 * k);
  for (int t0 = 0; t0 < T; t0 += 16) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kSteps; ++k) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k], b[k], acc, 0, 0, 0);
    if (t0 + 16 < T) load_rows<kSteps>(abase, astride, t0 + 16 + j, T, a);
    // D layout: lane holds rows t0 + 4g + i, column d0 + j.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i;
      if (t < T) out[(static_cast<size_t>(t) * H + h) * d_hc + d0 + j] = f32_to_bf16(acc[i]);
    }
  }
}

// up_v with shared activation rows: one workgroup of 4 waves per (head h, 64 output
// dims); wave w owns dims d0 = 64 x + 16 w .. +15, its W_UV slice in registers as above.
// Each 16-row block of o_latent[t][h][:] is read from memory once per workgroup, into
// LDS (rows padded by 16 bytes so the 16 rows of a fragment read start in different
// banks; two buffers, the next block requested while the current one is multiplied), and
// every wave takes its A fragments from there.  The rows of a head are then fetched
// d_hc / 64 times rather than d_hc / 16 times, which is what bounds up_v at large T.
constexpr int kUpCols = 64;

template <int kSteps>  // d_cg / 32
__global__ void __launch_bounds__(256)
up_v_lds_kernel(const uint16_t* __restrict__ o_lat, const uint16_t* __restrict__ w_uv,
                uint16_t* __restrict__ out, int T, int H, int d_hc) {
  constexpr int d_cg = kSteps * 32;
  constexpr int kRowBytes = d_cg * 2 + 16;
  constexpr int kBlockBytes = 16 * kRowBytes;
  constexpr int kChunks = d_cg / 8;                 // 16-byte pieces of one row
  constexpr int kPerThread = 16 * kChunks / 256;    // pieces of a block per thread
  static_assert(kPerThread * 256 == 16 * kChunks, "a block splits evenly over 256 threads");
  __shared__ __attribute__((aligned(16))) char buf[2 * kBlockBytes];
  const HeadTile ht = head_tile(d_hc / kUpCols, H);
  const int h = ht.head;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int d0 = ht.x * kUpCols + 16 * wave;
  const size_t astride = static_cast<size_t>(H) * d_cg;
  const uint16_t* abase = o_lat + static_cast<size_t>(h) * d_cg;
  // Piece i of this thread: block row (tid + 256 i) / kChunks, chunk (tid + 256 i) % kChunks.
  bf16x8 stage[kPerThread];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int pc = tid + 256 * i, row = pc / kChunks, ch = pc - row * kChunks;
      const int t = t0 + row;
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(abase + static_cast<size_t>(t < T ? t : 0) * astride + ch * 8);
      stage[i] = t < T ? v : bf16x8{};
    }
  };
  auto put = [&](int bi) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int pc = tid + 256 * i, row = pc / kChunks, ch = pc - row * kChunks;
      *reinterpret_cast<bf16x8*>(buf + bi * kBlockBytes + row * kRowBytes + ch * 16) = stage[i];
    }
  };
  fetch(0);
  const uint16_t* wrow = w_uv + (static_cast<size_t>(h) * d_hc + d0 + j) * d_cg + 8 * g;
  bf16x8 b[kSteps];
#pragma unroll
  for (int k = 0; k < kSteps; ++k) b[k] = *reinterpret_cast<const bf16x8*>(wrow + 32 * k);
  put(0);
  __syncthreads();
  int cur = 0;
  for (int t0 = 0; t0 < T; t0 += 16) {
    const bool more = t0 + 16 < T;
    if (more) fetch(t0 + 16);
    // A fragment, K-step k: row j, columns 32 k + 8 g .. +7.
    const char* arow = buf + cur * kBlockBytes + j * kRowBytes + 16 * g;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kSteps; ++k)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(arow + 64 * k), b[k],
                                                    acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i;
      if (t < T) out[(static_cast<size_t>(t) * H + h) * d_hc + d0 + j] = f32_to_bf16(acc[i]);
    }
    if (more) put(cur ^ 1);  // the other buffer: every wave left it at the last barrier
    __syncthreads();
    cur ^= 1;
  }
}

// ---------------------------------------------------------------- absorb
// One workgroup (4 waves) per (head h, 64 latent columns c0..c0+63).  The
// [d_hc x 64] slice of W_UK[h] is staged in LDS (rows padded to 144 B) and read
// back transposed with ds_read_b64_tr_b16, which hands each lane 4 consecutive d
// of one column c -- the K-contiguous B operand the MFMA needs.  Wave w owns
// columns c0 + 16w .. +15; A operand = q_c[t][h][d], 16 bytes per lane.
constexpr int kAbsCols = 64;
constexpr int kAbsRowBytes = kAbsCols * 2 + 16;

template <int kSteps>  // d_hc / 32
__global__ void __launch_bounds__(256)
absorb_mfma_kernel(const uint16_t* __restrict__ q_c, const uint16_t* __restrict__ w_uk,
                   uint16_t* __restrict__ q_abs, int T, int H, int d_cg) {
  constexpr int d_hc = kSteps * 32;
  // Query rows: each 16-row block of q_c[t][h][:] is read once per workgroup into LDS
  // (rows padded by 16 bytes, two buffers) and shared by the 4 waves, instead of once
  // per wave; one 16-byte piece per thread.
  constexpr int kARowBytes = d_hc * 2 + 16;
  constexpr int kABlockBytes = 16 * kARowBytes;
  constexpr int kAChunks = d_hc / 8;
  static_assert(16 * kAChunks == 256, "one piece of a query block per thread");
  __shared__ __attribute__((aligned(16))) char tile[d_hc * kAbsRowBytes];
  __shared__ __attribute__((aligned(16))) char abuf[2 * kABlockBytes];
  const HeadTile ht = head_tile(d_cg / kAbsCols, H);
  const int h = ht.head;
  const int c0 = ht.x * kAbsCols;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, j = lane & 15;
  const uint16_t* abase = q_c + static_cast<size_t>(h) * d_hc;
  const size_t astride = static_cast<size_t>(H) * d_hc;
  const int a_row = tid / kAChunks, a_ch = tid - a_row * kAChunks;
  auto fetch = [&](int t0) {
    const int t = t0 + a_row;
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(abase + static_cast<size_t>(t < T ? t : 0) * astride + a_ch * 8);
    return t < T ? v : bf16x8{};
  };
  auto put = [&](int bi, const bf16x8& v) {
    *reinterpret_cast<bf16x8*>(abuf + bi * kABlockBytes + a_row * kARowBytes + a_ch * 16) = v;
  };
  // The first block's query rows are requested before the weight tile, so both
  // round trips overlap.
  bf16x8 staged = fetch(0);
  // Stage the tile: thread -> (row d = tid/8 + 32r, chunk tid%8 of 8 columns).
  const uint16_t* wsrc = w_uk + static_cast<size_t>(h) * d_hc * d_cg + c0;
#pragma unroll
  for (int r = 0; r < d_hc / 32; ++r) {
    const int d = tid / 8 + 32 * r, ch = tid % 8;
    *reinterpret_cast<bf16x8*>(tile + d * kAbsRowBytes + ch * 16) =
        *reinterpret_cast<const bf16x8*>(wsrc + static_cast<size_t>(d) * d_cg + ch * 8);
  }
  put(0, staged);
  __syncthreads();
  // B fragments: K-step k covers d = 32k + 8g + {0..3} (first read) and {4..7} (second).
  const uint32_t tile_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)tile));
  const int col = 16 * wave + 4 * (j & 3);
  bf16x8 b[kSteps];
#pragma unroll
  for (int k = 0; k < kSteps; ++k) {
    const int d = 32 * k + 8 * g + (j >> 2);
    const uint32_t a1 = tile_base + d * kAbsRowBytes + col * 2;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(uintptr_t)(a1));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_bf16x4_t*)(uintptr_t)(a1 + 4 * kAbsRowBytes));
    b[k] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  const int cout = c0 + 16 * wave + j;
  int cur = 0;
  for (int t0 = 0; t0 < T; t0 += 16) {
    const bool more = t0 + 16 < T;
    if (more) staged = fetch(t0 + 16);
    // A fragment, K-step k: row j, dims 32 k + 8 g .. +7.
    const char* arow = abuf + cur * kABlockBytes + j * kARowBytes + 16 * g;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kSteps; ++k)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(arow + 64 * k), b[k],
                                                    acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * g + i;
      if (t < T) q_abs[(static_cast<size_t>(t) * H + h) * d_cg + cout] = f32_to_bf16(acc[i]);
    }
    if (more) put(cur ^ 1, staged);  // the other buffer: every wave left it at the last barrier
    __syncthreads();
    cur ^= 1;
  }
}

}  // namespace

bool up_v_mfma_supported(int d_hc, int d_cg, bool bf16) {
  return bf16 && d_hc % 16 == 0 && (d_cg == 256 || d_cg == 512);
}

bool absorb_mfma_supported(int d_hc, int d_cg, bool bf16) {
  return bf16 && d_hc == 128 && d_cg % kAbsCols == 0;
}

hipError_t launch_up_v_mfma(const void* o_lat, const void* w_uv, void* out, int T, int H, int d_hc,
                            int d_cg, hipStream_t s) {
  const auto* o = static_cast<const uint16_t*>(o_lat);
  const auto* wt = static_cast<const uint16_t*>(w_uv);
  auto* dst = static_cast<uint16_t*>(out);
  if (d_hc % kUpCols == 0) {
    const dim3 grid_l((d_hc / kUpCols) * H);
    if (d_cg == 512)
      up_v_lds_kernel<16><<<grid_l, 256, 0, s>>>(o, wt, dst, T, H, d_hc);
    else
      up_v_lds_kernel<8><<<grid_l, 256, 0, s>>>(o, wt, dst, T, H, d_hc);
    return hipGetLastError();
  }
  const dim3 grid((d_hc / 16) * H);
  if (d_cg == 512)
    up_v_mfma_kernel<16><<<grid, 64, 0, s>>>(o, wt, dst, T, H, d_hc);
  else
    up_v_mfma_kernel<8><<<grid, 64, 0, s>>>(o, wt, dst, T, H, d_hc);
  return hipGetLastError();
}

hipError_t launch_absorb_mfma(const void* q_c, const void* w_uk, void* q_abs, int T, int H,
                              int d_hc, int d_cg, hipStream_t s) {
  (void)d_hc;
  const dim3 grid((d_cg / kAbsCols) * H);
  absorb_mfma_kernel<4><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(q_c),
                                             static_cast<const uint16_t*>(w_uk),
                                             static_cast<uint16_t*>(q_abs), T, H, d_cg);
  return hipGetLastError();
}

}  // namespace mla
