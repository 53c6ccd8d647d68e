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
// weights.  up_v also comes fused with the split merge that produces its input
// (merge_up_v_kernel, mla_combine_up_v).  Tiles use v_mfma_f32_16x16x32_bf16 (M = 16 query rows per block),
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

// ---------------------------------------------------------------- split merge + up_v
// mla_combine followed by mla_up_v in one launch, for the shapes up_v_lds_kernel takes
// (bf16, d_hc a multiple of 64, d_cg 256 or 512) and up to 16 (d_cg 512) or 32 (d_cg
// 256) splits.  Same grid as up_v_lds_kernel (one workgroup per head and 64 output
// dims, the two workgroups of a head on one XCD), 16 waves.  The workgroup's
// [64 x d_cg] slice of W_UV[h] is staged in LDS (rows padded by 16 bytes, as the
// activation block).  Per 16-row block of query rows, wave w merges row t0 + w from the
// split partials exactly as the combine does (lane l owns columns kE l .. +kE-1, all of
// the row's partials requested together with its LSEs), rounds it to bf16 and puts it in
// the LDS block; then waves 0-3 take the block's MFMAs as up_v_lds_kernel (wave w: dims
// 16 w .. +15, one accumulator chain over the K-steps), with the W_UV operand from LDS.
// Sixteen merging waves keep four rows in flight per SIMD, which hides the merge's
// memory and reduction latency.  The arithmetic and its order are the combine's and
// then up_v's, so out (and o_latent / lse_out, written by the x = 0 workgroup of each
// head when given) are bit for bit those of the two calls; the merged rows need not go
// through memory, and a launch boundary goes.
constexpr int kMergeWaves = 16;

template <int kSteps, int kChunk>  // d_cg / 32, largest split count
__global__ void __launch_bounds__(kMergeWaves * 64)
merge_up_v_kernel(const uint16_t* __restrict__ o_part, const float* __restrict__ lse_part,
                  const uint16_t* __restrict__ w_uv, uint16_t* __restrict__ o_lat,
                  uint16_t* __restrict__ out, float* __restrict__ lse_out, int T, int H, int d_hc,
                  int S) {
  constexpr int d_cg = kSteps * 32;
  constexpr int kE = d_cg / 64;  // columns per lane in the merge
  constexpr int kW = kE / 2;     // 32-bit words per lane and split
  constexpr int kRowBytes = d_cg * 2 + 16;
  constexpr int kPieces = kUpCols * d_cg / 8 / (kMergeWaves * 64);  // 16-byte W pieces per thread
  static_assert(kChunk * kW <= 64, "at most 64 words of partials per lane");
  static_assert(kPieces * kMergeWaves * 64 * 8 == kUpCols * d_cg, "the W slice splits evenly");
  static_assert(kMergeWaves == 16, "one merged row per wave and 16-row block");
  __shared__ __attribute__((aligned(16))) char wsm[kUpCols * kRowBytes];
  __shared__ __attribute__((aligned(16))) char buf[16 * kRowBytes];
  const HeadTile ht = head_tile(d_hc / kUpCols, H);
  const int h = ht.head;
  const bool writer = ht.x == 0;  // writes o_latent and lse_out for this head
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, j = lane & 15;
  // W_UV[h][64 x + r][:] -> wsm row r; thread piece i = row (tid + 1024 i) / (d_cg / 8).
  bf16x8 wp[kPieces];
  const uint16_t* wslice = w_uv + (static_cast<size_t>(h) * d_hc + ht.x * kUpCols) * d_cg;
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int pc = tid + kMergeWaves * 64 * i;
    wp[i] = *reinterpret_cast<const bf16x8*>(wslice + static_cast<size_t>(pc) * 8);
  }
  bool staged = false;
  for (int t0 = 0; t0 < T; t0 += 16) {
    const int t = t0 + wave;
    const bool valid = t < T;
    const size_t row = static_cast<size_t>(valid ? t : 0) * H + h;
    const float l_lane = (valid && lane < S) ? lse_part[row * S + lane] : -INFINITY;
    uint32_t x[kChunk][kW];
    const uint16_t* base = o_part + row * S * d_cg + kE * lane;
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      if (valid && u < S) {
        if constexpr (kW == 4) {
          const uint4 v = *reinterpret_cast<const uint4*>(base + static_cast<size_t>(u) * d_cg);
          x[u][0] = v.x, x[u][1] = v.y, x[u][2] = v.z, x[u][3] = v.w;
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(base + static_cast<size_t>(u) * d_cg);
          x[u][0] = v.x, x[u][1] = v.y;
        }
      }
    if (!staged) {  // first block: the W slice into LDS while the partials are in flight
#pragma unroll
      for (int i = 0; i < kPieces; ++i) {
        const int pc = tid + kMergeWaves * 64 * i, r = pc / (d_cg / 8), ch = pc % (d_cg / 8);
        *reinterpret_cast<bf16x8*>(wsm + r * kRowBytes + ch * 16) = wp[i];
      }
      staged = true;
    }
    // The largest LSE of the row (lane u < S holds split u's): the same value as the
    // combine's butterfly, taken here with lane reads.
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      if (u < S) mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_lane), u)));
    float acc[kE];
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] = 0.f;
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const float l = u < S ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_lane), u))
                            : -INFINITY;
      const float wt = (l == -INFINITY || mx == -INFINITY) ? 0.f : expf(l - mx);
      sum += wt;
      if (wt != 0.f) {
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          const uint32_t wd = x[u][e >> 1];
          acc[e] += wt * __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
        }
      }
    }
    const float inv = mx == -INFINITY ? 0.f : 1.f / sum;
    uint32_t y[kW];
#pragma unroll
    for (int w = 0; w < kW; ++w)
      y[w] = static_cast<uint32_t>(f32_to_bf16(acc[2 * w] * inv)) |
             (static_cast<uint32_t>(f32_to_bf16(acc[2 * w + 1] * inv)) << 16);
    char* dst = buf + wave * kRowBytes + kE * 2 * lane;
    uint16_t* gdst = o_lat + (static_cast<size_t>(t) * H + h) * d_cg + kE * lane;
    if constexpr (kW == 4) {
      *reinterpret_cast<uint4*>(dst) = uint4{y[0], y[1], y[2], y[3]};
      if (writer && o_lat != nullptr && valid) *reinterpret_cast<uint4*>(gdst) = uint4{y[0], y[1], y[2], y[3]};
    } else {
      *reinterpret_cast<uint2*>(dst) = uint2{y[0], y[1]};
      if (writer && o_lat != nullptr && valid) *reinterpret_cast<uint2*>(gdst) = uint2{y[0], y[1]};
    }
    if (writer && lse_out != nullptr && lane == 0 && valid)
      lse_out[static_cast<size_t>(t) * H + h] = mx == -INFINITY ? -INFINITY : mx + logf(sum);
    __syncthreads();
    if (wave < 4) {
      // A: row j of the block, columns 32 k + 8 g .. +7; B: W_UV row 16 wave + j, same columns.
      const char* arow = buf + j * kRowBytes + 16 * g;
      const char* brow = wsm + (16 * wave + j) * kRowBytes + 16 * g;
      f32x4 o4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < kSteps; ++k)
        o4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(arow + 64 * k),
                                                     *reinterpret_cast<const bf16x8*>(brow + 64 * k), o4,
                                                     0, 0, 0);
      const int d = ht.x * kUpCols + 16 * wave + j;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = t0 + 4 * g + i;
        if (tt < T) out[(static_cast<size_t>(tt) * H + h) * d_hc + d] = f32_to_bf16(o4[i]);
      }
    }
    __syncthreads();  // the block buffer is rewritten by the next block's merge
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

bool merge_up_v_supported(int d_hc, int d_cg, int S, bool bf16) {
  return bf16 && d_hc % kUpCols == 0 && S >= 1 &&
         ((d_cg == 512 && S <= 16) || (d_cg == 256 && S <= 32));
}

hipError_t launch_merge_up_v(const void* o_part, const float* lse_part, const void* w_uv, void* o_lat,
                             void* out, float* lse_out, int T, int H, int d_hc, int d_cg, int S,
                             hipStream_t s) {
  const auto* op = static_cast<const uint16_t*>(o_part);
  const auto* wt = static_cast<const uint16_t*>(w_uv);
  auto* ol = static_cast<uint16_t*>(o_lat);
  auto* dst = static_cast<uint16_t*>(out);
  const dim3 grid((d_hc / kUpCols) * H), block(kMergeWaves * 64);
  if (d_cg == 512) {
    if (S <= 8)
      merge_up_v_kernel<16, 8><<<grid, block, 0, s>>>(op, lse_part, wt, ol, dst, lse_out, T, H, d_hc, S);
    else
      merge_up_v_kernel<16, 16><<<grid, block, 0, s>>>(op, lse_part, wt, ol, dst, lse_out, T, H, d_hc, S);
  } else {
    if (S <= 16)
      merge_up_v_kernel<8, 16><<<grid, block, 0, s>>>(op, lse_part, wt, ol, dst, lse_out, T, H, d_hc, S);
    else
      merge_up_v_kernel<8, 32><<<grid, block, 0, s>>>(op, lse_part, wt, ol, dst, lse_out, T, H, d_hc, S);
  }
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
