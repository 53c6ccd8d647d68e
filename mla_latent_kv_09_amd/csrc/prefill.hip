// The decompressed (non-absorbed) branch of MLA attention, for batches with many query
// rows per sequence (prefill).  nxmr.cn/news/151634 §3 and §6: the absorbed form pays
// 2 (d_c + d_R) + 2 d_c flops per (query, key, head), the decompressed form 2 (d_hc + d_R)
// + 2 d_hc plus the up-projection of every key, which pays off once a sequence has enough
// query rows; the page sets the switch-over at 256 query rows (kPrefillThresh) and routes
// prefill to this branch and decode to the absorbed one.
//
// Two kernels, bf16 storage, fp32 accumulation, 32x32x16 MFMA:
//  1. decompress: for every cache row j of the batch's sequences and every head h,
//       K[j, h, :] = W_UK[h] c_j   and   V[j, h, :] = W_UV[h] c_j      (page §4 path A)
//     into a caller workspace indexed by physical cache row (page * 64 + slot), so the
//     attention reads keys and values through the same page table as the cache.
//  2. attention: for every query row and head, softmax over the visible keys of
//       (q_c . K[j, h] + RoPE(q_R) . k_R[j]) * scale   (k_R shared by all heads)
//     weighted sum of V[j, h]: the output [T, H, d_hc] directly (no W_UV step after).
#include <math.h>

#include <atomic>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;

constexpr int kTok = 64;
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kDhc = 128;
constexpr int kRowBytes = (kDc + kDr) * 2;  // one bf16 cache row
constexpr float kJump = 64.f;               // softmax reference move threshold (log2 units)

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ bf16x8 lds_read8(uint32_t a) { return *(const lds_bf16x8_t*)(uintptr_t)a; }
__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
  return bf16x8{static_cast<__bf16>(x[0]), static_cast<__bf16>(x[1]), static_cast<__bf16>(x[2]),
                static_cast<__bf16>(x[3]), static_cast<__bf16>(x[4]), static_cast<__bf16>(x[5]),
                static_cast<__bf16>(x[6]), static_cast<__bf16>(x[7])};
}
__device__ __forceinline__ float halves_max(float x) {  // lanes l and l ^ 32
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// global -> LDS copy, 16 bytes per active lane, lane i at LDS byte lds + 16 i.
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
// A page-table entry read through the constant address space.  The table is not written
// while these kernels run, and there a uniform index gives a scalar load, whose wait does
// not also wait for the copies in flight (vector loads and copies share one counter).
__device__ __forceinline__ int32_t table_entry(const int32_t* t, int i) {
  return ((const __attribute__((address_space(4))) int32_t*)t)[i];
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ 1. decompression
//
// Workgroup = 8 waves, one head h, a run of up to a.dec_pages pages of one sequence.  Wave w
// computes columns 32 (w % 4) .. +31 of K (w < 4) or V (w >= 4) for all 64 rows of each
// page, its 32-column slice of W_UK[h] or W_UV[h] (the B operand of all 32 K-steps) held in
// registers for the whole run.  Pages stream through two 64 KB LDS stages (the latent part
// of each row, 1 KB, chunk c at 16-byte position c ^ f(t), f(t) = (t[1:0] << 2) | t[3:2] |
// (t[4] << 4): conflict-free row-wise reads, as in the decode kernel).  Rows past the
// sequence's end copy row 0, so the workspace holds finite values there (masked later).
// Workgroup L: head L mod H (a page run's heads are consecutive, so their reads of the
// page meet in L2), run (L / H) mod runs_per_seq of sequence (L / H) / runs_per_seq.
constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
// Pages per workgroup: as many as keep about four workgroups per CU (8 to 64).  Each
// workgroup first loads its head's 256 KB of W_UK and W_UV slices, so longer runs load
// them fewer times: on prefill_b8_l4096, 8 pages per run took 1.34 ms, 16 took 1.23, 32
// took 1.19 and 64 took 1.17 ms (interleaved A/B).
constexpr int kDecMinPages = 8, kDecMaxPages = 64, kDecTargetGroups = 1024;
constexpr int kDecStage = kTok * kDc * 2;  // 64 KB
constexpr int kDecLds = 2 * kDecStage;

__device__ __forceinline__ uint32_t swz_f(int t) {
  return static_cast<uint32_t>(((t & 3) << 2) | ((t >> 2) & 3) | (t & 16));
}

__global__ void __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
decompress_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int L = static_cast<int>(blockIdx.x);
  // Uniform values computed by VALU divisions, moved to scalar registers so that the page
  // table is read with scalar loads (a vector load's wait would also wait for the copies).
  const int h = __builtin_amdgcn_readfirstlane(L % a.heads);
  const int u = __builtin_amdgcn_readfirstlane(L / a.heads);
  const int runs = (a.max_pages + a.dec_pages - 1) / a.dec_pages;
  const int b = __builtin_amdgcn_readfirstlane(u / runs), run = u - b * runs;
  const int cap = a.max_pages * kTok;
  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > cap ? cap : len);
  const int n_pages = (len + kTok - 1) / kTok;
  const int p0 = run * a.dec_pages, p1 = min(p0 + a.dec_pages, n_pages);
  if (p0 >= p1) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int part = wave >> 2, cb = wave & 3;  // K or V, 32-column block
  const uint16_t* wsrc = static_cast<const uint16_t*>(part ? a.w_uv : a.w_uk) +
                         (static_cast<size_t>(h) * kDhc + 32 * cb + n) * kDc + 8 * hh;
  bf16x8 wreg[kDc / 16];
#pragma unroll
  for (int ks = 0; ks < kDc / 16; ++ks) wreg[ks] = *reinterpret_cast<const bf16x8*>(wsrc + 16 * ks);

  const char* kv = static_cast<const char*>(a.kv);
  const int32_t* ptab = a.page_table + static_cast<size_t>(b) * a.max_pages;
  const uint32_t smem_base = lds_addr(smem);
  // Rows 8 w .. 8 w + 7 of a page are this wave's copies (one 1 KB latent row each).
  auto page_id = [&](int p) { return clamp_page(table_entry(ptab, p), a.num_pool_pages); };
  auto copy_page = [&](int p, int id, uint32_t stage) {
    const char* page = kv + static_cast<size_t>(id) * kTok * kRowBytes;
    const int nv = min(kTok, len - p * kTok);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int t = 8 * wave + r;
      const int src = t < nv ? t : 0;
      dma16(page + src * kRowBytes, static_cast<uint32_t>((lane ^ static_cast<int>(swz_f(t))) << 4),
            stage + t * 1024);
    }
  };
  // Page ids are read one page ahead of their copies; the stores of page p reuse its id.
  int id_cur = page_id(p0);
  copy_page(p0, id_cur, smem_base);
  int id_next = p0 + 1 < p1 ? page_id(p0 + 1) : 0;
  const uint32_t s_lane = static_cast<uint32_t>(n * 1024) | ((swz_f(n) ^ static_cast<uint32_t>(hh)) << 4);
  char* ws = static_cast<char*>(a.workspace) +
             (part ? static_cast<size_t>(a.num_pool_pages) * kTok * a.heads * kDhc * 2 : 0);
  int stage = 0;
  for (int p = p0; p < p1; ++p) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's copies of page p landed
    __syncthreads();                     // ... and every wave's; the other stage is free
    const uint32_t st = smem_base + stage * kDecStage;
    if (p + 1 < p1) copy_page(p + 1, id_next, smem_base + (stage ^ 1) * kDecStage);
    const int id_after = p + 2 < p1 ? page_id(p + 2) : 0;
    f32x16 acc[2] = {};
    const uint32_t sb = opaque(st + s_lane);
#pragma unroll
    for (int ks = 0; ks < kDc / 16; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const uint32_t addr = (sb ^ static_cast<uint32_t>((2 * ks & 31) << 4)) + 512 * (ks >> 4) + 32768 * mb;
        acc[mb] = mfma32(lds_read8(addr), wreg[ks], acc[mb]);
      }
    }
    // Keep eight reads in flight ahead of the products.
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 2 * kDc / 16 - 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    // Row 32 mb + 8 (r / 4) + 4 hh + r % 4, column 32 cb + n: 32 lanes write 64 contiguous bytes.
    // The page's base (uniform) and the row offsets (compile-time multiples of the uniform
    // row stride) are scalar; each lane adds one fixed 32-bit offset.
    const int phys = id_cur;
    const size_t row_elems = static_cast<size_t>(a.heads) * kDhc;
    __bf16* page_out = reinterpret_cast<__bf16*>(ws) + static_cast<size_t>(phys) * kTok * row_elems +
                       static_cast<size_t>(h) * kDhc + 32 * cb;
    const uint32_t lane_off = static_cast<uint32_t>(4 * hh) * static_cast<uint32_t>(row_elems) +
                              static_cast<uint32_t>(n);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = 32 * mb + 8 * (r >> 2) + (r & 3);  // the row less 4 hh
        page_out[static_cast<size_t>(c) * row_elems + lane_off] = static_cast<__bf16>(acc[mb][r]);
      }
    id_cur = id_next;
    id_next = id_after;
    stage ^= 1;
  }
}

// ------------------------------------------------------------------ 2. attention
//
// Workgroup = 4 waves, one (sequence b, head h) and a block of 128 query rows of b; wave w
// takes rows 32 w .. 32 w + 31 of the block, lane n (and n + 32) query n.  Keys go by
// 64-token pages from key 0 to the block's last visible key.  A stage holds the page's
// K rows [64][128] and V rows [64][128] (bf16, 256 B each, read from the workspace) and
// k_R rows [64][64] (from the cache), 40 KB; two stages.
//   scores  S^T[64 keys x 32 queries] = [K | k_R] . [q_c | RoPE(q_R)]^T, 12 K-steps per
//           32-key block (8 over K, 4 over k_R); A from LDS, B = the queries in registers.
//   softmax fp32 per query, the fixed-reference form of the decode kernel (a query's first
//           page maximum; terms up to 2^kJump against it; a jump past that moves it and
//           rescales what was accumulated).
//   output  O[32 queries x 128] += P . V over 4 K-steps of 16 keys: A = P from the score
//           registers (no LDS round trip), B = V^T through transposing reads.
// Stage swizzles (16-byte chunk c of row t at position c ^ key(t)), chosen with an LDS
// probe's bank-conflict counters on gfx950 (SQ_LDS_BANK_CONFLICT: 0 for each of the three
// reads below, 2-way for the layouts first used here):
//   K row (256 B):   swz_k(t) = (t & 15) ^ ((t >> 4) & 1)   row-wise reads of 32 keys
//   V row (256 B):   swz_v(t) = (t & 3) << 2                transposing reads, 8 keys x 4 chunks
//   k_R row (128 B): swz_r(t) = (t >> 1) & 7                row-wise reads of 32 keys
constexpr int kAttWaves = 4;
constexpr int kAttThreads = kAttWaves * 64;
constexpr int kQBlock = 32 * kAttWaves;
constexpr int kKBytes = kTok * kDhc * 2;  // 16 KB
constexpr int kRBytes = kTok * kDr * 2;   // 8 KB
constexpr int kAttStage = 2 * kKBytes + kRBytes;
constexpr int kAttLds = 2 * kAttStage;

__device__ __forceinline__ int swz_k(int t) { return (t & 15) ^ ((t >> 4) & 1); }
__device__ __forceinline__ int swz_v(int t) { return (t & 3) << 2; }
__device__ __forceinline__ int swz_r(int t) { return (t >> 1) & 7; }

__global__ void __launch_bounds__(kAttThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_attn_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int n_qb = (a.max_q_len + kQBlock - 1) / kQBlock;
  // Workgroup j runs on XCD j mod 8, and each XCD has its own L2.  Logical index L numbers
  // each XCD's workgroups consecutively (XCD x takes L = base_x .. base_x + count_x - 1),
  // so the query blocks of a (sequence, head) pair, which read the same K/V pages, share
  // one L2 instead of fetching every page once per XCD.
  const int L = xcd_grouped(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  // The n_qb query blocks of a pair take n_qb consecutive logical indices, in an order
  // rotated by 9 per pair.  Causal blocks differ in length (block i reads 2 (i + 1) pages),
  // and the dispatcher deals an XCD's workgroups to its shader engines in turn, holding
  // the line at an engine with no free slot: without a rotation the engines would keep
  // meeting the same block lengths, and the chip would run at about half its workgroup
  // slots (measured on the grid order first used here).  With it, each (XCD, engine) slot
  // sees every block length in turn (9 is coprime to n_qb's factors of 2).
  const int pair = L / n_qb;
  const int qb = (L % n_qb + 9 * pair) % n_qb;
  // Scalar registers for these uniform values (see the decompression kernel).
  const int h = __builtin_amdgcn_readfirstlane(pair % a.heads);
  const int b = __builtin_amdgcn_readfirstlane(pair / a.heads);
  const int q0 = a.cu_q[b], q1 = a.cu_q[b + 1];
  const int q_len = q1 - q0;
  if (qb * kQBlock >= q_len) return;
  const int cap = a.max_pages * kTok;
  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > cap ? cap : len);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int qi = qb * kQBlock + 32 * wave + n;  // query index within the sequence
  const bool q_valid = qi < q_len;
  const int t = q0 + (q_valid ? qi : 0);        // packed query row
  const int pos = len - q_len + (q_valid ? qi : 0);
  // Keys this block needs: up to the last valid query's position (causal), else all.
  const int last_q = min(q_len, (qb + 1) * kQBlock) - 1;
  const int k_end = a.causal ? min(len, len - q_len + last_q + 1) : len;
  const int n_pages = k_end > 0 ? (k_end + kTok - 1) / kTok : 0;
  const int vis = a.causal ? min(pos + 1, len) : len;  // this lane's query sees keys [0, vis)

  // Queries: q_c (K-steps 0..7) and the rotated q_R (K-steps 8..11), lane half hh taking
  // dims 8 hh .. 8 hh + 7 of each 16-dim K-step.
  bf16x8 q[12];
  {
    const uint16_t* qc = static_cast<const uint16_t*>(a.q_c) + (static_cast<size_t>(t) * a.heads + h) * kDhc + 8 * hh;
#pragma unroll
    for (int k = 0; k < 8; ++k) q[k] = *reinterpret_cast<const bf16x8*>(qc + 16 * k);
    const uint16_t* qr = static_cast<const uint16_t*>(a.q_r) + (static_cast<size_t>(t) * a.heads + h) * kDr + 8 * hh;
    const int p = min(max(pos, 0), max(a.rope_max_pos - 1, 0));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(qr[16 * k + e]);
      if (a.rope_cos != nullptr) {
        const float* cs = a.rope_cos + static_cast<size_t>(p) * (kDr / 2) + 8 * k + 4 * hh;
        const float* sn = a.rope_sin + static_cast<size_t>(p) * (kDr / 2) + 8 * k + 4 * hh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = x[2 * i], x1 = x[2 * i + 1];
          x[2 * i] = fmaf(x0, cs[i], -x1 * sn[i]);
          x[2 * i + 1] = fmaf(x0, sn[i], x1 * cs[i]);
        }
      }
      q[8 + k] = to_bf16x8(x);
    }
  }

  const char* kv = static_cast<const char*>(a.kv);
  const char* ws_k = static_cast<const char*>(a.workspace);
  const char* ws_v = ws_k + static_cast<size_t>(a.num_pool_pages) * kTok * a.heads * kDhc * 2;
  const int32_t* ptab = a.page_table + static_cast<size_t>(b) * a.max_pages;
  const uint32_t smem_base = lds_addr(smem);
  // Copies of page p: K and V rows 16 w .. 16 w + 15 (4 rows of 256 B per instruction),
  // k_R rows 16 w .. +15 (8 rows of 128 B per instruction): 10 per wave.
  auto page_id = [&](int p) { return clamp_page(table_entry(ptab, p), a.num_pool_pages); };
  auto copy_page = [&](int id, uint32_t st) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t0 = 16 * wave + 4 * r;
      const int tk = t0 + (lane >> 4);
      const uint32_t row = static_cast<uint32_t>((static_cast<size_t>(tk) * a.heads + h) * kDhc * 2);
      const char* kbase = ws_k + static_cast<size_t>(id) * kTok * a.heads * kDhc * 2;
      const char* vbase = ws_v + static_cast<size_t>(id) * kTok * a.heads * kDhc * 2;
      dma16(kbase, row + (((lane & 15) ^ swz_k(tk)) << 4), st + t0 * 256);
      dma16(vbase, row + (((lane & 15) ^ swz_v(tk)) << 4), st + kKBytes + t0 * 256);
    }
    const char* page = kv + static_cast<size_t>(id) * kTok * kRowBytes;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int t0 = 16 * wave + 8 * r;
      const int tk = t0 + (lane >> 3);
      dma16(page, static_cast<uint32_t>(tk * kRowBytes + kDc * 2 + (((lane & 7) ^ swz_r(tk)) << 4)),
            st + 2 * kKBytes + t0 * 128);
    }
  };
  if (n_pages > 0) copy_page(page_id(0), smem_base);
  int id_next = n_pages > 1 ? page_id(1) : 0;  // ids are read one page ahead of their copies

  const float scale_log2 = a.scale * kLog2e;
  float m_ref = -INFINITY, l_run = 0.f;
  f32x16 o[4] = {};
  // Lane parts of the LDS addresses.
  //   K read, block mb, K-step ks (0..7):  st + (32 mb + n) * 256 + (((2 ks + hh) ^ swz_k(n)) << 4)
  //   k_R read, step rs:                   st + 2 kKBytes + (32 mb + n) * 128 + (((2 rs + hh) ^ swz_r(n)) << 4)
  //   V^T read (nb, mb, q, part pp): lane i = lane % 16 of group gr = lane / 16 reads key
  //     32 mb + 16 q + 8 pp + 4 (gr >> 1) + i / 4, columns 32 nb + 16 (gr & 1) + 4 (i % 4) .. +3.
  const int li = lane & 15, lg = lane >> 4;
  const int tv = 4 * (lg >> 1) + (li >> 2);            // key within an 8-key group
  const uint32_t vpart = static_cast<uint32_t>(8 * (li & 1));
  // The swizzle of key 32 mb + n is that of key n, and the V^T swizzle depends only on tv,
  // so mb, qq and pp shift an address by a constant (the LDS offset field): one lane part
  // per K-step of K (8), of k_R (4) and per column block of V (4).
  uint32_t k_off[8], r_off[4], v_off[4];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    k_off[ks] = static_cast<uint32_t>(n * 256 + (((2 * ks + hh) ^ swz_k(n)) << 4));
#pragma unroll
  for (int rs = 0; rs < 4; ++rs)
    r_off[rs] = static_cast<uint32_t>(2 * kKBytes + n * 128 + (((2 * rs + hh) ^ swz_r(n)) << 4));
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int c = 4 * nb + 2 * (lg & 1) + ((li & 3) >> 1);
    v_off[nb] = static_cast<uint32_t>(kKBytes + tv * 256 + ((c ^ swz_v(tv)) << 4)) + vpart;
  }
  int stage = 0;
  for (int p = 0; p < n_pages; ++p) {
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    const uint32_t st = smem_base + stage * kAttStage;
    if (p + 1 < n_pages) copy_page(id_next, smem_base + (stage ^ 1) * kAttStage);
    id_next = p + 2 < n_pages ? page_id(p + 2) : 0;
    const int j0 = p * kTok;

    // ---- scores
    f32x16 s[2] = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 kf = lds_read8(st + k_off[ks] + 32 * 256 * mb);
        s[mb] = mfma32(kf, q[ks], s[mb]);
      }
#pragma unroll
    for (int rs = 0; rs < 4; ++rs)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 rf = lds_read8(st + r_off[rs] + 32 * 128 * mb);
        s[mb] = mfma32(rf, q[8 + rs], s[mb]);
      }
    // Keep six reads in flight ahead of the products.
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int i = 0; i < 18; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);

    // ---- softmax.  s[mb][r] is key j0 + 32 mb + 8 (r / 4) + 4 hh + r % 4 of query n.
    const bool partial = j0 + kTok > vis;
    if (partial) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (j0 + 32 * mb + 8 * (r >> 2) + 4 * hh + (r & 3) >= vis) s[mb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
    mx = halves_max(mx) * scale_log2;
    // A page whose maximum exceeds the reference by more than kJump moves it there, and
    // what was accumulated is multiplied by 2^(old - new) (rare).
    const float m_old = m_ref;
    const bool grow = mx > m_old + kJump;  // true on a query's first page with a key
    if (grow) m_ref = mx;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_old - mx) : 1.f;  // 0 from -inf
    l_run *= alpha;
    // O rows are queries: element r of this lane is query 8 (r / 4) + 4 hh + r % 4, whose
    // factor is held by that query's lane.
    if (__builtin_amdgcn_ballot_w64(grow && m_old != -INFINITY) != 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ar = __shfl(alpha, 8 * (r >> 2) + 4 * hh + (r & 3));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) o[nb][r] *= ar;
      }
    }
    const float m_sub = m_ref == -INFINITY ? 0.f : m_ref;
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[mb][r], scale_log2, -m_sub));
        s[mb][r] = pv;
        psum += pv;
      }
    l_run += psum;
    // P as the A operand of K-step kq = 2 mb + q: elements 8 q .. 8 q + 7 of block mb.
    bf16x8 pa[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = s[kq >> 1][8 * (kq & 1) + e];
      pa[kq] = to_bf16x8(x);
    }

    // ---- O[32 queries x 128] += P . V
    uint32_t vb[4];  // opaque, so the row constants below stay in the offset field
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) vb[nb] = opaque(st + v_off[nb]);
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const int mb = kq >> 1, qq = kq & 1;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        bf16x4 part[2];
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const uint32_t addr = vb[nb] + (32 * mb + 16 * qq + 8 * pp) * 256;
          part[pp] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(uintptr_t)addr);
        }
        const bf16x8 vf = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
        o[nb] = mfma32(pa[kq], vf, o[nb]);
      }
    }
    stage ^= 1;
  }

  // ---- output: O / l for query 8 (r / 4) + 4 hh + r % 4 of the wave, columns 32 nb + n.
  const float l_tot = halves_sum(l_run);
  if (q_valid && hh == 0 && a.lse_out != nullptr)
    a.lse_out[static_cast<size_t>(t) * a.heads + h] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  __bf16* out = static_cast<__bf16*>(a.out);
  const int qbase = q0 + qb * kQBlock + 32 * wave;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int qr = 8 * (r >> 2) + 4 * hh + (r & 3);
    const float w = __shfl(inv, qr);
    if (qb * kQBlock + 32 * wave + qr < q_len) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        out[(static_cast<size_t>(qbase + qr) * a.heads + h) * kDhc + 32 * nb + n] =
            static_cast<__bf16>(o[nb][r] * w);
    }
  }
}

}  // namespace

bool prefill_supported(const PrefillArgs& a) {
  return a.groups == 1 && a.d_hc == kDhc && a.d_c == kDc && a.d_R == kDr && a.page_size == kTok;
}

hipError_t launch_decompress(const PrefillArgs& a, hipStream_t s) {
  static std::atomic<uint64_t> dec_set{0};
  const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(decompress_kernel), kDecLds, dec_set);
  if (e != hipSuccess) return e;
  PrefillArgs d = a;
  const long long work = static_cast<long long>(a.batch) * a.max_pages * a.heads;
  d.dec_pages = kDecMinPages;
  while (d.dec_pages < kDecMaxPages && work / (2 * d.dec_pages) >= kDecTargetGroups) d.dec_pages *= 2;
  const long long runs = (a.max_pages + d.dec_pages - 1) / d.dec_pages;
  decompress_kernel<<<dim3(static_cast<unsigned>(runs * a.batch * a.heads)), kDecThreads, kDecLds, s>>>(d);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const PrefillArgs& a, hipStream_t s) {
  static std::atomic<uint64_t> att_set{0};
  const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(prefill_attn_kernel), kAttLds, att_set);
  if (e != hipSuccess) return e;
  const long long n_qb = (a.max_q_len + kQBlock - 1) / kQBlock;
  prefill_attn_kernel<<<dim3(static_cast<unsigned>(n_qb * a.batch * a.heads)), kAttThreads, kAttLds, s>>>(a);
  return hipGetLastError();
}

}  // namespace mla
