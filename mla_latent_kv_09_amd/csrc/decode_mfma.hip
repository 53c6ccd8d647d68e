// Split-KV absorbed-MLA decode on bf16 MFMA (gfx950), 128 (or 64) query rows per
// workgroup.  Instantiated for one latent group (MLA: every head sees the 512-d latent)
// and for two groups (grouped latent attention, www.hotelren.com/news/5324130 §1: heads
// 0-63 see latent columns 0-255, heads 64-127 columns 256-511, all share k_R).
//
// Computes, for one query token t and one split of its sequence's pages, the
// softmax-normalised latent output and log-sum-exp of
//     s_j = scale * (q_abs . c_KV[j] + RoPE(q_R) . k_R[j])          (nxmr.cn/news/151634 §4)
// over the split's keys, for all H = 128 heads at once (or, with the head split HS = 2
// below, for 64 heads in each of two workgroups that run side by side on one XCD), so
// every streamed latent page is read from HBM once per (token, split) and shared by all
// heads
// (nxmr.cn/news/151634 §1: the 512-d latent plus the 64-d shared RoPE key is all a
// token stores).  Softmax statistics are fp32 (online, one page at a time).
//
// Softmax reference: the exponentials of a page are taken against a per-head
// reference m that only moves when a page's maximum exceeds it by more than kSlack
// (log2 units), so p <= 2^kSlack and the running output is rescaled only on those
// rare moves.  Output and log-sum-exp are normalised against the same m at the end,
// so the result is the same softmax.
//
// Work layout (workgroup = 8 waves, two per SIMD; HS = 1):
//   wave w owns heads 16w .. 16w+15; lane l owns head 16w + l%16, and the four
//   lanes l%16 + 16g (g = 0..3) split that head's keys (scores) and latent
//   columns (output) between them.
//   Scores:  S^T[64 tok x 16 heads] = C[64 x 576] . Q^T   on v_mfma_f32_16x16x32_bf16,
//            C read from LDS (ds_read_b128), Q held in registers for the whole split.
//   Output:  O^T[512 x 16 heads] += C^T[512 x 64] . P^T    on the same MFMA,
//            C^T read from LDS with ds_read_b64_tr_b16, P taken straight from the
//            score accumulators (no LDS round trip).
// Pages: one 64-token page (72 KB) per stage, two stages in LDS (144 KB of 160 KB),
// fetched with global_load_lds (16 B per lane) in a swizzled layout that keeps both
// the b128 score reads and the transposing output reads free of bank conflicts.  The
// next page's nine copies per wave are spread through the score loop (issued
// together they stall every wave's instruction issue behind the memory pipeline);
// fragment rings keep 3 score and 6 output reads in flight per wave, the most the
// 256-register budget of two waves per SIMD leaves room for.
#include <math.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kHeads = 128;              // rows per workgroup (8 waves x 16)
constexpr int kTok = 64;                 // tokens per stage = one page
constexpr int kDc = 512;                 // latent width
constexpr int kDr = 64;                  // RoPE key width
constexpr int kRowBytes = (kDc + kDr) * 2;
constexpr int kCBytes = kTok * kDc * 2;  // 64 KB latent part of a stage
constexpr int kRBytes = kTok * kDr * 2;  // 8 KB RoPE part
constexpr int kStageBytes = kCBytes + kRBytes;
constexpr int kQrOff = 2 * kStageBytes;   // rotated q_R of all heads lives after the two stages
constexpr int kLdsBytes = kQrOff + kHeads * kDr * 2;
constexpr float kSlack = 8.f;             // softmax reference slack, log2 units
template <int G> struct Shape {
  static constexpr int kDcg = kDc / G;        // latent columns seen by one head
  static constexpr int kQSteps = kDcg / 32;   // latent K-steps of 32 dims (+2 RoPE steps)
  static constexpr int kColBlocks = kDcg / 16;  // 16-column output tiles
  static constexpr int kWavesPerGroup = kWaves / G;
};
static_assert(kLdsBytes <= 160 * 1024, "stages + q_R must fit the 160 KB LDS of a gfx950 CU");

// Swizzles (16-byte chunk index XOR).  LDS serves a 16-byte-per-lane read 32 lanes at a
// time out of one 512-byte bank row, and an 8-byte transposing read 32 lanes at a time
// too, so a layout is conflict-free when the 32 lanes of each half-wave touch 32
// distinct 16-byte (resp. 8-byte) slots of a 512-byte row.
// Latent part: token t's chunk c sits at position c ^ swz_c(t), an XOR inside aligned
// 32-chunk blocks.  A score read (16 consecutive tokens j x chunks c, c+1) then covers
// all 32 slots (bit 0 from the chunk, bits 1-4 from the token), and so does a
// transposing read (8 tokens x 2 chunks x 2 halves).
__device__ __forceinline__ int swz_c(int t) { return 2 * (t & 15); }
// RoPE part (8 chunks = 128 B per token, 4 tokens per 512-byte row): the XOR separates
// the 4 tokens that share row slots, so 16 tokens x chunks c, c+1 are conflict-free.
__device__ __forceinline__ int swz_r(int t) { return 2 * ((t >> 2) & 3); }
// Rotated q_R (8 chunks per head): 16 consecutive heads x one chunk -> 16 groups.
__device__ __forceinline__ uint32_t qr_slot(int h, int c) { return h * 128 + ((c ^ ((h >> 1) & 7)) << 4); }

// Reductions over the four 16-lane rows of a wave (lanes j, j+16, j+32, j+48 hold the
// same head): v_permlane16_swap / v_permlane32_swap exchange rows without lane-index
// arithmetic; max and + are symmetric, so every lane of a head ends with the same value.
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS byte offset of a pointer into a __shared__ array, and back.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}
__device__ __forceinline__ lds_bf16x4_t* lds_bf16x4(uint32_t byte) { return (lds_bf16x4_t*)(uintptr_t)(byte); }

// Pass a value through an empty asm so the compiler treats it as unknown: used on
// per-iteration LDS base addresses so that only compile-time offsets vary between
// the reads of a page (they fold into the ds_read offset field) and no per-read
// address is hoisted out of the page loop.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ bf16x8 to_bf16x8(float x0, float x1, float x2, float x3, float x4,
                                            float x5, float x6, float x7) {
  return bf16x8{static_cast<__bf16>(x0), static_cast<__bf16>(x1), static_cast<__bf16>(x2),
                static_cast<__bf16>(x3), static_cast<__bf16>(x4), static_cast<__bf16>(x5),
                static_cast<__bf16>(x6), static_cast<__bf16>(x7)};
}

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4) addressed as a
// wave-uniform base (SGPR pair) plus a 32-bit per-lane byte offset: active lane i's 16
// bytes land at LDS byte lds + 16 i.  Issued as inline asm on purpose: the compiler
// then does not know that an LDS DMA is in flight, so it does not make every later LDS
// read of the page being computed wait for the *next* page's copy (it cannot prove
// they do not alias).  Completion is awaited explicitly with s_waitcnt vmcnt(0) + a
// barrier before a stage is read; every wait the compiler emits for its own loads only
// counts ops it knows about, which stays safe.
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// This wave's share of one page in LDS stage `c_base`: latent rows 8w .. 8w+7 (one
// 1 KB copy each, `row` = 0..7) and the RoPE rows of the same 8 tokens (row 8).  Rows
// at or past n_valid fetch row 0 instead (always valid), so no stale or uninitialised
// slot enters the MFMAs.  For row t = 8w + k the latent swizzle key is
// swz_c(t) = 16 (w & 1) + 2k.  The copies are spread through the score loop rather
// than issued together: the memory pipeline takes 64 B per clock per CU, and nine
// back-to-back 1 KB copies from every wave would stall each wave's issue for
// thousands of cycles.
__device__ __forceinline__ void load_row(uint32_t c_base, const char* page, int n_valid,
                                         int wave, int lane, int row) {
  if (row < 8) {
    const int t = wave * 8 + row;
    const int src_t = t < n_valid ? t : 0;
    const int key = 16 * (wave & 1) + 2 * row;
    dma16(page + src_t * kRowBytes, static_cast<uint32_t>((lane ^ key) << 4), c_base + t * 1024);
  } else {
    const int t = wave * 8 + (lane >> 3);
    const int src_t = t < n_valid ? t : 0;
    dma16(page, static_cast<uint32_t>(src_t * kRowBytes + kDc * 2 + (((lane & 7) ^ swz_r(t)) << 4)),
          c_base + kCBytes + wave * 1024);
  }
}

__device__ __forceinline__ void load_page(uint32_t smem_base, int stage, const char* page,
                                          int n_valid, int wave, int lane_v) {
  asm volatile("" : "+v"(lane_v));
  const uint32_t c_base = smem_base + stage * kStageBytes;
#pragma unroll
  for (int row = 0; row < 9; ++row) load_row(c_base, page, n_valid, wave, lane_v, row);
}

constexpr int kRing = 4;  // LDS fragments in flight per wave

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo), b = static_cast<__bf16>(hi);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a)) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b)) << 16);
}

// Writes two output tiles of this lane's row: x = columns 16nb + 4g .. +3 and
// y = columns 16(nb+1) + 4g .. +3 (nb even).  v_permlane16_swap trades x of lane rows 1
// and 3 for y of rows 0 and 2, after which lane row g holds the 8 consecutive columns
// 16nb + 16(g & 1) + 8(g >> 1) .. +7 and writes them as one 16-byte store: 64 contiguous
// bytes per head and store instead of 32, which halves the stores and the L2 write
// requests of the partials.
__device__ __forceinline__ void store_pair(__bf16* o_row, int nb, const f32x4& x, const f32x4& y, int g) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint32_t x0 = pack_bf16x2(x[0], x[1]), x1 = pack_bf16x2(x[2], x[3]);
  const uint32_t y0 = pack_bf16x2(y[0], y[1]), y1 = pack_bf16x2(y[2], y[3]);
  const auto s0 = __builtin_amdgcn_permlane16_swap(x0, y0, false, false);
  const auto s1 = __builtin_amdgcn_permlane16_swap(x1, y1, false, false);
  *reinterpret_cast<u32x4*>(o_row + 16 * nb + 16 * (g & 1) + 8 * (g >> 1)) =
      u32x4{s0[0], s1[0], s0[1], s1[1]};
}

// Latent score fragment (mb, k): A operand of S^T for tokens 16mb + j, latent dims
// 32k + 8g .. +7 (chunk 4k + g).  The token blocks alternate in the step order so that
// consecutive MFMAs accumulate into different registers.  With key 2j the chunk sits
// at position 32 (k / 8) + 4 ((k % 8) ^ (j / 2)) + (g ^ 2 (j % 2)): `lb` is the stage
// base plus the per-lane row and low bits, `jx` = (j / 2) << 6, so each fragment costs
// one xor-add and an immediate offset.
__device__ __forceinline__ bf16x8 score_frag(uint32_t lb, uint32_t jx, int mb, int k) {
  const uint32_t a = lb + (jx ^ static_cast<uint32_t>((k & 7) << 6));
  return *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(a + 16384 * mb + 512 * (k >> 3));
}

// Output-step fragment st = ks * nC + nb: A operand of O^T for columns 16nb + j,
// tokens 32ks + 4g + {0..3} and 32ks + 16 + 4g + {0..3}, via two transposing reads.
// Column chunk 2nb + h of token tok sits at position 2 (nb ^ tok) + h: `lb` holds the
// per-lane row, chunk half and in-chunk offset, `tx` = tok << 5.
template <int kColBlocks>
__device__ __forceinline__ bf16x8 out_frag(uint32_t lb, uint32_t tx, int st) {
  const int ks = st / kColBlocks, nb = st % kColBlocks;
  const uint32_t a1 = lb + (tx ^ static_cast<uint32_t>((nb & 15) << 5)) + 32768 * ks + 512 * (nb >> 4);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lds_bf16x4(a1));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(lds_bf16x4(a1 + 16384));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// HS = 1: one workgroup per (token, split) covers all 128 heads; wave w owns heads
// 16w .. 16w+15 over all 64 tokens of each page.
// HS = 2 (one latent group only): two workgroups per (token, split), 64 heads each, so
// a batch with few (token, split) pairs still fills the device with half as many
// split partials to write and merge.  Wave w owns heads 16 (w % 4) .. +15 of its half
// over tokens 32 (w / 4) .. +31 of each page; waves w and w + 4 (one SIMD) keep their
// own softmax state and merge it through LDS at the end.  Both halves of a pair stream
// the same pages, and run side by side on one XCD, so the second read of a page is
// served by that XCD's L2.
template <int G, int HS>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_mfma_kernel(DecodeArgs a) {
  static_assert(HS == 1 || (HS == 2 && G == 1), "head split only for one latent group");
  using Sh = Shape<G>;
  constexpr int kDcg = Sh::kDcg, kQSteps = Sh::kQSteps, kColBlocks = Sh::kColBlocks;
  constexpr int kMB = 4 / HS;           // 16-token score blocks per wave and page
  constexpr int kHeadsWG = kHeads / HS;  // heads of one workgroup
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int S = a.num_splits;
  // 1-D grid in split-fastest order over pairs P = t * S + split.  The dispatcher deals
  // workgroups to the 8 XCDs in turn (L mod 8), so the splits of one token spread over
  // the XCDs, and a batch whose sequences differ in length loads every XCD alike.
  // HS = 2 (short batches, where the first page and the query load are much of the
  // kernel): when T is a multiple of 8, the 2 S workgroups of token t all go to XCD
  // t mod 8, consecutive in its order, the two halves of a pair adjacent.  The token's
  // query rows then reach one L2 instead of all eight, and both halves of a pair read
  // their pages from the same L2.  Otherwise blocks of 8 pairs take 16 consecutive
  // workgroups: half h2 of pair 8k + i is workgroup 16k + 8 h2 + i (in a last block of
  // r < 8 pairs, 16k + r h2 + i), so the halves of a pair in a full block share an XCD.
  const Unit u = HS == 1 ? unit_split_fastest(static_cast<int>(blockIdx.x), S)
                         : unit_mfma_half(static_cast<int>(blockIdx.x), S, a.total_q);
  const int t = u.t, split = u.split, h2 = u.half;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int g = lane >> 4, j = lane & 15;   // 16-lane group, position in group
  const int hb = HS == 1 ? wave : (wave & 3);  // 16-head block within the workgroup
  const int th = HS == 1 ? 0 : (wave >> 2);    // token half of each page (HS = 2)
  const int hl = hb * 16 + j;                  // head within the workgroup
  const int head = h2 * kHeadsWG + hl;
  const int grp = wave / Sh::kWavesPerGroup;             // latent group of this wave
  const uint32_t grp_off = static_cast<uint32_t>(grp) * kDcg * 2;  // its columns in a token row
  // Three independent loads go out before the first wait: the sequence table, the page
  // ids of the first pages this split would read if token t were sequence t (true of a
  // batch with one query row per sequence), and this lane's query rows.  Only one round
  // trip then precedes the first page's copies; the guessed ids are used only once the
  // lookup has confirmed the guess.
  SeqIndex ix;
  ix.load(a.cu_q, a.seq_lens, a.batch);
  const int page0_guess = split * a.pages_per_split;
  const bool can_guess = t < a.batch && a.pages_per_split > 0;
  int pid_guess = 0;
  if (can_guess && page0_guess + lane < a.max_pages)
    pid_guess = a.page_table[static_cast<size_t>(t) * a.max_pages + page0_guess + lane];
  // Q fragments: B operand of S^T = C . Q^T.  K-step k covers latent dims 32k .. 32k+31;
  // this lane holds dims 32k + 8g .. +7 of its head.
  bf16x8 q[kQSteps];  // latent part of the query
  {
    const uint16_t* qa = static_cast<const uint16_t*>(a.q_abs) +
                         (static_cast<size_t>(t) * kHeads + head) * kDcg + g * 8;
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) q[k] = *reinterpret_cast<const bf16x8*>(qa + 32 * k);
  }
  const QueryWork w = query_work(ix, t, split, S, a.pages_per_split, kTok, a.max_pages, a.causal);
  const size_t row = (static_cast<size_t>(t) * kHeads + head) * S + split;
  __bf16* o_out = static_cast<__bf16*>(a.o_part) + row * kDcg;  // bf16 partials
  if (w.k0 >= w.k1) {  // empty split: only the LSE is written
    if (g == 0 && th == 0) a.lse_part[row] = -INFINITY;
    return;
  }
  const char* kv = static_cast<const char*>(a.kv);
  const int32_t* ptab = a.page_table + static_cast<size_t>(w.b) * a.max_pages;
  // Page ids of the split, 64 at a time: lane l holds the id of page 64c + l of the
  // split, read out with readlane when a page is issued.
  const int page0 = w.k0 / kTok;
  const int n_split_pages = (w.k1 - w.k0 + kTok - 1) / kTok;
  int pid_v = 0;
  auto fetch_ids = [&](int chunk) {
    const int idx = chunk * 64 + lane;
    pid_v = idx < n_split_pages ? ptab[page0 + idx] : 0;
    asm volatile("" : "+v"(pid_v));  // wait for the load here, on this rarely taken path
  };
  auto page_ptr = [&](int i) {  // i = page index within the split (wave-uniform)
    const int id = clamp_page(__builtin_amdgcn_readlane(pid_v, i & 63), a.num_pool_pages);
    return kv + static_cast<size_t>(id) * kTok * kRowBytes;
  };
  if (can_guess && w.b == t && page0 == page0_guess)
    pid_v = pid_guess;  // lanes past the split's pages hold ids that are never read
  else
    fetch_ids(0);

  // First page in flight before anything else.
  int j0 = w.k0;
  load_page(lds_addr(smem), 0, page_ptr(0), min(kTok, w.k1 - j0), wave, lane);

  // The RoPE half of the query is rotated here in fp32 and parked, as bf16, in LDS (read
  // back twice per page; with HS = 2 the token-half-0 wave of a head block writes it for
  // both).
  if (th == 0) {
    const uint16_t* qr = static_cast<const uint16_t*>(a.q_r) +
                         (static_cast<size_t>(t) * kHeads + head) * kDr + g * 8;
    const int p = min(max(w.pos, 0), max(a.rope_max_pos - 1, 0));
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(qr[32 * k + e]);
      if (a.rope_cos != nullptr) {
        const int pair0 = (32 * k + g * 8) / 2;
        const float* cs = a.rope_cos + static_cast<size_t>(p) * (kDr / 2) + pair0;
        const float* sn = a.rope_sin + static_cast<size_t>(p) * (kDr / 2) + pair0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = x[2 * i], x1 = x[2 * i + 1];
          x[2 * i] = fmaf(x0, cs[i], -x1 * sn[i]);
          x[2 * i + 1] = fmaf(x0, sn[i], x1 * cs[i]);
        }
      }
      *(__attribute__((address_space(3))) bf16x8*)(uintptr_t)(lds_addr(smem) + kQrOff +
                                                             qr_slot(hl, 4 * k + g)) =
          to_bf16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
    }
  }

  const float scale_log2 = a.scale * kLog2e;
  float m_ref = -INFINITY;   // softmax reference of this lane's head (log2 units), same in its 4 lanes
  float l_run = 0.f;         // this lane's share of the running sum against m_ref
  f32x4 o[kColBlocks];       // O^T block nb: columns 16nb + 4g .. +3 of this lane's head
#pragma unroll
  for (int nb = 0; nb < kColBlocks; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Per-lane LDS offsets inside a stage.  The swizzle keys depend only on the low
  // four bits of the token index, so every address is a per-lane base, one xor of a
  // per-lane key with a compile-time constant, and a compile-time immediate:
  //   score read  (token 16mb + j, chunk 4k + g):  base_s + (jx ^ 64 (k%8)) + 16384 mb + 512 (k/8)
  //   RoPE read   (token 16mb + j, chunk 4k + g):  base_r(k) + 2048 mb
  //   output read (token 32ks + 4g + j/4 (+16), column 16nb + 4(j%4)):
  //                           base_o + (tx ^ 32 (nb%16)) + 32768 ks (+16384) + 512 (nb/16)
  // (with HS = 2 the token half th moves every base by 32 tokens: mb = 2 th + 0..1,
  // ks = th).  The bases are recomputed from the lane index every page (a few VALU ops)
  // rather than kept in registers across the loop.
  const uint32_t smem_base = lds_addr(smem);
  const uint32_t half_c = static_cast<uint32_t>(th) * 32768;  // 32 tokens of latent rows
  const uint32_t half_r = static_cast<uint32_t>(th) * 4096;   // 32 tokens of RoPE rows
  int stage = 0;
  for (; j0 < w.k1; j0 += kTok) {
    const int n_valid = min(kTok, w.k1 - j0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's page loads have landed
    __syncthreads();                     // ... and every wave's; the other stage is free again
    // The next page's copy is issued from inside the score loop below.
    const int j_next = j0 + kTok;
    const bool has_next = j_next < w.k1;
    const char* next_page = kv;
    const int next_valid = min(kTok, w.k1 - j_next);
    if (has_next) {
      const int i_next = (j_next - w.k0) / kTok;
      if ((i_next & 63) == 0) fetch_ids(i_next >> 6);
      next_page = page_ptr(i_next);
    }
    const uint32_t next_base = smem_base + (stage ^ 1) * kStageBytes;
    const uint32_t st_base = smem_base + stage * kStageBytes;
    const int lv = static_cast<int>(opaque(static_cast<uint32_t>(lane)));
    const int lj = lv & 15, lg = lv >> 4;
    const uint32_t sb = opaque(st_base + half_c + grp_off + lj * 1024 + ((lg ^ (2 * (lj & 1))) << 4));
    const uint32_t sjx = opaque(static_cast<uint32_t>(lj >> 1) << 6);

    // ---- scores S^T for tokens mb*16 .. mb*16+15 of the page.  RoPE part first
    // (the q_R fragments are live only here), then the (mb, k) latent steps in order
    // through a ring of prefetched LDS fragments.
    f32x4 s[kMB];
    {
      const int swr = swz_r(lj);
      const uint32_t rb0 = st_base + half_r + kCBytes + lj * 128 + (((lg) ^ swr) << 4);
      const uint32_t rb1 = st_base + half_r + kCBytes + lj * 128 + (((4 + lg) ^ swr) << 4);
      const uint32_t qr_head = smem_base + kQrOff + (hb * 16 + lj) * 128;
      const int swq = (lj >> 1) & 7;
      const uint32_t qr_addr0 = qr_head + ((lg ^ swq) << 4);
      const uint32_t qr_addr1 = qr_head + (((4 + lg) ^ swq) << 4);
      const bf16x8 qr0 = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(qr_addr0);
      const bf16x8 qr1 = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(qr_addr1);
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        const bf16x8 c0 = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(
            rb0 + 2048 * mb);
        const bf16x8 c1 = *(const __attribute__((address_space(3))) bf16x8*)(uintptr_t)(
            rb1 + 2048 * mb);
        s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c0, qr0, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c1, qr1, s[mb], 0, 0, 0);
      }
    }
    {
      constexpr int kSteps = kMB * kQSteps;  // (mb, k) steps
      constexpr int kSRing = 3;
      bf16x8 ring[kSRing];
#pragma unroll
      for (int st = 0; st < kSRing; ++st) ring[st] = score_frag(sb, sjx, st % kMB, st / kMB);
      constexpr int kRowEvery = kSteps / 8;  // one page-row copy every kRowEvery steps
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        const bf16x8 c = ring[st % kSRing];
        if (st + kSRing < kSteps)
          ring[st % kSRing] = score_frag(sb, sjx, (st + kSRing) % kMB, (st + kSRing) / kMB);
        const int mb = st % kMB, k = st / kMB;
        s[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c, q[k], s[mb], 0, 0, 0);
        if (st % kRowEvery == kRowEvery / 2 && has_next)
          load_row(next_base, next_page, next_valid, wave, static_cast<int>(opaque(lane)), st / kRowEvery);
        if (st == kSteps / 2 + 1 && has_next)
          load_row(next_base, next_page, next_valid, wave, static_cast<int>(opaque(lane)), 8);
      }
    }

    // ---- online softmax.  s[mb][i] is the raw score of token 32th + mb*16 + 4g + i; only
    // the last page of a split can be partial, so the mask is skipped on full pages, and
    // the scale is applied in the exponent (it is positive, so it commutes with the max).
    if (n_valid < kTok) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (32 * th + mb * 16 + 4 * g + i >= n_valid) s[mb][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[mb][i]);
    mx = rows_max(mx) * scale_log2;
    const float m_old = m_ref;
    const bool grow = mx > m_old + kSlack;   // always true on a first page with a valid key
    const float m_new = grow ? mx : m_old;
    // With HS = 2 the second token half of a split's only (partial) page can hold no
    // valid key: the reference then stays -inf and is subtracted as 0, which keeps
    // every exponential at 0 instead of NaN.  (Token 0 of a page is always valid, so
    // with HS = 1 the first page already sets a finite reference.)
    const float m_sub = (HS == 2 && m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_old - m_sub);  // 0 before the first valid key
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][i], scale_log2, -m_sub));
        s[mb][i] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_ref = m_new;
    // The output only needs rescaling when a reference that was already in use moves
    // (before the first page it is still zero).
    if (__any(grow && m_old != -INFINITY)) {
#pragma unroll
      for (int nb = 0; nb < kColBlocks; ++nb) o[nb] *= alpha;
    }

    // ---- P^T operands: K-step ks covers tokens 32ks + 4g + {0..3} and 32ks + 16 + 4g + {0..3}
    // (with HS = 2 the one K-step of token half th)
    constexpr int kKS = kMB / 2;
    bf16x8 pb[kKS];
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      pb[ks] = to_bf16x8(s[2 * ks][0], s[2 * ks][1], s[2 * ks][2], s[2 * ks][3],
                         s[2 * ks + 1][0], s[2 * ks + 1][1], s[2 * ks + 1][2], s[2 * ks + 1][3]);

    // ---- O^T[cols 16nb .. +15] += C^T . P^T, (ks, nb) steps through the ring
    const int otok = 4 * lg + (lj >> 2);
    const int colb = 4 * (lj & 3);
    const uint32_t ob =
        opaque(st_base + half_c + grp_off + otok * 1024 + ((colb >> 3) << 4) + (colb & 7) * 2);
    const uint32_t otx = opaque(static_cast<uint32_t>(otok) << 5);
    {
      constexpr int kSteps = kKS * kColBlocks;
      constexpr int kORing = 6;
      bf16x8 ring[kORing];
#pragma unroll
      for (int st = 0; st < kORing; ++st) ring[st] = out_frag<kColBlocks>(ob, otx, st);
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        const bf16x8 ct = ring[st % kORing];
        if (st + kORing < kSteps) ring[st % kORing] = out_frag<kColBlocks>(ob, otx, st + kORing);
        const int ks = st / kColBlocks, nb = st % kColBlocks;
        o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ct, pb[ks], o[nb], 0, 0, 0);
      }
      // Keep kORing fragments (2 transposing reads each) in flight.
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kORing, 0);
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (st + kORing < kSteps) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    }
    stage ^= 1;
  }

  // ---- finalize: normalise and write this split's partial output and LSE
  const float l_tot = rows_sum(l_run);
  if constexpr (HS == 1) {
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int nb = 0; nb < kColBlocks; nb += 2) store_pair(o_out, nb, o[nb] * inv, o[nb + 1] * inv, g);
    if (g == 0) a.lse_part[row] = (m_ref + __log2f(l_tot)) * kLn2;
  } else {
    // Merge the two token halves of each head: wave w keeps output columns
    // 256 th .. +255 and hands the other half, with its (m, l), to its partner w ^ 4
    // through LDS (the stages are free once every wave has finished the last page).
    // Lane-linear 16-byte slots: conflict-free.
    constexpr int kHalf = kColBlocks / 2;
    const uint32_t xo_mine = smem_base + static_cast<uint32_t>(wave) * (kHalf * 1024) + lane * 16;
    const uint32_t xo_part = smem_base + static_cast<uint32_t>(wave ^ 4) * (kHalf * 1024) + lane * 16;
    const uint32_t ml_mine = smem_base + kWaves * kHalf * 1024 + (wave * 64 + lane) * 8;
    const uint32_t ml_part = smem_base + kWaves * kHalf * 1024 + ((wave ^ 4) * 64 + lane) * 8;
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;
    typedef __attribute__((address_space(3))) float lds_f32_t;
    __syncthreads();  // every wave is done with the stages
    if (th == 0) {
#pragma unroll
      for (int i = 0; i < kHalf; ++i) *(lds_f32x4_t*)(uintptr_t)(xo_mine + i * 1024) = o[kHalf + i];
    } else {
#pragma unroll
      for (int i = 0; i < kHalf; ++i) *(lds_f32x4_t*)(uintptr_t)(xo_mine + i * 1024) = o[i];
    }
    *(lds_f32_t*)(uintptr_t)(ml_mine) = m_ref;
    *(lds_f32_t*)(uintptr_t)(ml_mine + 4) = l_tot;
    __syncthreads();
    const float m_p = *(lds_f32_t*)(uintptr_t)(ml_part);
    const float l_p = *(lds_f32_t*)(uintptr_t)(ml_part + 4);
    const float m = fmaxf(m_ref, m_p);  // finite: token 0 of every page is in half 0
    const float a_me = __builtin_amdgcn_exp2f(m_ref - m), a_p = __builtin_amdgcn_exp2f(m_p - m);
    const float l = l_tot * a_me + l_p * a_p;
    const float inv = 1.f / l;
    const float w_me = a_me * inv, w_p = a_p * inv;
    auto emit = [&](int nb, const f32x4& m0, const f32x4& m1, uint32_t slot) {
      const f32x4 p0 = *(lds_f32x4_t*)(uintptr_t)(slot);
      const f32x4 p1 = *(lds_f32x4_t*)(uintptr_t)(slot + 1024);
      store_pair(o_out, nb, m0 * w_me + p0 * w_p, m1 * w_me + p1 * w_p, g);
    };
    if (th == 0) {
#pragma unroll
      for (int i = 0; i < kHalf; i += 2) emit(i, o[i], o[i + 1], xo_part + i * 1024);
      if (g == 0) a.lse_part[row] = (m + __log2f(l)) * kLn2;
    } else {
#pragma unroll
      for (int i = 0; i < kHalf; i += 2) emit(kHalf + i, o[kHalf + i], o[kHalf + i + 1], xo_part + i * 1024);
    }
  }
}

}  // namespace

bool decode_mfma_supported(const DecodeArgs& a, bool bf16) {
  return bf16 && a.heads == kHeads && (a.groups == 1 || a.groups == 2) && a.d_c == kDc &&
         a.d_R == kDr && a.page_size == kTok;
}

template <int G, int HS>
hipError_t launch_decode_mfma_k(const DecodeArgs& a, hipStream_t s) {
  static std::atomic<uint64_t> lds_limit_set{0};
  const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(decode_mfma_kernel<G, HS>), kLdsBytes,
                                        lds_limit_set);
  if (e != hipSuccess) return e;
  const dim3 grid(a.total_q * a.num_splits * HS);
  decode_mfma_kernel<G, HS><<<grid, kThreads, kLdsBytes, s>>>(a);
  return hipGetLastError();
}

int decode_mfma_head_split(const DecodeArgs& a, int cu_count) {
  if (a.groups != 1) return 1;
  if (a.head_split == 1 || a.head_split == 2) return a.head_split;
  return 2LL * a.total_q * a.num_splits <= cu_count ? 2 : 1;
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int head_split, hipStream_t s) {
  if (a.groups == 2) return launch_decode_mfma_k<2, 1>(a, s);
  return head_split == 2 ? launch_decode_mfma_k<1, 2>(a, s) : launch_decode_mfma_k<1, 1>(a, s);
}

}  // namespace mla
