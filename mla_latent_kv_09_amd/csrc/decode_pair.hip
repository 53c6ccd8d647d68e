// Split-KV absorbed-MLA decode on bf16 MFMA (gfx950), wave-pair layout.
// Instantiated for one latent group (MLA: every head sees the 512-d latent) and for
// two groups (grouped latent attention, www.hotelren.com/news/5324130 §1: heads
// 0-63 see latent columns 0-255, heads 64-127 columns 256-511, all share k_R).
//
// Computes, for one query token t and one split of its sequence's pages, the
// softmax-normalised latent output and log-sum-exp of
//     s_j = scale * (q_abs . c_KV[j] + RoPE(q_R) . k_R[j])          (nxmr.cn/news/151634 §4)
// over the split's keys for all 128 heads, so every latent row streamed from HBM is
// read once per (token, split) and shared by all heads (nxmr.cn/news/151634 §1: the
// latent plus the shared RoPE key is all a token stores).  Softmax statistics are
// fp32, online, updated every 32 keys.
//
// Work layout (workgroup = 8 waves, two per SIMD).  The heads form 4 blocks of 32;
// waves 2p and 2p+1 ("role" 0 and 1) share head block p.  Per 32-token step:
//   Scores   role r contracts its half of the score dimension -- latent columns
//            [r*d/2, (r+1)*d/2) of the head's group and RoPE dims [32r, 32r+32) --
//            for all 32 heads of the block: S_r^T[32 tok x 32 heads] on
//            v_mfma_f32_16x16x32_bf16, the latent operand read from LDS with
//            ds_read_b128, each read feeding two MFMAs (two 16-head halves), the query
//            held in registers.  The two halves are swapped through LDS and added
//            (S = S_0 + S_1 in both waves: the same bits, since fp32 addition commutes).
//   Softmax  both waves of the pair run the same online softmax on the same S, so
//            both hold the same P, running max and running sum; nothing more is
//            exchanged.
//   Output   role r owns latent columns [r*d/2, (r+1)*d/2) of the output for the 32
//            heads: O^T += C^T . P^T, C^T read with the transposing ds_read_b64_tr_b16,
//            P taken from the score registers.
// Compared with one wave per 16 heads, every latent byte staged in LDS is read by
// half as many waves in both phases.
//
// Schedule: waves 0-3 and 4-7 run the same steps half a step apart ("ping-pong"), so
// that while one wave of a SIMD issues score MFMAs the other runs its softmax and
// output MFMAs; workgroup barriers separate the half-step intervals.
// Staging: 3 slots of 32 tokens (36 KB each) in LDS, filled by global_load_lds
// (16 B per lane, 5 instructions per wave per step), issued 1.5 steps ahead.
#include <math.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kHeads = 128;
constexpr int kPageTok = 64;                          // tokens per cache page
constexpr int kStep = 32;                             // tokens per step (half a page)
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kRowBytes = (kDc + kDr) * 2;            // 1152 B per cached token
constexpr int kSlotC = kStep * kDc * 2;               // 32 KB latent rows of a step
constexpr int kSlotBytes = kSlotC + kStep * kDr * 2;  // + 4 KB RoPE rows
constexpr int kSlots = 3;
constexpr int kXOff = kSlots * kSlotBytes;            // partial-score exchange area
constexpr int kXWave = 4 * 64 * 16;                   // 2x2 tiles x 64 lanes x 16 B per wave
constexpr int kQrOff = kXOff + kWaves * kXWave;     // rotated q_R, 2 x 64 lanes x 16 B per wave
constexpr int kLdsBytes = kQrOff + kWaves * 2 * 1024;
static_assert(kLdsBytes <= 160 * 1024, "slots + exchange + q_R must fit the 160 KB LDS of a gfx950 CU");
constexpr int kRing = 4;  // LDS fragments in flight per wave

template <int G> struct Shape {
  static constexpr int kDcg = kDc / G;   // latent columns seen by one head
  static constexpr int kHalf = kDcg / 2; // latent columns per role (scores and output)
  static constexpr int kQK = kHalf / 32; // latent K-steps per role
  static constexpr int kCB = kHalf / 16; // 16-column output blocks per role
  static constexpr int kPairsPerGroup = 4 / G;
};

// Swizzles (16-byte chunk index XOR).  Latent part: token t's chunk c sits at slot
// c ^ swz_c(t); 16 consecutive tokens x one chunk hit 16 distinct bank groups (b128
// score reads), and 8 aligned tokens x 2 aligned chunks do too (transposing reads).
__device__ __forceinline__ int swz_c(int t) { return 2 * (t & 7) + ((t >> 3) & 1); }
// RoPE part (8 chunks per token): 16 consecutive tokens x one chunk -> 16 groups.
__device__ __forceinline__ int swz_r(int t) { return (t & 7) ^ ((t >> 3) & 1); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}
__device__ __forceinline__ bf16x8 lds_b128(uint32_t byte) { return *(const lds_bf16x8_t*)(uintptr_t)(byte); }
__device__ __forceinline__ bf16x4 lds_tr16(uint32_t byte) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(uintptr_t)(byte));
}

// Hide a value from the optimiser: per-lane LDS bases are rebuilt from it every step
// (a few VALU ops) instead of being hoisted and kept live across the loop.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Reductions over the four 16-lane rows of a wave (lanes j, j+16, j+32, j+48 hold the
// same head): v_permlane16_swap / v_permlane32_swap exchange rows without any lane
// index arithmetic; max and + are symmetric, so every lane of a head ends with the
// same value.
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

__device__ __forceinline__ bf16x8 to_bf16x8(float x0, float x1, float x2, float x3, float x4,
                                            float x5, float x6, float x7) {
  return bf16x8{static_cast<__bf16>(x0), static_cast<__bf16>(x1), static_cast<__bf16>(x2),
                static_cast<__bf16>(x3), static_cast<__bf16>(x4), static_cast<__bf16>(x5),
                static_cast<__bf16>(x6), static_cast<__bf16>(x7)};
}

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4): active lane i's
// 16 bytes land at LDS byte lds + 16 i.  Issued as inline asm so that the compiler
// does not know an LDS DMA is in flight and does not make unrelated LDS reads wait
// for it; completion is awaited explicitly (s_waitcnt vmcnt + barrier).
__device__ __forceinline__ void dma16(const char* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(gptr)
               : "memory");
}

// This wave's share of one step (32 cached tokens starting at `src`) into the slot at
// LDS byte `slot`: latent rows 4w .. 4w+3 (one instruction each) and, with half the
// lanes, the RoPE rows of the same four tokens -- exactly kDmaPerWave instructions.
// Rows at or past n_valid fetch row 0 of the step instead (always valid), so no stale
// or uninitialised slot enters the MFMAs.
constexpr int kDmaPerWave = 5;
__device__ __forceinline__ void load_step(uint32_t slot, const char* src, int n_valid, int wave,
                                          int lane_v) {
  asm volatile("" : "+v"(lane_v));
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int t = wave * 4 + k;
    const int src_t = t < n_valid ? t : 0;
    dma16(src + src_t * kRowBytes + ((lane_v ^ swz_c(t)) << 4), slot + t * 1024);
  }
  if (lane_v < 32) {
    const int t = wave * 4 + (lane_v >> 3);
    const int src_t = t < n_valid ? t : 0;
    dma16(src + src_t * kRowBytes + kDc * 2 + (((lane_v & 7) ^ swz_r(t)) << 4),
          slot + kSlotC + wave * 512);
  }
}

// Wait until at most `n` of this wave's vector-memory operations are outstanding
// (n is 0 or kDmaPerWave), then barrier.  LDS operations are drained too.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N == 0 || N == kDmaPerWave, "unexpected count");
  if constexpr (N == 0) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int G>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_pair_kernel(DecodeArgs a) {
  using Sh = Shape<G>;
  constexpr int kDcg = Sh::kDcg, kHalf = Sh::kHalf, kQK = Sh::kQK, kCB = Sh::kCB;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int t = blockIdx.x, split = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  // Waves 2p and 2p+1 share head block p (roles 0 and 1).  Waves 0-3 (ping-pong group
  // 0) and 4-7 (group 1) run half a step apart; a SIMD holds one wave of each.
  const int pair = wave >> 1, role = wave & 1, pp = wave >> 2;
  const int g = lane >> 4, j = lane & 15;
  const int head0 = pair * 32;                             // heads head0 + 16 hb + j
  const int grp = pair / Sh::kPairsPerGroup;               // latent group of the head block
  const int col0 = grp * kDcg + role * kHalf;              // first latent column of this role
  const int S = a.num_splits;
  const QueryWork w = query_work(a.cu_q, a.seq_lens, a.batch, t, split, S,
                                 a.pages_per_split, kPageTok, a.max_pages, a.causal);
  // Output row of head head0 + 16 hb + j: (t * H + head) * S + split.
  auto out_row = [&](int hb, int lane_j) {
    return (static_cast<size_t>(t) * kHeads + head0 + 16 * hb + lane_j) * S + split;
  };
  if (w.k0 >= w.k1) {  // empty split: only the LSE is written
    if (role == 0 && g == 0) {
      a.lse_part[out_row(0, j)] = -INFINITY;
      a.lse_part[out_row(1, j)] = -INFINITY;
    }
    return;
  }
  const char* kv = static_cast<const char*>(a.kv);
  const int32_t* ptab = a.page_table + static_cast<size_t>(w.b) * a.max_pages;
  // Page ids of the split, 64 at a time: lane l holds the id of page 64c + l of the
  // split, read out with readlane when a step is issued.
  const int page0 = w.k0 / kPageTok;
  const int n_split_pages = (w.k1 - w.k0 + kPageTok - 1) / kPageTok;
  const int n_steps = (w.k1 - w.k0 + kStep - 1) / kStep;
  int pid_v = 0;
  // The load is awaited right here (the empty asm consumes the value) so that the wait
  // stays on this rarely taken path instead of landing before every page issue.
  auto fetch_ids = [&](int chunk) {
    const int idx = chunk * 64 + lane;
    pid_v = idx < n_split_pages ? ptab[page0 + idx] : 0;
    asm volatile("" : "+v"(pid_v));
  };
  const uint32_t smem_base = lds_addr(smem);
  auto issue_step = [&](int i) {  // i = step index within the split (wave-uniform)
    const int pg = i >> 1;
    if ((i & 1) == 0 && (pg & 63) == 0 && pg > 0) fetch_ids(pg >> 6);
    const int id = clamp_page(__builtin_amdgcn_readlane(pid_v, pg & 63), a.num_pool_pages);
    const char* src = kv + (static_cast<size_t>(id) * kPageTok + (i & 1) * kStep) * kRowBytes;
    load_step(smem_base + (i % kSlots) * kSlotBytes, src, min(kStep, w.k1 - w.k0 - i * kStep),
              wave, lane);
  };
  fetch_ids(0);
  issue_step(0);

  // Query operands (B of S^T = C . Q^T): latent K-step k of this role covers columns
  // col0 + 32k .. +31; lane (g, j) holds columns +8g .. +7 of head head0 + 16 hb + j.
  // The RoPE half of the role (dims 32 role + 8g .. +7) is rotated here in fp32 and
  // parked as bf16 in LDS, private to the lane (read back once per step).
  bf16x8 q[2][kQK];
  const uint32_t qr_wave = smem_base + kQrOff + wave * 2048;
  {
    const uint32_t qr_lane = qr_wave + lane * 16;
    const int p = min(max(w.pos, 0), max(a.rope_max_pos - 1, 0));
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const size_t hrow = static_cast<size_t>(t) * kHeads + head0 + 16 * hb + j;
      const uint16_t* qa = static_cast<const uint16_t*>(a.q_abs) + hrow * kDcg + role * kHalf + g * 8;
#pragma unroll
      for (int k = 0; k < kQK; ++k) q[hb][k] = *reinterpret_cast<const bf16x8*>(qa + 32 * k);
      const uint16_t* qrp = static_cast<const uint16_t*>(a.q_r) + hrow * kDr + 32 * role + g * 8;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(qrp[e]);
      if (a.rope_cos != nullptr) {
        const int pair0 = (32 * role + g * 8) / 2;
        const float* cs = a.rope_cos + static_cast<size_t>(p) * (kDr / 2) + pair0;
        const float* sn = a.rope_sin + static_cast<size_t>(p) * (kDr / 2) + pair0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = x[2 * i], x1 = x[2 * i + 1];
          x[2 * i] = fmaf(x0, cs[i], -x1 * sn[i]);
          x[2 * i + 1] = fmaf(x0, sn[i], x1 * cs[i]);
        }
      }
      *(lds_bf16x8_t*)(uintptr_t)(qr_lane + hb * 1024) =
          to_bf16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
    }
  }
  // Make the compiler wait for the query loads here, before the second step's copy is
  // issued: its own wait counts only the loads it knows of, so a wait placed after
  // the copy would also wait for the copy.
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
    for (int k = 0; k < kQK; ++k) asm volatile("" : : "v"(q[hb][k]));
  }
  if (n_steps > 1) issue_step(1);

  const float scale_log2 = a.scale * kLog2e;
  float m_run[2] = {-INFINITY, -INFINITY};  // running max (log2 units), same in both waves of the pair
  float l_run[2] = {0.f, 0.f};              // this lane's share of the running sum
  f32x4 o[kCB][2];                          // O^T block (cb, hb): columns 16cb + 4g .. +3 of head hb
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    o[cb][0] = f32x4{0.f, 0.f, 0.f, 0.f};
    o[cb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t x_own = smem_base + kXOff + wave * kXWave;
  const uint32_t x_pair = smem_base + kXOff + (wave & ~1) * kXWave;  // role 0's area, role 1's follows

  // The step's slot (the first step's copy) must have landed before interval 0.
  if (n_steps > 1) wait_vm_barrier<kDmaPerWave>(); else wait_vm_barrier<0>();

  // Intervals k = 0 .. 2 n_steps, separated by workgroup barriers.  Group pp computes
  // the partial scores of step i in interval 2i + pp and finishes the step (swap,
  // softmax, output) in interval 2i + pp + 1, so in every interval one wave of each
  // SIMD runs score MFMAs while the other runs softmax and output MFMAs.  The copy of
  // step i is issued at the start of interval 2i - 3 into slot i % 3, whose previous
  // step (i - 3) was last read in interval 2i - 4, and awaited at the end of interval
  // 2i - 1 (after which group 0 scores step i).  Each group runs its own straight-line
  // loop; both pass the same 2 n_steps barriers.
  auto score_step = [&](int i) __attribute__((always_inline)) {
    const uint32_t slot = smem_base + (i % kSlots) * kSlotBytes;
    const int lv = static_cast<int>(opaque(static_cast<uint32_t>(lane)));
    const int lj = lv & 15, lg = lv >> 4;
      // ---- partial scores: S_r^T[16tb + (4g + e)][16hb + j]
      f32x4 s[2][2];
      {
        const uint32_t rb = opaque(slot + kSlotC + lj * 128 + (((4 * role + lg) ^ swz_r(lj)) << 4));
        const bf16x8 c0 = lds_b128(rb);
        const bf16x8 c1 = lds_b128(rb + 2048);
        const uint32_t qr_lane = qr_wave + lv * 16;
        const bf16x8 qr0 = lds_b128(qr_lane), qr1 = lds_b128(qr_lane + 1024);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        s[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c0, qr0, z, 0, 0, 0);
        s[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c0, qr1, z, 0, 0, 0);
        s[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c1, qr0, z, 0, 0, 0);
        s[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c1, qr1, z, 0, 0, 0);
      }
      {
        // Latent fragment st = 2k + tb: tokens 16tb + j, columns col0 + 32k + 8g .. +7.
        // The column chunk (col0/8 + 4k + g) ^ swz_c(j) splits into a per-lane base
        // for k % 4 plus the immediate 256 (k / 4), since col0/8 is a multiple of 16.
        uint32_t sb[4];
        const int sw = swz_c(lj);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          sb[q4] = opaque(slot + lj * 1024 + 2 * col0 + (((4 * q4 + lg) ^ sw) << 4));
        auto frag = [&](int st) {
          const int kq = st >> 1, tb = st & 1;
          return lds_b128(sb[kq & 3] + 16384 * tb + 256 * (kq >> 2));
        };
        constexpr int kSteps = 2 * kQK;
        bf16x8 ring[kRing];
#pragma unroll
        for (int st = 0; st < kRing; ++st) ring[st] = frag(st);
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          const bf16x8 c = ring[st % kRing];
          if (st + kRing < kSteps) ring[st % kRing] = frag(st + kRing);
          const int kq = st >> 1, tb = st & 1;
          s[tb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c, q[0][kq], s[tb][0], 0, 0, 0);
          s[tb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c, q[1][kq], s[tb][1], 0, 0, 0);
        }
        // Keep kRing fragment reads in flight: the scheduler's own latency model would
        // otherwise issue each read right before its two MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);      // RoPE rows + rotated q_R
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);      // RoPE MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, kRing, 0);  // first latent fragments
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          if (st + kRing < kSteps) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      // ---- park the partial scores for the partner (read in the next interval)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          *(lds_f32x4_t*)(uintptr_t)(x_own + (tb * 2 + hb) * 1024 + lv * 16) = s[tb][hb];
  };
  auto finish_step = [&](int i) __attribute__((always_inline)) {
    const uint32_t slot = smem_base + (i % kSlots) * kSlotBytes;
    const int lv = static_cast<int>(opaque(static_cast<uint32_t>(lane)));
    const int lj = lv & 15, lg = lv >> 4;
      const int n_valid = min(kStep, w.k1 - w.k0 - i * kStep);
      // ---- full scores S = S_0 + S_1, added in role order in both waves
      f32x4 s[2][2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const uint32_t xa = x_pair + (tb * 2 + hb) * 1024 + lv * 16;
          s[tb][hb] = *(const lds_f32x4_t*)(uintptr_t)(xa);
          s[tb][hb] += *(const lds_f32x4_t*)(uintptr_t)(xa + kXWave);
        }

      // ---- online softmax per head; s[tb][hb][e] is token 16tb + 4g + e
      bf16x8 pb[2];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tok = 16 * tb + 4 * lg + e;
            const float x = tok < n_valid ? s[tb][hb][e] * scale_log2 : -INFINITY;
            s[tb][hb][e] = x;
            mx = fmaxf(mx, x);
          }
        mx = rows_max(mx);
        const float m_new = fmaxf(m_run[hb], mx);
        const float alpha = m_run[hb] == m_new ? 1.f : __builtin_amdgcn_exp2f(m_run[hb] - m_new);
        float psum = 0.f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pe = __builtin_amdgcn_exp2f(s[tb][hb][e] - m_new);
            s[tb][hb][e] = pe;
            psum += pe;
          }
        l_run[hb] = l_run[hb] * alpha + psum;
        m_run[hb] = m_new;
        if (__any(alpha != 1.f)) {
#pragma unroll
          for (int cb = 0; cb < kCB; ++cb) o[cb][hb] *= alpha;
        }
        // P^T operand: K index 8g + e <-> token 4g + e (e < 4), 16 + 4g + (e - 4) (e >= 4)
        pb[hb] = to_bf16x8(s[0][hb][0], s[0][hb][1], s[0][hb][2], s[0][hb][3], s[1][hb][0],
                           s[1][hb][1], s[1][hb][2], s[1][hb][3]);
      }

      // ---- O^T[columns of this role] += C^T . P^T
      {
        const int tok = 4 * lg + (lj >> 2);
        const int swo = swz_c(tok);
        const int colb = 4 * (lj & 3);
        const uint32_t rowb = slot + tok * 1024 + 2 * col0 + (colb & 7) * 2;
        const uint32_t chunk_lo = colb >> 3;
        // A operand of column block cb: columns 16cb + j, tokens in the P^T order, via
        // two transposing reads (tokens 4g.. and 16 + 4g..); the swizzled address is
        // rebuilt per block (two VALU ops) rather than kept in eight registers.
        auto frag = [&](int cb) {
          const uint32_t a1 = rowb + ((((2 * (cb & 7)) + chunk_lo) ^ swo) << 4) + 256 * (cb >> 3);
          const bf16x4 lo = lds_tr16(a1);
          const bf16x4 hi = lds_tr16(a1 + 16384);
          return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8 ring[kRing];
#pragma unroll
        for (int st = 0; st < kRing; ++st) ring[st] = frag(st);
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
          const bf16x8 ct = ring[cb % kRing];
          if (cb + kRing < kCB) ring[cb % kRing] = frag(cb + kRing);
          o[cb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ct, pb[0], o[cb][0], 0, 0, 0);
          o[cb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ct, pb[1], o[cb][1], 0, 0, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kRing, 0);
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          if (cb + kRing < kCB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
  };
  // End of an odd interval: the next interval scores step (k + 1) / 2, whose copy must
  // have landed; the copy issued in this interval may still be in flight.
  auto end_odd_interval = [&](int k) __attribute__((always_inline)) {
    if ((k + 3) / 2 < n_steps) wait_vm_barrier<kDmaPerWave>(); else wait_vm_barrier<0>();
  };
  if (pp == 0) {
    for (int i = 0; i < n_steps; ++i) {
      score_step(i);                                   // interval 2i
      lds_barrier();
      if (i + 2 < n_steps) issue_step(i + 2);          // interval 2i + 1
      finish_step(i);
      end_odd_interval(2 * i + 1);
    }
  } else {
    for (int i = 0; i <= n_steps; ++i) {
      if (i > 0) finish_step(i - 1);                   // interval 2i
      if (i == n_steps) break;
      lds_barrier();
      if (i + 2 < n_steps) issue_step(i + 2);          // interval 2i + 1
      score_step(i);
      end_odd_interval(2 * i + 1);
    }
  }

  // ---- finalize: normalise and write this role's columns of the partial output; role
  // 0 writes the log-sum-exp (both waves hold the same statistics)
  {
    const int lv = static_cast<int>(opaque(static_cast<uint32_t>(lane)));
    const int lj = lv & 15, lg = lv >> 4;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const float l_tot = rows_sum(l_run[hb]);
      const float inv = 1.f / l_tot;
      const size_t r = out_row(hb, lj);
      float* o_out = a.o_part + r * kDcg + role * kHalf + 4 * lg;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) *reinterpret_cast<f32x4*>(o_out + 16 * cb) = o[cb][hb] * inv;
      if (role == 0 && lg == 0) a.lse_part[r] = (m_run[hb] + __log2f(l_tot)) * kLn2;
    }
  }
}

}  // namespace

bool decode_pair_supported(const DecodeArgs& a, bool bf16) {
  return bf16 && a.heads == kHeads && (a.groups == 1 || a.groups == 2) && a.d_c == kDc &&
         a.d_R == kDr && a.page_size == kPageTok;
}

template <int G>
hipError_t launch_decode_pair_g(const DecodeArgs& a, hipStream_t s) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_pair_kernel<G>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const dim3 grid(a.total_q, a.num_splits);
  decode_pair_kernel<G><<<grid, kThreads, kLdsBytes, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode_pair(const DecodeArgs& a, hipStream_t s) {
  return a.groups == 2 ? launch_decode_pair_g<2>(a, s) : launch_decode_pair_g<1>(a, s);
}

}  // namespace mla
