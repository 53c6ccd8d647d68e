// Split-KV absorbed-MLA decode on the 32x32x16 bf16 MFMA (gfx950), one latent group:
// one workgroup of four waves per (token, split), wave w owning heads 32w .. 32w+31
// over all 64 tokens of every page.
//
// Computes, for one query token and one split of its sequence's pages, the
// softmax-normalised latent output and log-sum-exp of
//     s_j = scale * (q_abs . c_KV[j] + RoPE(q_R) . k_R[j])          (nxmr.cn/news/151634 §4)
// over the split's keys, for all 128 heads at once, so every streamed latent page is
// read from HBM once per (token, split) and shared by all heads (nxmr.cn/news/151634
// §1: the 512-d latent plus the 64-d shared RoPE key is all a token stores).
//
// Why 32x32x16 with one wave per SIMD: one wave issuing v_mfma_f32_32x32x16_bf16
// keeps the matrix pipe of its SIMD busy on its own (about 95 % of the bf16 peak with
// two independent accumulators, measured), where the 16x16x32 form needs two waves in
// the same phase to get there (one wave alone reaches 38-59 %).  Each 16-byte LDS
// fragment also feeds twice the flops of a 16x16x32 step, halving LDS reads.  The
// price is registers: the query (576 dims of 32 heads, 128 VGPRs plus the RoPE part
// from LDS) stays in VGPRs and the output O^T[512 x 32 heads] (256 fp32 per lane)
// needs the accumulator half of the 512-register file.
//
// Per page and wave:
//   scores  S^T[64 tok x 32 heads] = C[64 x 576] . Q^T as two 32-token blocks of 36
//           K-steps (32 latent + 4 RoPE); A = C from LDS (ds_read_b128), B = Q.
//           Lane l then holds head l % 32 and 16 tokens per block:
//           token 8 (r / 4) + 4 (l / 32) + r % 4 of accumulator element r.
//   softmax fp32, per head, the two lane halves combined with v_permlane32_swap.
//   output  O^T[cols x heads] += C^T . P^T over four 16-token K-steps.  The K order of a
//           step is the order the score accumulators hold the tokens in (elements
//           8q .. 8q+7 of block mb), so P^T is the score registers converted in place
//           and the matching C^T fragment is two transposing reads of 4 tokens each.
// Pages: one 64-token page (72 KB) per stage, two stages (144 KB) plus the rotated q_R
// of all heads (16 KB) fill the 160 KB LDS.  Copies (global_load_lds, 16 B per lane)
// of the next page are spread through the score loop.
//
// LDS layout of a stage: latent row t (1 KB) holds chunk c (8 dims) at 16-byte position
// c ^ f(t), f(t) = (t[1:0] << 2) | t[3:2] | (t[4] << 4) (a bit permutation of t mod 32).
// A score read (32 consecutive tokens, one chunk) then hits 32 distinct 16-byte slots of
// a 512-byte bank row, and so does a transposing read (4 tokens x 4 chunks x 2 halves).
// RoPE row t (128 B) holds chunk c at c ^ ((t >> 2) & 7); q_R of head n the same with n.
//
// FP8 cache (kFmtFp8; the quantized latent gather of nxmr.cn/news/151634, intro and §5,
// on gfx950's E4M3 format): a page holds the latent codes [64][512] (E4M3, 32 KB), k_R
// [64][64] (bf16, 8 KB) and one float32 scale per token (256 B), 41 KB in all.  The copies
// land in an FP8 stage; once per page the four waves convert each code times its token's
// scale, a power of two, to bf16 exactly (v_cvt_scalef32_pk_bf16_fp8) into one stage of the
// bf16 form's layout and move the page's k_R rows beside them, so the score and output
// loops are the bf16 form's, with no scale work.  LDS: the bf16 stage (72 KB), the FP8 stage
// (41 KB) and q_R (16 KB); the copies of page i + 1 go out once page i is converted.  The
// MXFP4 cache (kFmtFp4: packed E2M1 codes, one power-of-two scale byte per 32 elements,
// 25 KB pages) takes the same path with its own copies and conversion.
#include <math.h>

#include <type_traits>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kHeads = 128;
constexpr int kTok = 64;
constexpr int kDc = 512;
constexpr int kDr = 64;
constexpr int kRowBytes = (kDc + kDr) * 2;
constexpr int kCBytes = kTok * kDc * 2;  // 64 KB latent part of a stage
constexpr int kRBytes = kTok * kDr * 2;  // 8 KB RoPE part
constexpr int kStageBytes = kCBytes + kRBytes;
constexpr int kQrOff = 2 * kStageBytes;
constexpr int kLdsBytes = kQrOff + kHeads * kDr * 2;
constexpr int kQSteps = kDc / 16;        // 32 latent K-steps
constexpr int kRSteps = kDr / 16;        // 4 RoPE K-steps
constexpr int kColBlocks = kDc / 32;     // 16 output blocks of 32 columns
constexpr float kJump = 64.f;            // reference move threshold, log2 units
static_assert(kLdsBytes <= 160 * 1024, "stages + q_R must fit the 160 KB LDS of a gfx950 CU");

// FP8 cache page in HBM: codes, then k_R, then the token scales.
constexpr int kC8Bytes = kTok * kDc;              // 32 KB of E4M3 codes
constexpr int kR8Off = kC8Bytes;                  // k_R [64][64] bf16
constexpr int kS8Off = kC8Bytes + kRBytes;        // scales [64] float32
constexpr int kPage8Bytes = kS8Off + kTok * 4;    // 41216 B, the page stride in HBM
constexpr int kCopies8 = 11;                      // global->LDS copies per wave and page
// FP8 LDS: one bf16 stage (read by the loops), the FP8 stage the copies land in (latent row
// t at 512 t, k_R and scales as in HBM, k_R rows swizzled as in the bf16 stage), then q_R.
// The 64-head form's final merge uses the first 130 KB.
constexpr int kQOff = kStageBytes;
constexpr int kQrOff8 = kQOff + kPage8Bytes;
constexpr int kMergeBytes = 4 * 32768 + kThreads * 8;
constexpr int kLds8Bytes = kQrOff8 + kHeads * kDr * 2 > kMergeBytes ? kQrOff8 + kHeads * kDr * 2 : kMergeBytes;
static_assert(kLds8Bytes <= 160 * 1024, "the FP8 form's LDS must fit the 160 KB of a gfx950 CU");
static_assert(kPage8Bytes % 16 == 0 && kQOff % 16 == 0, "FP8 pages are whole 16-byte units");
static_assert(kLdsBytes >= kMergeBytes, "the 64-head merge fits the bf16 form's LDS");

// MXFP4 cache page in HBM: packed E2M1 codes (byte j of a row: elements 2j, 2j + 1 in its
// low and high nibble), then k_R, then one E8M0 scale byte per 32 latent elements.
constexpr int kC4Bytes = kTok * kDc / 2;               // 16 KB of codes
constexpr int kR4Off = kC4Bytes;                       // k_R [64][64] bf16
constexpr int kS4Off = kC4Bytes + kRBytes;             // scale bytes [64][16]
constexpr int kPage4Bytes = kS4Off + kTok * kDc / 32;  // 25600 B, the page stride in HBM
constexpr int kCopies4 = 7;                            // global->LDS copies per wave and page
// MXFP4 LDS: the FP8 form's layout with the MXFP4 page in the quantized stage.
constexpr int kQrOff4 = kQOff + kPage4Bytes;
constexpr int kLds4Bytes = kQrOff4 + kHeads * kDr * 2 > kMergeBytes ? kQrOff4 + kHeads * kDr * 2 : kMergeBytes;
static_assert(kLds4Bytes <= 160 * 1024 && kPage4Bytes % 16 == 0, "MXFP4 stage layout");

// Cache formats of the kernel template.
enum : int { kFmtBf16 = 0, kFmtFp8 = 1, kFmtFp4 = 2 };

template <int KF>
struct Form {
  static constexpr int kPage = KF == kFmtFp8 ? kPage8Bytes : KF == kFmtFp4 ? kPage4Bytes : kTok * kRowBytes;
  static constexpr int kQr = KF == kFmtFp8 ? kQrOff8 : KF == kFmtFp4 ? kQrOff4 : kQrOff;
  static constexpr int kLds = KF == kFmtFp8 ? kLds8Bytes : KF == kFmtFp4 ? kLds4Bytes : kLdsBytes;
  static constexpr int kCopies = KF == kFmtFp8 ? kCopies8 : KF == kFmtFp4 ? kCopies4 : 18;
};

__device__ __forceinline__ uint32_t swz_f(int t) {
  return static_cast<uint32_t>(((t & 3) << 2) | ((t >> 2) & 3) | (t & 16));
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ bf16x8 lds_read8(uint32_t a) { return *(const lds_bf16x8_t*)(uintptr_t)a; }
__device__ __forceinline__ float halves_max(float x) {  // lanes l and l ^ 32
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ bf16x8 to_bf16x8(float x0, float x1, float x2, float x3, float x4,
                                            float x5, float x6, float x7) {
  return bf16x8{static_cast<__bf16>(x0), static_cast<__bf16>(x1), static_cast<__bf16>(x2),
                static_cast<__bf16>(x3), static_cast<__bf16>(x4), static_cast<__bf16>(x5),
                static_cast<__bf16>(x6), static_cast<__bf16>(x7)};
}

// Score MFMAs in inline asm so that their accumulators stay in VGPRs (the compiler
// puts the result of every MFMA builtin of this kernel in the accumulator registers,
// which the 256 output values already fill).  Chained steps accumulate in place
// (srcC = vdst, which the hardware forwards without wait states); the first step of a
// chain takes srcC = 0, so no vector-ALU write precedes an MFMA read of the
// accumulator.  Vector-ALU reads of the result wait behind mfma_results_ready().
__device__ __forceinline__ void mfma32_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// Wait states between the last asm MFMA writing s0 / s1 and the first vector-ALU read
// of them (the compiler inserts none for asm): 3 x s_nop 7 = 24, more than the
// 32x32 MFMA's result latency requires.  The operands tie the pad after those MFMAs.
__device__ __forceinline__ void mfma_results_ready(f32x16& s0, f32x16& s1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s0), "+v"(s1));
}

// o[nb] *= alpha for all 16 accumulator blocks, one block at a time through VGPRs (the
// blocks live in the accumulator registers, which a vector multiply cannot write).
__device__ __forceinline__ void scale_acc(f32x16 (&o)[16], float alpha) {
#pragma unroll
  for (int nb = 0; nb < 16; ++nb) {
    asm volatile("" : "+a"(o[nb]));
    f32x16 t = o[nb];
    asm volatile("" : "+v"(t));
    t *= alpha;
    o[nb] = t;
    asm volatile("" : "+a"(o[nb]));
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4), wave-uniform base
// plus per-lane offset; active lane i's 16 bytes land at LDS byte lds + 16 i.  Inline
// asm so that the compiler does not make later LDS reads of the current stage wait for
// it; completion is awaited with s_waitcnt vmcnt(0) + a barrier before a stage is read.
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// E4M3 -> bf16 of the two codes in the low (kHi = false) or high 16 bits of v, times the
// power of two `scale`: exact (code * 2^e has at most 4 significant bits and stays in bf16's
// range for the scales the append writes).  Inline asm: the builtin's bf16x2 result is
// split wrongly by the compiler.
template <bool kHi>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t v, float scale) {
  uint32_t r;
  if constexpr (kHi)
    asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, %2 op_sel:[1,0,0]" : "=v"(r) : "v"(v), "v"(scale));
  else
    asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, %2" : "=v"(r) : "v"(v), "v"(scale));
  return r;
}
// FP8 form: copy `row` (0..10) of this wave's share of a page into the FP8 stage `f8`:
// rows 0..7 are the codes of tokens 16w + 2 row and 16w + 2 row + 1 (512 B each, one per
// lane half), rows 8, 9 the k_R rows of tokens 16w + 8 (row - 8) .. +7, row 10 the scales
// of tokens 16w .. 16w+15 (lanes 0..3).  Rows at or past n_valid fetch token 0.
__device__ __forceinline__ void load_row8(uint32_t f8, const char* page, int n_valid, int wave,
                                          int lane, int row) {
  if (row < 8) {
    const int t0 = wave * 16 + 2 * row;
    const int t = t0 + (lane >> 5);
    const int src_t = t < n_valid ? t : 0;
    dma16(page, static_cast<uint32_t>(src_t * kDc + ((lane & 31) << 4)), f8 + t0 * kDc);
  } else if (row < 10) {
    const int t0 = wave * 16 + 8 * (row - 8);
    const int t = t0 + (lane >> 3);
    const int src_t = t < n_valid ? t : 0;
    dma16(page, static_cast<uint32_t>(kR8Off + src_t * 128 + (((lane & 7) ^ ((t >> 2) & 7)) << 4)),
          f8 + kR8Off + t0 * 128);
  } else if (lane < 4) {
    // Scales of tokens past n_valid may be anything: the conversion takes 1 for those rows.
    dma16(page, static_cast<uint32_t>(kS8Off + wave * 64 + 16 * lane), f8 + kS8Off + wave * 64);
  }
}

// FP8 form: the page in the FP8 stage becomes the bf16 stage at `base`.  Wave w takes
// tokens 16w .. 16w+15: lane l converts codes 8l .. 8l+7 of each latent row times the
// token's scale (exactly) into the 16-byte chunk l of that bf16 row, stored at its
// swizzled position l ^ f(t); rows at or past n_valid (copies of token 0) take scale 1,
// whatever their scale slot holds, so every row of the stage is finite.  The k_R rows
// (already in the bf16 stage's order) are moved as they are.  Both the 8-byte reads and
// the 16-byte writes meet distinct banks.
template <int kBatch>
__device__ __forceinline__ void convert_page8(uint32_t base, int wave, int lane, int n_valid) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) u32x2 lds_u32x2_t;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
  typedef __attribute__((address_space(3))) float lds_f32_t;
  const uint32_t f8 = base + kQOff;
  const uint32_t src = f8 + static_cast<uint32_t>(wave * 16 * kDc + 8 * lane);
  const uint32_t ssrc = f8 + static_cast<uint32_t>(kS8Off + wave * 64);
  // token 16w + r: swz_f(16w + r) = swz_f(r) | 16 (w & 1), swz_f(r) < 16
  const uint32_t dst = base + static_cast<uint32_t>(wave * 16 * 1024) +
                       (static_cast<uint32_t>(lane ^ (16 * (wave & 1))) << 4);
  // The reads of kBatch code rows and their scales (with one batch, the k_R rows too), then
  // the conversions and writes, so that the LDS latency is paid once per batch.  (The
  // 64-head form takes two batches and moves k_R after them: it has fewer registers to
  // spare here.)
  const uint32_t kr_off = static_cast<uint32_t>(wave * 2048 + 16 * lane);
  const int lim = n_valid - 16 * wave;  // row r of this wave is a key iff r < lim
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += kBatch) {
    const bool last = kBatch == 16;
    u32x2 raw[kBatch];
    float sc[kBatch];
    u32x4 kr0, kr1;
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      raw[r] = *(const lds_u32x2_t*)(uintptr_t)(src + (r0 + r) * kDc);
      sc[r] = *(const lds_f32_t*)(uintptr_t)(ssrc + 4 * (r0 + r));
    }
    if (last) {
      kr0 = *(const lds_u32x4_t*)(uintptr_t)(f8 + kR8Off + kr_off);
      kr1 = *(const lds_u32x4_t*)(uintptr_t)(f8 + kR8Off + kr_off + 1024);
    }
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const float s = r0 + r < lim ? sc[r] : 1.f;
      const u32x4 v{fp8x2_to_bf16x2<false>(raw[r][0], s), fp8x2_to_bf16x2<true>(raw[r][0], s),
                    fp8x2_to_bf16x2<false>(raw[r][1], s), fp8x2_to_bf16x2<true>(raw[r][1], s)};
      *(lds_u32x4_t*)(uintptr_t)((dst + (r0 + r) * 1024) ^ (swz_f(r0 + r) << 4)) = v;
    }
    if (last) {
      *(lds_u32x4_t*)(uintptr_t)(base + kCBytes + kr_off) = kr0;
      *(lds_u32x4_t*)(uintptr_t)(base + kCBytes + kr_off + 1024) = kr1;
    }
  }
  if constexpr (kBatch < 16) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      *(lds_u32x4_t*)(uintptr_t)(base + kCBytes + kr_off + 1024 * j) =
          *(const lds_u32x4_t*)(uintptr_t)(f8 + kR8Off + kr_off + 1024 * j);
  }
}

// MXFP4 form: copy `row` (0..6) of this wave's share of a page into the quantized stage
// `f4` (the page's own layout): rows 0..3 are the codes of tokens 16w + 4 row .. +3 (256 B
// each, one per 16-lane group), rows 4, 5 the k_R rows of tokens 16w + 8 (row - 4) .. +7
// (swizzled as in the bf16 stage), row 6 the scale bytes of tokens 16w .. 16w+15 (lanes
// 0..15).  Rows at or past n_valid fetch token 0.
__device__ __forceinline__ void load_row4(uint32_t f4, const char* page, int n_valid, int wave,
                                          int lane, int row) {
  if (row < 4) {
    const int t0 = wave * 16 + 4 * row;
    const int t = t0 + (lane >> 4);
    const int src_t = t < n_valid ? t : 0;
    dma16(page, static_cast<uint32_t>(src_t * (kDc / 2) + ((lane & 15) << 4)), f4 + t0 * (kDc / 2));
  } else if (row < 6) {
    const int t0 = wave * 16 + 8 * (row - 4);
    const int t = t0 + (lane >> 3);
    const int src_t = t < n_valid ? t : 0;
    dma16(page, static_cast<uint32_t>(kR4Off + src_t * 128 + (((lane & 7) ^ ((t >> 2) & 7)) << 4)),
          f4 + kR4Off + t0 * 128);
  } else if (lane < 16) {
    const int t = wave * 16 + lane;
    const int src_t = t < n_valid ? t : 0;
    dma16(page, static_cast<uint32_t>(kS4Off + src_t * 16), f4 + kS4Off + wave * 256);
  }
}

// Exact E2M1 -> bf16 of the two codes in byte kByte of v, times the power of two `scale`
// (v_cvt_scalef32_pk_bf16_fp4: the low nibble to the low half).  Inline asm, as for the
// FP8 conversion.
template <int kByte>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t v, float scale) {
  uint32_t r;
  if constexpr (kByte == 0)
    asm("v_cvt_scalef32_pk_bf16_fp4 %0, %1, %2" : "=v"(r) : "v"(v), "v"(scale));
  else if constexpr (kByte == 1)
    asm("v_cvt_scalef32_pk_bf16_fp4 %0, %1, %2 op_sel:[1,0,0]" : "=v"(r) : "v"(v), "v"(scale));
  else if constexpr (kByte == 2)
    asm("v_cvt_scalef32_pk_bf16_fp4 %0, %1, %2 op_sel:[0,1,0]" : "=v"(r) : "v"(v), "v"(scale));
  else
    asm("v_cvt_scalef32_pk_bf16_fp4 %0, %1, %2 op_sel:[1,1,0]" : "=v"(r) : "v"(v), "v"(scale));
  return r;
}

// MXFP4 form: the page in the quantized stage becomes the bf16 stage at `base`.  Wave w
// takes tokens 16w .. 16w+15: lane l converts the 8 codes of dword l of a row (elements
// 8l .. 8l+7, one block, so one scale: byte l / 4 of the row's scales) into the 16-byte
// chunk l of that bf16 row at its swizzled position l ^ f(t); the value is code * 2^(s-127)
// exactly (the scale bytes are 1 .. 254, normal float32 powers of two).  The k_R rows are
// moved as they are.
template <int kBatch>
__device__ __forceinline__ void convert_page4(uint32_t base, int wave, int lane) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
  typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4_t;
  const uint32_t f4 = base + kQOff;
  const uint32_t src = f4 + static_cast<uint32_t>(wave * 16 * (kDc / 2) + 4 * lane);
  const uint32_t ssrc = f4 + static_cast<uint32_t>(kS4Off + wave * 256 + (lane >> 2));
  const uint32_t dst = base + static_cast<uint32_t>(wave * 16 * 1024) +
                       (static_cast<uint32_t>(lane ^ (16 * (wave & 1))) << 4);
  const uint32_t kr_off = static_cast<uint32_t>(wave * 2048 + 16 * lane);
#pragma unroll
  for (int r0 = 0; r0 < 16; r0 += kBatch) {
    uint32_t raw[kBatch], sb[kBatch];
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      raw[r] = *(const lds_u32_t*)(uintptr_t)(src + (r0 + r) * (kDc / 2));
      sb[r] = *(const lds_u8_t*)(uintptr_t)(ssrc + (r0 + r) * 16);
    }
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const float sc = __uint_as_float(sb[r] << 23);
      const u32x4 v{fp4x2_to_bf16x2<0>(raw[r], sc), fp4x2_to_bf16x2<1>(raw[r], sc),
                    fp4x2_to_bf16x2<2>(raw[r], sc), fp4x2_to_bf16x2<3>(raw[r], sc)};
      *(lds_u32x4_t*)(uintptr_t)((dst + (r0 + r) * 1024) ^ (swz_f(r0 + r) << 4)) = v;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
    *(lds_u32x4_t*)(uintptr_t)(base + kCBytes + kr_off + 1024 * j) =
        *(const lds_u32x4_t*)(uintptr_t)(f4 + kR4Off + kr_off + 1024 * j);
}

// Copy `row` (0..17) of this wave's share of a page into stage `c_base`: rows 0..15 are
// the latent rows of tokens 16w + row (1 KB each), rows 16, 17 the RoPE rows of tokens
// 16w + 8 (row - 16) .. +7.  Rows at or past n_valid fetch token 0 (always valid).
__device__ __forceinline__ void load_row(uint32_t c_base, const char* page, int n_valid,
                                         int wave, int lane, int row) {
  if (row < 16) {
    const int t = wave * 16 + row;
    const int src_t = t < n_valid ? t : 0;
    dma16(page + src_t * kRowBytes, static_cast<uint32_t>((lane ^ static_cast<int>(swz_f(t))) << 4),
          c_base + t * 1024);
  } else {
    const int t0 = wave * 16 + 8 * (row - 16);
    const int t = t0 + (lane >> 3);
    const int src_t = t < n_valid ? t : 0;
    dma16(page, static_cast<uint32_t>(src_t * kRowBytes + kDc * 2 + (((lane & 7) ^ ((t >> 2) & 7)) << 4)),
          c_base + kCBytes + t0 * 128);
  }
}

// HS = 1: one workgroup per (token, split), wave w owns heads 32w .. 32w+31 over all
// 64 tokens of a page.
// HS = 2: two workgroups of 64 heads per (token, split).  Wave w owns heads
// 32 (w % 2) .. +31 of its half over tokens 32 (w / 2) .. +31 of each page; waves w and
// w ^ 2 (same heads, other token half) merge their outputs through LDS at the end.
template <int HS, int KF>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_m32_kernel(DecodeArgs a) {
  using Fm = Form<KF>;
  constexpr bool F8 = KF == kFmtFp8, F4 = KF == kFmtFp4;
  constexpr bool Q = F8 || F4;  // a quantized cache: copies land in the quantized stage
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int S = a.num_splits;
  // Launch order (HS = 1): every sequence's non-empty (token, split) units first, then
  // the empty ones (unit_active_first).  Within a sequence of one token the splits run in
  // order; with n tokens, which read the same pages, each block of 8 splits takes 8 n
  // consecutive workgroups, token-major, so the n workgroups of one split are 8 apart:
  // the dispatcher (workgroup L to XCD L mod 8) places them on one XCD at about the same
  // time, and that XCD's L2 serves the later reads of each page.
  SeqIndex ix;
  ix.load(a.cu_q, a.seq_lens, a.batch);
  Unit u;
  if constexpr (HS == 2) {
    u = unit_pair_blocks(static_cast<int>(blockIdx.x), S, a.total_q);
  } else {
    u = unit_active_first_wave(static_cast<int>(blockIdx.x), S, a.pages_per_split, kTok, a.max_pages,
                               a.cu_q, a.seq_lens, a.batch);
    if (u.t < 0 || u.t >= a.total_q || u.split < 0 || u.split >= S)
      u = unit_split_fastest(static_cast<int>(blockIdx.x), S);  // malformed cu_q
  }
  const int t = u.t, split = u.split, h2 = u.half;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;  // head within the wave, lane half
  const int hb = HS == 1 ? wave : (wave & 1);  // 32-head block within the workgroup
  const int th = HS == 1 ? 0 : (wave >> 1);    // token half of each page (HS = 2)
  const int hl = hb * 32 + n;                  // head within the workgroup
  const int head = h2 * (kHeads / HS) + hl;
  const QueryWork w = query_work(ix, t, split, S, a.pages_per_split, kTok, a.max_pages, a.causal);
  const size_t row = (static_cast<size_t>(t) * kHeads + head) * S + split;
  __bf16* o_out = static_cast<__bf16*>(a.o_part) + row * kDc;
  if (w.k0 >= w.k1) {  // empty split: only the LSE is written
    if (h == 0 && th == 0) a.lse_part[row] = -INFINITY;
    return;
  }
  const char* kv = static_cast<const char*>(a.kv);
  const int32_t* ptab = a.page_table + static_cast<size_t>(w.b) * a.max_pages;
  const int page0 = w.k0 / kTok;
  const int n_split_pages = (w.k1 - w.k0 + kTok - 1) / kTok;
  int pid_v = 0;
  auto fetch_ids = [&](int chunk) {
    const int idx = chunk * 64 + lane;
    pid_v = idx < n_split_pages ? ptab[page0 + idx] : 0;
    asm volatile("" : "+v"(pid_v));
  };
  auto page_ptr = [&](int i) {
    const int id = clamp_page(__builtin_amdgcn_readlane(pid_v, i & 63), a.num_pool_pages);
    return kv + static_cast<size_t>(id) * Fm::kPage;
  };
  fetch_ids(0);
  const uint32_t smem_base = lds_addr(smem);
  int j0 = w.k0;
  {  // page 0 into stage 0 (FP8: into the FP8 stage)
    const char* p0 = page_ptr(0);
    const int nv = min(kTok, w.k1 - j0);
    if constexpr (F8) {
#pragma unroll
      for (int r = 0; r < kCopies8; ++r) load_row8(smem_base + kQOff, p0, nv, wave, lane, r);
    } else if constexpr (F4) {
#pragma unroll
      for (int r = 0; r < kCopies4; ++r) load_row4(smem_base + kQOff, p0, nv, wave, lane, r);
    } else {
#pragma unroll
      for (int r = 0; r < 18; ++r) load_row(smem_base, p0, nv, wave, lane, r);
    }
  }

  // Query: latent part in registers (B operand of the scores: head n, dims 16 ks + 8 h ..),
  // RoPE part rotated in fp32 and parked in LDS as bf16.
  bf16x8 q[kQSteps];
  {
    const uint16_t* qa = static_cast<const uint16_t*>(a.q_abs) +
                         (static_cast<size_t>(t) * kHeads + head) * kDc + 8 * h;
#pragma unroll
    for (int k = 0; k < kQSteps; ++k) q[k] = *reinterpret_cast<const bf16x8*>(qa + 16 * k);  // dims 16 k + 8 h ..
  }
  if (th == 0) {
    const uint16_t* qr = static_cast<const uint16_t*>(a.q_r) +
                         (static_cast<size_t>(t) * kHeads + head) * kDr;
    const int p = min(max(w.pos, 0), max(a.rope_max_pos - 1, 0));
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // chunks h, h + 2, h + 4, h + 6 of this head
      const int c = 2 * k + h;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(qr[8 * c + e]);
      if (a.rope_cos != nullptr) {
        const float* cs = a.rope_cos + static_cast<size_t>(p) * (kDr / 2) + 4 * c;
        const float* sn = a.rope_sin + static_cast<size_t>(p) * (kDr / 2) + 4 * c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x0 = x[2 * i], x1 = x[2 * i + 1];
          x[2 * i] = fmaf(x0, cs[i], -x1 * sn[i]);
          x[2 * i + 1] = fmaf(x0, sn[i], x1 * cs[i]);
        }
      }
      *(lds_bf16x8_t*)(uintptr_t)(smem_base + Fm::kQr + hl * 128 + ((c ^ ((hl >> 2) & 7)) << 4)) =
          to_bf16x8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
    }
  }

  const float scale_log2 = a.scale * kLog2e;
  float m_ref = -INFINITY;  // softmax reference of this lane's head (log2 units)
  float l_run = 0.f;        // this lane's share of the running sum against m_ref
  f32x16 o[kColBlocks];     // O^T block nb: columns 32 nb + 8 (r/4) + 4 h + r%4, head n
#pragma unroll
  for (int nb = 0; nb < kColBlocks; ++nb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) o[nb][r] = 0.f;
    asm volatile("" : "+a"(o[nb]));  // accumulator registers from the start
  }

  // Per-lane parts of the LDS addresses (stage base added per page).
  //   score read, block mb, latent step ks: st + (n * 1024 | ((f(n) ^ h) << 4)) ^ ((2 ks & 31) << 4)
  //                                          + 512 (ks >= 16) + 32768 mb
  //   RoPE read, step rs:  st + kCBytes + n * 128 + (((2 rs + h) ^ ((n >> 2) & 7)) << 4) + 4096 mb
  //   output read (nb, mb, q, part p): lane i = lane % 16 of 16-lane group g = lane / 16 reads
  //     token 32 mb + 16 q + 8 p + 4 (g >> 1) + i / 4, column 32 nb + 16 (g & 1) + 4 (i % 4):
  //     st + (tok_l * 1024 + 8 (i & 1) | (key_l << 4)) ^ (K(nb, p, q) << 4) + 32768 mb + 16384 q + 8192 p
  //     with tok_l = 4 (g >> 1) + i / 4, key_l = (2 (g & 1) + ((i & 3) >> 1)) ^ ((i >> 2) << 2 | (g >> 1)),
  //     K = 4 nb ^ 2 p ^ 16 q.
  const int li = lane & 15, lg = lane >> 4;
  const uint32_t s_lane = static_cast<uint32_t>(n * 1024) | ((swz_f(n) ^ static_cast<uint32_t>(h)) << 4);
  const int tok_l = 4 * (lg >> 1) + (li >> 2);
  const uint32_t key_l = static_cast<uint32_t>((2 * (lg & 1) + ((li & 3) >> 1)) ^ (((li >> 2) << 2) | (lg >> 1)));
  const uint32_t o_lane = static_cast<uint32_t>(tok_l * 1024 + 8 * (li & 1)) | (key_l << 4);

  // Latent-row copies, 128-head form: wave w copies tokens 16 w + r, whose chunk c sits at
  // c ^ swz_f(16 w + r) = c ^ swz_f(r) ^ 16 (w & 1); the lane part of the source offset.
  const uint32_t cp_lane = static_cast<uint32_t>(lane ^ (16 * (wave & 1))) << 4;
  const char* cur_page = page_ptr(0);  // this iteration's page
  int stage = 0;
  for (; j0 < w.k1; j0 += kTok) {
    const int n_valid = min(kTok, w.k1 - j0);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's page copies have landed
    __syncthreads();  // ... and every wave's; the stage of the previous page is free again
    if constexpr (Q) {
      if constexpr (F8)
        convert_page8<HS == 1 ? 16 : 8>(smem_base, wave, lane, n_valid);
      else
        convert_page4<HS == 1 ? 16 : 8>(smem_base, wave, lane);
      __syncthreads();  // the bf16 stage is complete and the quantized stage free again
    }
    // The page whose copies this iteration issues: the next one, into the other stage
    // (a quantized cache: into the quantized stage).
    const int j_next = j0 + kTok;
    const bool has_next = j_next < w.k1;
    const char* next_page = kv;
    const int next_valid = min(kTok, w.k1 - j_next);
    if (has_next) {
      const int i_next = (j_next - w.k0) / kTok;
      if ((i_next & 63) == 0) fetch_ids(i_next >> 6);
      next_page = page_ptr(i_next);
    }
    const uint32_t next_base = Q ? smem_base + kQOff : smem_base + (stage ^ 1) * kStageBytes;
    const uint32_t st_base = smem_base + stage * kStageBytes;
    const uint32_t sb = opaque(st_base + s_lane);
    // ---- scores.  HS = 1: the latent steps, then the RoPE steps, the two 32-token blocks
    // alternating.  HS = 2: this wave's one 32-token block, two chains over alternate
    // K-steps (summed below); bf16: RoPE steps first, FP8: after the latent steps.
    f32x16 s[2];
    {
      const uint32_t rb = opaque(st_base + kCBytes + n * 128);
      // (quantized caches: through an empty asm, so that the q_R addresses are not kept
      // across the loop)
      const uint32_t qb = Q ? opaque(smem_base + Fm::kQr + hl * 128) : smem_base + Fm::kQr + hl * 128;
      const int swr = (n >> 2) & 7, swq = (hl >> 2) & 7;
      auto qr_frag = [&](int rs) { return lds_read8(qb + (((2 * rs + h) ^ swq) << 4)); };
      auto rope_frag = [&](int rs, int mb) { return lds_read8(rb + (((2 * rs + h) ^ swr) << 4) + 4096 * mb); };
      auto lat_frag = [&](int ks, int mb) {
        return lds_read8((sb ^ static_cast<uint32_t>((2 * ks & 31) << 4)) + 512 * (ks >> 4) + 32768 * mb);
      };
      constexpr int kRing = 4;
      bf16x8 ring[kRing];
      if constexpr (HS == 2) {
        // RoPE steps first, then the 32 latent steps of this wave's block through a ring of
        // reads, the two chains over alternate K-steps; the copies go with the odd steps.
#pragma unroll
        for (int rs = 0; rs < kRSteps; ++rs) {
          const bf16x8 qrf = qr_frag(rs);
          const bf16x8 cf = rope_frag(rs, th);
          if (rs < 2)
            mfma32_first(s[rs & 1], cf, qrf);
          else
            mfma32_acc(s[rs & 1], cf, qrf);
        }
#pragma unroll
        for (int st = 0; st < kRing; ++st) ring[st] = lat_frag(st, th);
#pragma unroll
        for (int st = 0; st < kQSteps; ++st) {
          const bf16x8 cf = ring[st % kRing];
          if (st + kRing < kQSteps) ring[st % kRing] = lat_frag(st + kRing, th);
          mfma32_acc(s[st & 1], cf, q[st]);
          if ((st & 1) == 1 && has_next) {
            if constexpr (F8) {  // the 11 copies of the next FP8 page
              if ((st >> 1) < kCopies8)
                load_row8(next_base, next_page, next_valid, wave, static_cast<int>(opaque(lane)), st >> 1);
            } else if constexpr (F4) {  // the 7 copies of the next MXFP4 page
              if ((st >> 1) < kCopies4)
                load_row4(next_base, next_page, next_valid, wave, static_cast<int>(opaque(lane)), st >> 1);
            } else {  // latent rows 0..15 over the 32 steps
              load_row(next_base, next_page, next_valid, wave, static_cast<int>(opaque(lane)), st >> 1);
            }
          }
        }
      } else {
        // The 64 latent (ks, mb) steps, then the 8 RoPE (rs, mb) steps, all through one
        // ring of fragment reads issued kRing steps ahead (the q_R operands of the RoPE
        // steps in a ring of their own), so no step waits for a read issued just before it.
        constexpr int kLat = 2 * kQSteps, kSteps = kLat + 2 * kRSteps;
        auto frag = [&](int st) {
          return st < kLat ? lat_frag(st >> 1, st & 1) : rope_frag((st - kLat) >> 1, st & 1);
        };
        bf16x8 qr_ring[3];  // q_R of RoPE step rs in slot rs % 3, read with rs's first fragment
        auto refill = [&](int st) {  // request the fragment(s) of step st + kRing
          if (st + kRing < kSteps) {
            ring[st % kRing] = frag(st + kRing);
            const int rn = st + kRing - kLat;  // RoPE step of the fragment just requested
            if (rn >= 0 && (rn & 1) == 0) qr_ring[(rn >> 1) % 3] = qr_frag(rn >> 1);
          }
        };
        // Copies of the next page's rows: copy k is prepared at step 4k and issued at step
        // 4k + 2, so each gap between two MFMAs takes only a few of its instructions.  bf16:
        // latent rows k < 16, RoPE rows k = 16, 17, into the other stage.  FP8: code rows
        // k < 8, k_R rows k = 8, 9, the scales k = 10, into the FP8 stage.  The last page
        // copies itself instead (into the unused stage, or the FP8 stage it has converted),
        // so the copies need no branch.
        constexpr int kCopies = Fm::kCopies;
        const char* cp_page = has_next ? next_page : cur_page;
        const int cp_valid = has_next ? next_valid : kTok;
        const int cp_lim = cp_valid - 16 * wave;  // latent row r of this wave is a key iff r < cp_lim
        const uint32_t cp_m0 = next_base + 16384u * static_cast<uint32_t>(wave);
        uint32_t cp_voff = 0, cp_lds = 0;
        auto cp_prepare = [&](int k) {
          if constexpr (F8) {
            // lane through an empty asm, so that no lane constant is kept across the loop
            const int ln = static_cast<int>(opaque(lane));
            if (k < 8) {  // codes of tokens 16 w + 2 k and + 1, one per lane half
              const int t0 = 16 * wave + 2 * k;
              const int tt = t0 + (ln >> 5);
              const int src_t = tt < cp_valid ? tt : 0;
              cp_voff = static_cast<uint32_t>(src_t * kDc + ((ln & 31) << 4));
              cp_lds = next_base + static_cast<uint32_t>(t0 * kDc);
            } else if (k < 10) {  // k_R rows of tokens t0 .. t0 + 7
              const int t0 = wave * 16 + 8 * (k - 8);
              const int tt = t0 + (ln >> 3);
              const int src_t = tt < cp_valid ? tt : 0;
              cp_voff = static_cast<uint32_t>(kR8Off + src_t * 128 + (((ln & 7) ^ ((tt >> 2) & 7)) << 4));
              cp_lds = next_base + static_cast<uint32_t>(kR8Off + t0 * 128);
            } else {  // the scales of tokens 16 w .. +15 (lanes 0..3)
              cp_voff = static_cast<uint32_t>(kS8Off + wave * 64 + 16 * ln);
              cp_lds = next_base + static_cast<uint32_t>(kS8Off + wave * 64);
            }
          } else if constexpr (F4) {
            const int ln = static_cast<int>(opaque(lane));
            if (k < 4) {  // codes of tokens 16 w + 4 k .. +3, one per 16-lane group
              const int t0 = 16 * wave + 4 * k;
              const int tt = t0 + (ln >> 4);
              const int src_t = tt < cp_valid ? tt : 0;
              cp_voff = static_cast<uint32_t>(src_t * (kDc / 2) + ((ln & 15) << 4));
              cp_lds = next_base + static_cast<uint32_t>(t0 * (kDc / 2));
            } else if (k < 6) {  // k_R rows of tokens t0 .. t0 + 7
              const int t0 = wave * 16 + 8 * (k - 4);
              const int tt = t0 + (ln >> 3);
              const int src_t = tt < cp_valid ? tt : 0;
              cp_voff = static_cast<uint32_t>(kR4Off + src_t * 128 + (((ln & 7) ^ ((tt >> 2) & 7)) << 4));
              cp_lds = next_base + static_cast<uint32_t>(kR4Off + t0 * 128);
            } else {  // the scale bytes of tokens 16 w .. +15 (lanes 0..15)
              const int tt = 16 * wave + ln;
              const int src_t = tt < cp_valid ? tt : 0;
              cp_voff = static_cast<uint32_t>(kS4Off + src_t * 16);
              cp_lds = next_base + static_cast<uint32_t>(kS4Off + wave * 256);
            }
          } else if (k < 16) {  // token 16 w + k; rows past the keys fetch token 0
            const int roff = k < cp_lim ? (16 * wave + k) * kRowBytes : 0;
            cp_voff = (cp_lane ^ (swz_f(k) << 4)) + static_cast<uint32_t>(roff);
            cp_lds = cp_m0 + 1024u * static_cast<uint32_t>(k);
          } else {  // RoPE rows of tokens t0 .. t0 + 7
            const int t0 = wave * 16 + 8 * (k - 16);
            const int tt = t0 + (static_cast<int>(opaque(lane)) >> 3);
            const int src_t = tt < cp_valid ? tt : 0;
            cp_voff = static_cast<uint32_t>(src_t * kRowBytes + kDc * 2 +
                                            (((lane & 7) ^ ((tt >> 2) & 7)) << 4));
            cp_lds = next_base + kCBytes + static_cast<uint32_t>(t0 * 128);
          }
        };
        // Issue order = source order within each step: the read for step st + kRing, the
        // MFMA of step st, the copy's part.  (Left to itself the scheduler may move each read
        // next to its MFMA, which then waits for it.)
        auto copy_part = [&](int st) {
          const int k = st >> 2;
          if ((st & 3) == 0 && k < kCopies) cp_prepare(k);
          if ((st & 3) == 2 && k < kCopies) {
            if (F8 && k == 10) {
              if (lane < 4) dma16(cp_page, cp_voff, cp_lds);
            } else if (F4 && k == 6) {
              if (lane < 16) dma16(cp_page, cp_voff, cp_lds);
            } else {
              dma16(cp_page, cp_voff, cp_lds);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        };
#pragma unroll
        for (int st = 0; st < kRing; ++st) ring[st] = frag(st);
#pragma unroll
        for (int st = 0; st < kLat; ++st) {
          const bf16x8 cf = ring[st % kRing];
          refill(st);
          if (st < 2)
            mfma32_first(s[st & 1], cf, q[0]);
          else
            mfma32_acc(s[st & 1], cf, q[st >> 1]);
          copy_part(st);
        }
#pragma unroll
        for (int st = kLat; st < kSteps; ++st) {
          const bf16x8 cf = ring[st % kRing];
          refill(st);
          mfma32_acc(s[st & 1], cf, qr_ring[((st - kLat) >> 1) % 3]);
          copy_part(st);
        }
      }
    }

    // ---- online softmax.  HS = 1: s[mb][r] is the raw score of token 32 mb + 8 (r/4) +
    // 4 h + r%4.  HS = 2: s[0][r] (after the two chains are summed) is that of token
    // 32 th + 8 (r/4) + 4 h + r%4.
    mfma_results_ready(s[0], s[1]);
    if constexpr (HS == 2) s[0] += s[1];
    constexpr int kBlocks = HS == 1 ? 2 : 1;
    if (n_valid < kTok) {
#pragma unroll
      for (int mb = 0; mb < kBlocks; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * (HS == 1 ? mb : th) + 8 * (r >> 2) + 4 * h + (r & 3) >= n_valid) s[mb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < kBlocks; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mb][r]);
    mx = halves_max(mx) * scale_log2;
    // Reference: a head's first page maximum.  Later terms are taken against it, up to
    // 2^kJump (no overflow in fp32 or bf16, whose range is 2^127), so the output is
    // rescaled only when a page's maximum exceeds the reference by more than kJump: the
    // reference moves to that maximum and what was accumulated is multiplied by
    // 2^(old - new).  Output and log-sum-exp are normalised against the final reference,
    // so the result is the same softmax.
    const float m_old = m_ref;
    const bool grow = mx > m_old + kJump;  // true on a head's first page with a key
    if (grow) m_ref = mx;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_old - mx) : 1.f;  // 0 from -inf
    l_run *= alpha;
    if (__builtin_amdgcn_ballot_w64(grow && m_old != -INFINITY) != 0) scale_acc(o, alpha);  // rare
    // With HS = 2 a token half can hold no key yet (the second half of a split's only,
    // partial page): its reference is still -inf and is subtracted as 0, so its
    // exponentials are 0 rather than NaN.
    const float m_sub = (HS == 2 && m_ref == -INFINITY) ? 0.f : m_ref;
    float psum = 0.f;
#pragma unroll
    for (int mb = 0; mb < kBlocks; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][r], scale_log2, -m_sub));
        s[mb][r] = p;
        psum += p;
      }
    l_run += psum;

    // ---- P^T operands: K-step kq = 2 mb + q holds elements 8q .. 8q+7 of block mb
    constexpr int kKQ = 4 / HS;  // 16-token K-steps of the output
    bf16x8 pb[kKQ];
#pragma unroll
    for (int kq = 0; kq < kKQ; ++kq) {
      const f32x16& v = s[kq >> 1];
      const int b8 = 8 * (kq & 1);
      pb[kq] = to_bf16x8(v[b8], v[b8 + 1], v[b8 + 2], v[b8 + 3], v[b8 + 4], v[b8 + 5], v[b8 + 6], v[b8 + 7]);
    }

    // ---- O^T[cols 32 nb .. +31] += C^T . P^T, (kq, nb) steps through a ring
    const uint32_t ob = opaque(st_base + o_lane);
    {
      constexpr int kSteps = kKQ * kColBlocks;
      constexpr int kRing = 4;
      auto frag = [&](int st) {
        const int kq = st / kColBlocks, nb = st % kColBlocks;
        const int mb = HS == 1 ? kq >> 1 : th, qq = HS == 1 ? (kq & 1) : kq;
        const uint32_t k0 = static_cast<uint32_t>((4 * nb) ^ (16 * qq)) << 4;
        const uint32_t k1 = static_cast<uint32_t>((4 * nb) ^ 2 ^ (16 * qq)) << 4;
        const uint32_t a0 = (ob ^ k0) + 32768 * mb + 16384 * qq;
        const uint32_t a1 = (ob ^ k1) + 32768 * mb + 16384 * qq + 8192;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(uintptr_t)a0);
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(uintptr_t)a1);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8 ring[kRing];
#pragma unroll
      for (int st = 0; st < kRing; ++st) ring[st] = frag(st);
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        const bf16x8 cf = ring[st % kRing];
        if (st + kRing < kSteps) ring[st % kRing] = frag(st + kRing);
        const int kq = st / kColBlocks, nb = st % kColBlocks;
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cf, pb[kq], o[nb], 0, 0, 0);
        if constexpr (HS == 2 && !Q) {  // the RoPE rows of the next page
          if ((st == 8 || st == 24) && has_next)
            load_row(next_base, next_page, next_valid, wave, static_cast<int>(opaque(lane)),
                     st == 8 ? 16 : 17);
        }
      }
    }
    // Keep the output accumulators in the accumulator registers across the loop (the
    // allocator otherwise moves some of them to VGPRs and spills).
#pragma unroll
    for (int nb = 0; nb < kColBlocks; ++nb) asm volatile("" : "+a"(o[nb]));
    if constexpr (!Q) stage ^= 1;
    if (has_next) cur_page = next_page;
  }
  // The 128-head form copies on every page, the last one included: its copies must land
  // before the workgroup's LDS is released.
  if constexpr (HS == 1) __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  // ---- finalize: normalise and write this split's partial output (bf16) and LSE
  const float l_tot = halves_sum(l_run);
  if constexpr (HS == 1) {
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int nb = 0; nb < kColBlocks; ++nb) {  // one 32-column block at a time
      asm volatile("" : "+a"(o[nb]));
      const f32x16 v = o[nb];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<bf16x4*>(o_out + 32 * nb + 8 * j + 4 * h) =
            bf16x4{static_cast<__bf16>(v[4 * j] * inv), static_cast<__bf16>(v[4 * j + 1] * inv),
                   static_cast<__bf16>(v[4 * j + 2] * inv), static_cast<__bf16>(v[4 * j + 3] * inv)};
      __builtin_amdgcn_sched_barrier(0);
    }
    if (h == 0) a.lse_part[row] = (m_ref + __log2f(l_tot)) * kLn2;
  } else {
    // Merge the two token halves of each head: wave w keeps column blocks 8 th .. +7 and
    // hands the other 8, with its (m, l), to its partner w ^ 2 through LDS (the stages are
    // free once every wave has finished the last page).  Lane-linear 64-byte slots.
    typedef __attribute__((address_space(3))) f32x16 lds_f32x16_t;
    typedef __attribute__((address_space(3))) float lds_f32_t;
    const uint32_t xo_mine = smem_base + static_cast<uint32_t>(wave) * 32768 + lane * 64;
    const uint32_t xo_part = smem_base + static_cast<uint32_t>(wave ^ 2) * 32768 + lane * 64;
    const uint32_t ml_mine = smem_base + 4 * 32768 + (wave * 64 + lane) * 8;
    const uint32_t ml_part = smem_base + 4 * 32768 + ((wave ^ 2) * 64 + lane) * 8;
    __syncthreads();  // every wave is done with the stages
    auto hand_over = [&](auto first) {  // blocks first .. first + 7 to the partner
#pragma unroll
      for (int i = 0; i < kColBlocks / 2; ++i) {
        asm volatile("" : "+a"(o[decltype(first)::value + i]));
        *(lds_f32x16_t*)(uintptr_t)(xo_mine + i * 4096) = o[decltype(first)::value + i];
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (th == 0)
      hand_over(std::integral_constant<int, 8>{});
    else
      hand_over(std::integral_constant<int, 0>{});
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
    auto finish = [&](auto first) {  // merge and store blocks first .. first + 7
#pragma unroll
      for (int i = 0; i < kColBlocks / 2; ++i) {
        constexpr int kFirst = decltype(first)::value;
        asm volatile("" : "+a"(o[kFirst + i]));
        const f32x16 other = *(lds_f32x16_t*)(uintptr_t)(xo_part + i * 4096);
        const f32x16 v = o[kFirst + i] * w_me + other * w_p;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<bf16x4*>(o_out + 32 * (kFirst + i) + 8 * j + 4 * h) =
              bf16x4{static_cast<__bf16>(v[4 * j]), static_cast<__bf16>(v[4 * j + 1]),
                     static_cast<__bf16>(v[4 * j + 2]), static_cast<__bf16>(v[4 * j + 3])};
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (th == 0)
      finish(std::integral_constant<int, 0>{});
    else
      finish(std::integral_constant<int, 8>{});
    if (th == 0 && h == 0) a.lse_part[row] = (m + __log2f(l)) * kLn2;
  }
}

}  // namespace

bool decode_m32_supported(const DecodeArgs& a, bool bf16) {
  return bf16 && a.heads == kHeads && a.groups == 1 && a.d_c == kDc && a.d_R == kDr &&
         a.page_size == kTok;
}

template <int HS, int KF>
hipError_t launch_decode_m32_k(const DecodeArgs& a, hipStream_t s) {
  static std::atomic<uint64_t> lds_limit_set{0};
  const hipError_t e = ensure_lds_limit(reinterpret_cast<const void*>(decode_m32_kernel<HS, KF>),
                                        Form<KF>::kLds, lds_limit_set);
  if (e != hipSuccess) return e;
  const dim3 grid(a.total_q * a.num_splits * HS);
  decode_m32_kernel<HS, KF><<<grid, kThreads, Form<KF>::kLds, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_decode_m32(const DecodeArgs& a, int head_split, hipStream_t s) {
  return head_split == 2 ? launch_decode_m32_k<2, kFmtBf16>(a, s) : launch_decode_m32_k<1, kFmtBf16>(a, s);
}

bool decode_fp8_supported(const DecodeArgs& a) {
  return a.heads == kHeads && a.groups == 1 && a.d_c == kDc && a.d_R == kDr && a.page_size == kTok;
}

hipError_t launch_decode_fp8(const DecodeArgs& a, int head_split, hipStream_t s) {
  return head_split == 2 ? launch_decode_m32_k<2, kFmtFp8>(a, s) : launch_decode_m32_k<1, kFmtFp8>(a, s);
}

hipError_t launch_decode_mxfp4(const DecodeArgs& a, int head_split, hipStream_t s) {
  return head_split == 2 ? launch_decode_m32_k<2, kFmtFp4>(a, s) : launch_decode_m32_k<1, kFmtFp4>(a, s);
}

}  // namespace mla
