// Host-side launch entry points of the kernels behind the C ABI.  The ABI
// layer (mla_abi.hip) validates arguments and then calls exactly one of these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace mla {

// Raise kernel `fn`'s dynamic-LDS limit to `bytes` on the current device, once per
// device.  `done` holds one bit per device id below 64; concurrent first calls may both
// set the attribute, which is idempotent.  Devices 64 and up set it on every call.
inline hipError_t ensure_lds_limit(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

struct DecodeArgs {
  const void* q_abs;
  const void* q_r;
  const void* kv;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* cu_q;
  const float* rope_cos;
  const float* rope_sin;
  int rope_max_pos;
  void* o_part;      // [T, H, S, d_cg] in the storage type (bf16 or fp32)
  float* lse_part;
  int batch, total_q, max_pages, num_pool_pages;
  int heads, groups, d_c, d_R, page_size, num_splits, pages_per_split;
  float scale;
  int causal;
  int head_split;    // MFMA decode, one latent group: 0 = chosen from the grid size, 1 or 2
};

// mla_decode_paged in two steps.  decode_validate checks every argument on the host
// (o_part / lse_part only when check_parts) and fills *out; it returns MLA_OK without
// filling anything for total_q == 0.  decode_launch picks the kernel for the device and
// enqueues it (returns an MLA_* status).
int decode_validate(const void* q_abs, const void* q_r, const void* kv_cache,
                    const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                    const float* rope_cos, const float* rope_sin, int rope_max_pos, void* o_part,
                    float* lse_part, int batch, int total_q, int max_pages_per_seq,
                    int num_pool_pages, int heads, int groups, int d_hc, int d_c, int d_R,
                    int page_size, int num_splits, int pages_per_split, float softmax_scale,
                    int causal, int dtype, bool check_parts, DecodeArgs* out, bool* bf16);
int decode_launch(DecodeArgs& a, bool bf16, hipStream_t s);

// Decompressed (non-absorbed) branch: K / V up-projection of every cache row of the batch
// into a workspace indexed by physical row, then attention over them.
struct PrefillArgs {
  const void* q_c;         // [T, H, d_hc] bf16
  const void* q_r;         // [T, H, d_R] bf16, before rotation
  const void* kv;          // [num_pool_pages, 64, d_c + d_R] bf16
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* cu_q;
  const float* rope_cos;
  const float* rope_sin;
  int rope_max_pos;
  const void* w_uk;        // [H, d_hc, d_c] bf16
  const void* w_uv;
  void* workspace;         // K then V: [num_pool_pages * 64, H, d_hc] bf16 each
  void* out;               // [T, H, d_hc] bf16
  float* lse_out;          // [T, H] or NULL
  int batch, total_q, max_pages, num_pool_pages, max_q_len;
  int heads, groups, d_hc, d_c, d_R, page_size;
  float scale;
  int causal;
  int dec_pages;  // pages per decompress workgroup; set by launch_decompress
};
bool prefill_supported(const PrefillArgs& a);
hipError_t launch_decompress(const PrefillArgs& a, hipStream_t s);    // K / V into the workspace
hipError_t launch_prefill_attn(const PrefillArgs& a, hipStream_t s);  // attention over them

// Latent-cache append of the new tokens' rows (c_KV | RoPE(k_R, pos)).
struct AppendArgs {
  const void* c_new;   // [T, d_c] storage type
  const void* k_new;   // [T, d_R] storage type, before rotation
  void* kv;            // [num_pool_pages, page_size, d_c + d_R] storage type
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* cu_q;
  const float* rope_cos;  // [rope_max_pos, d_R / 2] or NULL
  const float* rope_sin;
  int rope_max_pos;
  int batch, total_q, max_pages, num_pool_pages;
  int d_c, d_R, page_size;
};
hipError_t launch_append_kv(const AppendArgs& a, bool bf16, hipStream_t s);
// FP8 cache: bf16 inputs, pages of [64][d_c] E4M3 codes, [64][d_R] bf16 k_R, [64] f32 scales.
hipError_t launch_append_kv_fp8(const AppendArgs& a, hipStream_t s);
// MXFP4 cache: bf16 inputs, pages of [64][d_c / 2] packed E2M1 codes, [64][d_R] bf16 k_R,
// [64][d_c / 32] E8M0 scale bytes.
hipError_t launch_append_kv_mxfp4(const AppendArgs& a, hipStream_t s);

// Generic kernels: any (d_cg <= 1024, d_R <= 256), bf16 or fp32 storage.
hipError_t launch_absorb_generic(const void* q_c, const void* w_uk, void* q_abs, int T, int H,
                                 int d_hc, int d_cg, bool bf16, hipStream_t s);
hipError_t launch_up_v_generic(const void* o_lat, const void* w_uv, void* out, int T, int H,
                               int d_hc, int d_cg, bool bf16, hipStream_t s);
hipError_t launch_decode_generic(const DecodeArgs& a, bool bf16, hipStream_t s);

// Combine and RoPE table (one implementation each).
hipError_t launch_combine(const void* o_part, const float* lse_part, void* o_lat, float* lse_out,
                          int T, int H, int d_cg, int S, bool bf16, hipStream_t s);
hipError_t launch_rope_table(float* cos_out, float* sin_out, int max_pos, int d_R, double base,
                             hipStream_t s);

}  // namespace mla

namespace mla {
// MFMA split-KV decode: bf16, 128 heads, d_c 512, d_R 64, one or two latent groups.
// With one latent group the heads of a (token, split) pair are either covered by one
// workgroup (head split 1) or by two of 64 heads each (head split 2, the default when
// 2 * total_q * num_splits <= cu_count, i.e. when one workgroup per pair would leave
// compute units idle).
bool decode_mfma_supported(const DecodeArgs& a, bool bf16);
// 32x32x16 MFMA split-KV decode: bf16, 128 heads, one latent group, d_c 512, d_R 64;
// one workgroup of four 32-head waves per (token, split) (head split 1), or two
// workgroups of 64 heads, each wave covering half of every page's tokens (head split 2).
bool decode_m32_supported(const DecodeArgs& a, bool bf16);
hipError_t launch_decode_m32(const DecodeArgs& a, int head_split, hipStream_t s);
// The same kernel over an FP8 cache (pages of [64][512] E4M3 codes, [64][64] bf16 k_R and
// [64] float32 scales): 128 heads, one latent group, d_c 512, d_R 64.
bool decode_fp8_supported(const DecodeArgs& a);
hipError_t launch_decode_fp8(const DecodeArgs& a, int head_split, hipStream_t s);
// The same kernel over an MXFP4 cache (pages of [64][256] packed E2M1 codes, [64][64] bf16
// k_R and [64][16] E8M0 scale bytes): the shapes decode_fp8_supported accepts.
hipError_t launch_decode_mxfp4(const DecodeArgs& a, int head_split, hipStream_t s);
int decode_mfma_head_split(const DecodeArgs& a, int cu_count);
hipError_t launch_decode_mfma(const DecodeArgs& a, int head_split, hipStream_t s);
}  // namespace mla

namespace mla {
// MFMA projections: bf16; absorb needs d_hc == 128 and d_cg % 64 == 0, up_v needs
// d_hc % 16 == 0 and d_cg in {256, 512}.
bool absorb_mfma_supported(int d_hc, int d_cg, bool bf16);
bool up_v_mfma_supported(int d_hc, int d_cg, bool bf16);
hipError_t launch_absorb_mfma(const void* q_c, const void* w_uk, void* q_abs, int T, int H,
                              int d_hc, int d_cg, hipStream_t s);
hipError_t launch_up_v_mfma(const void* o_lat, const void* w_uv, void* out, int T, int H, int d_hc,
                            int d_cg, hipStream_t s);
// The split merge and up_v in one launch: bf16, d_hc % 64 == 0, d_cg 512 with S <= 16 or
// d_cg 256 with S <= 32.  o_lat and lse_out may be null.
bool merge_up_v_supported(int d_hc, int d_cg, int S, bool bf16);
hipError_t launch_merge_up_v(const void* o_part, const float* lse_part, const void* w_uv, void* o_lat,
                             void* out, float* lse_out, int T, int H, int d_hc, int d_cg, int S,
                             hipStream_t s);
}  // namespace mla
