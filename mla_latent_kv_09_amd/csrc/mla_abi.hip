// C ABI of the MLA decode library: argument validation on the host, then one
// kernel launch per call on the caller's stream.  See include/mla_kv.h for the
// contract of every entry point.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "mla_internal.h"
#include "mla_kv.h"

namespace {

constexpr int kMaxSplits = 256;
constexpr int kMaxGenericCols = 1024;  // d_cg limit of the generic kernels
constexpr int kMaxGenericRope = 256;   // d_R limit of the generic kernels
constexpr int kMaxGenericHeadDim = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dtype(int dtype) {
  return (dtype == MLA_DTYPE_BF16 || dtype == MLA_DTYPE_FP32) ? MLA_OK : MLA_ERR_DTYPE;
}

// Shared checks of heads / groups / latent width.
int check_heads(int heads, int groups, int d_c) {
  if (heads <= 0 || groups <= 0 || d_c <= 0) return MLA_ERR_DIM;
  if (heads % groups != 0 || d_c % groups != 0) return MLA_ERR_DIM;
  return MLA_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_LAUNCH; }

// Decode kernel selection: MLA_KV_DECODE_KERNEL = "generic" forces the shape-generic
// kernel, "mfma" requires an MFMA kernel (unsupported shapes then fail with
// MLA_ERR_UNSUPPORTED) with the head split chosen from the grid size, "mfma128" and
// "mfma64" require the 16x16x32 kernel with one workgroup of 128 heads, resp. two of 64
// heads (one latent group only), per (token, split), "mfma32" requires the 32x32x16
// kernel (one latent group; head split chosen from the grid size), "mfma32-128" and
// "mfma32-64" require it with the given heads per workgroup; anything else picks
// an MFMA kernel whenever the shape has one: for one latent group the 32x32x16 kernel
// when one workgroup per (token, split) fills the device, else the 64-head split.
enum class DecodeKernel { kAuto, kGeneric, kMfma, kMfma128, kMfma64, kMfma32, kMfma32x128, kMfma32x64 };
DecodeKernel decode_kernel_choice() {
  const char* v = getenv("MLA_KV_DECODE_KERNEL");
  if (v == nullptr) return DecodeKernel::kAuto;
  if (strcmp(v, "generic") == 0) return DecodeKernel::kGeneric;
  if (strcmp(v, "mfma") == 0) return DecodeKernel::kMfma;
  if (strcmp(v, "mfma128") == 0) return DecodeKernel::kMfma128;
  if (strcmp(v, "mfma64") == 0) return DecodeKernel::kMfma64;
  if (strcmp(v, "mfma32") == 0) return DecodeKernel::kMfma32;
  if (strcmp(v, "mfma32-128") == 0) return DecodeKernel::kMfma32x128;
  if (strcmp(v, "mfma32-64") == 0) return DecodeKernel::kMfma32x64;
  return DecodeKernel::kAuto;
}

// Compute units of the current device, looked up once per device (0 if unknown).  The
// cache is atomic: concurrent first calls may both query the device and store the same
// value.
int cu_count_of_current_device() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c != 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace

namespace mla {

int decode_validate(const void* q_abs, const void* q_r, const void* kv_cache,
                    const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                    const float* rope_cos, const float* rope_sin, int rope_max_pos, void* o_part,
                    float* lse_part, int batch, int total_q, int max_pages_per_seq,
                    int num_pool_pages, int heads, int groups, int d_hc, int d_c, int d_R,
                    int page_size, int num_splits, int pages_per_split, float softmax_scale,
                    int causal, int dtype, bool check_parts, DecodeArgs* out, bool* bf16) {
  int st = check_dtype(dtype);
  if (st != MLA_OK) return st;
  if (total_q < 0 || batch <= 0 || d_hc <= 0 || d_R <= 0 || (d_R & 1) || num_splits <= 0 ||
      pages_per_split < 0 || max_pages_per_seq <= 0 || num_pool_pages <= 0 || page_size <= 0)
    return MLA_ERR_DIM;
  if ((st = check_heads(heads, groups, d_c)) != MLA_OK) return st;
  if (page_size != MLA_PAGE_SIZE || num_splits > kMaxSplits) return MLA_ERR_UNSUPPORTED;
  if (static_cast<long long>(total_q) * num_splits > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if (static_cast<long long>(max_pages_per_seq) * page_size > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if (d_c / groups > kMaxGenericCols || d_R > kMaxGenericRope) return MLA_ERR_UNSUPPORTED;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return MLA_ERR_NULL;
  if (rope_cos != nullptr && rope_max_pos <= 0) return MLA_ERR_DIM;
  if (total_q == 0) return MLA_OK;
  if (!q_abs || !q_r || !kv_cache || !page_table || !seq_lens || !cu_q) return MLA_ERR_NULL;
  if (check_parts && (!o_part || !lse_part)) return MLA_ERR_NULL;
  const void* ptrs[] = {q_abs, q_r, kv_cache, page_table, seq_lens, cu_q};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MLA_ERR_ALIGN;
  if (check_parts && (!aligned16(o_part) || !aligned16(lse_part))) return MLA_ERR_ALIGN;
  if (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) return MLA_ERR_ALIGN;

  out->q_abs = q_abs;
  out->q_r = q_r;
  out->kv = kv_cache;
  out->page_table = page_table;
  out->seq_lens = seq_lens;
  out->cu_q = cu_q;
  out->rope_cos = rope_cos;
  out->rope_sin = rope_sin;
  out->rope_max_pos = rope_max_pos;
  out->o_part = o_part;
  out->lse_part = lse_part;
  out->batch = batch;
  out->total_q = total_q;
  out->max_pages = max_pages_per_seq;
  out->num_pool_pages = num_pool_pages;
  out->heads = heads;
  out->groups = groups;
  out->d_c = d_c;
  out->d_R = d_R;
  out->page_size = page_size;
  out->num_splits = num_splits;
  // A split longer than the page table covers every page of a sequence: any larger
  // value gives the same plan.
  out->pages_per_split = pages_per_split < max_pages_per_seq ? pages_per_split : max_pages_per_seq;
  out->scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(d_hc + d_R));
  out->causal = causal != 0;
  *bf16 = dtype == MLA_DTYPE_BF16;
  return MLA_OK;
}

int decode_launch(DecodeArgs& a, bool bf16, hipStream_t s) {
  const DecodeKernel choice = decode_kernel_choice();
  if (choice == DecodeKernel::kMfma32 || choice == DecodeKernel::kMfma32x128 ||
      choice == DecodeKernel::kMfma32x64) {
    if (!mla::decode_m32_supported(a, bf16)) return MLA_ERR_UNSUPPORTED;
    a.head_split = choice == DecodeKernel::kMfma32x128 ? 1 : choice == DecodeKernel::kMfma32x64 ? 2 : 0;
    const int hs = mla::decode_mfma_head_split(a, cu_count_of_current_device());
    if (static_cast<long long>(a.total_q) * a.num_splits * hs > INT32_MAX) return MLA_ERR_UNSUPPORTED;
    return launch_status(mla::launch_decode_m32(a, hs, s));
  }
  const bool mfma_ok = mla::decode_mfma_supported(a, bf16);
  const bool mfma_required = choice == DecodeKernel::kMfma || choice == DecodeKernel::kMfma128 ||
                             choice == DecodeKernel::kMfma64;
  if (mfma_required && !mfma_ok) return MLA_ERR_UNSUPPORTED;
  if (choice == DecodeKernel::kMfma64 && a.groups != 1) return MLA_ERR_UNSUPPORTED;
  if (mfma_ok && choice != DecodeKernel::kGeneric) {
    a.head_split = choice == DecodeKernel::kMfma128 ? 1 : choice == DecodeKernel::kMfma64 ? 2 : 0;
    const int hs = mla::decode_mfma_head_split(a, cu_count_of_current_device());
    if (static_cast<long long>(a.total_q) * a.num_splits * hs > INT32_MAX) return MLA_ERR_UNSUPPORTED;
    // One workgroup of 128 heads per (token, split): the 32x32x16 kernel, unless the
    // 16x16x32 one was asked for by name.
    if (hs == 1 && choice != DecodeKernel::kMfma128 && mla::decode_m32_supported(a, bf16))
      return launch_status(mla::launch_decode_m32(a, 1, s));
    return launch_status(mla::launch_decode_mfma(a, hs, s));
  }
  return launch_status(mla::launch_decode_generic(a, bf16, s));
}


}  // namespace mla

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_DIM: return "invalid dimension (non-positive size, heads or d_c not divisible by "
                             "groups, or odd d_R)";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration (page_size must be 64; "
                                     "dimension or split count beyond the implemented limits)";
    case MLA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MLA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case MLA_ERR_DTYPE: return "unknown dtype";
    default: return "unknown status";
  }
}

size_t mla_decode_workspace_bytes(int total_q, int heads, int groups, int d_c, int num_splits,
                                  int dtype) {
  if (total_q < 0 || num_splits <= 0 || check_heads(heads, groups, d_c) != MLA_OK) return 0;
  if (check_dtype(dtype) != MLA_OK) return 0;
  const size_t elem = dtype == MLA_DTYPE_BF16 ? 2 : 4;
  const size_t rows = static_cast<size_t>(total_q) * heads * num_splits;
  return rows * (static_cast<size_t>(d_c / groups) * elem + sizeof(float));
}

int mla_absorb_q(const void* q_c, const void* w_uk, void* q_abs, int total_q, int heads, int groups,
                 int d_hc, int d_c, int dtype, void* stream) {
  int st = check_dtype(dtype);
  if (st != MLA_OK) return st;
  if (total_q < 0 || d_hc <= 0) return MLA_ERR_DIM;
  if ((st = check_heads(heads, groups, d_c)) != MLA_OK) return st;
  if (d_hc > kMaxGenericHeadDim) return MLA_ERR_UNSUPPORTED;
  if (total_q == 0) return MLA_OK;
  if (!q_c || !w_uk || !q_abs) return MLA_ERR_NULL;
  if (!aligned16(q_c) || !aligned16(w_uk) || !aligned16(q_abs)) return MLA_ERR_ALIGN;
  const bool bf16 = dtype == MLA_DTYPE_BF16;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (mla::absorb_mfma_supported(d_hc, d_c / groups, bf16))
    return launch_status(mla::launch_absorb_mfma(q_c, w_uk, q_abs, total_q, heads, d_hc,
                                                 d_c / groups, s));
  return launch_status(mla::launch_absorb_generic(q_c, w_uk, q_abs, total_q, heads, d_hc,
                                                  d_c / groups, bf16, s));
}

int mla_rope_table(float* cos_out, float* sin_out, int max_pos, int d_R, double base, void* stream) {
  if (max_pos <= 0 || d_R <= 0 || (d_R & 1) || !(base > 0.0)) return MLA_ERR_DIM;
  if (!cos_out || !sin_out) return MLA_ERR_NULL;
  if (!aligned16(cos_out) || !aligned16(sin_out)) return MLA_ERR_ALIGN;
  return launch_status(mla::launch_rope_table(cos_out, sin_out, max_pos, d_R, base,
                                              static_cast<hipStream_t>(stream)));
}

int mla_decode_paged(const void* q_abs, const void* q_r, const void* kv_cache,
                     const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                     const float* rope_cos, const float* rope_sin, int rope_max_pos,
                     void* o_part, float* lse_part, int batch, int total_q, int max_pages_per_seq,
                     int num_pool_pages, int heads, int groups, int d_hc, int d_c, int d_R,
                     int page_size, int num_splits, int pages_per_split, float softmax_scale,
                     int causal, int dtype, void* stream) {
  mla::DecodeArgs a{};
  bool bf16 = false;
  const int st = mla::decode_validate(q_abs, q_r, kv_cache, page_table, seq_lens, cu_q, rope_cos,
                                      rope_sin, rope_max_pos, o_part, lse_part, batch, total_q,
                                      max_pages_per_seq, num_pool_pages, heads, groups, d_hc, d_c,
                                      d_R, page_size, num_splits, pages_per_split, softmax_scale,
                                      causal, dtype, true, &a, &bf16);
  if (st != MLA_OK || total_q == 0) return st;
  return mla::decode_launch(a, bf16, static_cast<hipStream_t>(stream));
}

int mla_append_kv(const void* c_kv_new, const void* k_r_new, void* kv_cache,
                  const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                  const float* rope_cos, const float* rope_sin, int rope_max_pos, int batch,
                  int total_q, int max_pages_per_seq, int num_pool_pages, int d_c, int d_R,
                  int page_size, int dtype, void* stream) {
  int st = check_dtype(dtype);
  if (st != MLA_OK) return st;
  if (total_q < 0 || batch <= 0 || d_c <= 0 || d_R <= 0 || (d_R & 1) || max_pages_per_seq <= 0 ||
      num_pool_pages <= 0 || page_size <= 0)
    return MLA_ERR_DIM;
  if (page_size != MLA_PAGE_SIZE) return MLA_ERR_UNSUPPORTED;
  const int piece = dtype == MLA_DTYPE_BF16 ? 8 : 4;  // elements per 16-byte piece
  if (d_c % piece != 0 || d_R % piece != 0) return MLA_ERR_UNSUPPORTED;
  if (static_cast<long long>(max_pages_per_seq) * page_size > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if (static_cast<long long>(total_q) * ((d_c + d_R) / piece) > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return MLA_ERR_NULL;
  if (rope_cos != nullptr && rope_max_pos <= 0) return MLA_ERR_DIM;
  if (total_q == 0) return MLA_OK;
  if (!c_kv_new || !k_r_new || !kv_cache || !page_table || !seq_lens || !cu_q) return MLA_ERR_NULL;
  const void* ptrs[] = {c_kv_new, k_r_new, kv_cache, page_table, seq_lens, cu_q};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MLA_ERR_ALIGN;
  if (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) return MLA_ERR_ALIGN;
  mla::AppendArgs a{};
  a.c_new = c_kv_new;
  a.k_new = k_r_new;
  a.kv = kv_cache;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.cu_q = cu_q;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.rope_max_pos = rope_max_pos;
  a.batch = batch;
  a.total_q = total_q;
  a.max_pages = max_pages_per_seq;
  a.num_pool_pages = num_pool_pages;
  a.d_c = d_c;
  a.d_R = d_R;
  a.page_size = page_size;
  return launch_status(mla::launch_append_kv(a, dtype == MLA_DTYPE_BF16,
                                             static_cast<hipStream_t>(stream)));
}

size_t mla_prefill_workspace_bytes(int num_pool_pages, int heads, int d_hc, int dtype) {
  if (num_pool_pages <= 0 || heads <= 0 || d_hc <= 0 || dtype != MLA_DTYPE_BF16) return 0;
  return 2 * static_cast<size_t>(num_pool_pages) * MLA_PAGE_SIZE * heads * d_hc * 2;
}

int mla_branch(const int32_t* q_lens, int batch, int threshold) {
  if (!q_lens) return MLA_ERR_NULL;
  if (batch <= 0 || threshold <= 0) return MLA_ERR_DIM;
  int max_q = 0;
  for (int b = 0; b < batch; ++b) {
    if (q_lens[b] < 0) return MLA_ERR_DIM;
    max_q = q_lens[b] > max_q ? q_lens[b] : max_q;
  }
  return max_q >= threshold ? MLA_BRANCH_DECOMPRESSED : MLA_BRANCH_ABSORBED;
}

// Checks of the decompressed branch's calls.  Stage 1 = mla_decompress_kv (cache, page
// table, lengths, weights, workspace), 2 = mla_prefill_attention (queries, cache, page
// table, lengths, query offsets, workspace, output), 3 = both.  Fills *a on success.
int prefill_validate(int stage, const void* q_c, const void* q_r, const void* kv_cache,
                     const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                     const float* rope_cos, const float* rope_sin, int rope_max_pos,
                     const void* w_uk, const void* w_uv, void* workspace, void* out,
                     float* lse_out, int batch, int total_q, int max_pages_per_seq,
                     int num_pool_pages, int max_q_len, int heads, int groups, int d_hc, int d_c,
                     int d_R, int page_size, float softmax_scale, int causal, int dtype,
                     mla::PrefillArgs* a) {
  int st = check_dtype(dtype);
  if (st != MLA_OK) return st;
  const bool attn = stage & 2, dec = stage & 1;
  if (total_q < 0 || batch <= 0 || (attn && max_q_len <= 0) || d_hc <= 0 || d_R <= 0 || (d_R & 1) ||
      max_pages_per_seq <= 0 || num_pool_pages <= 0 || page_size <= 0)
    return MLA_ERR_DIM;
  if ((st = check_heads(heads, groups, d_c)) != MLA_OK) return st;
  a->groups = groups;
  a->d_hc = d_hc;
  a->d_c = d_c;
  a->d_R = d_R;
  a->page_size = page_size;
  if (dtype != MLA_DTYPE_BF16 || !mla::prefill_supported(*a)) return MLA_ERR_UNSUPPORTED;
  if (static_cast<long long>(max_pages_per_seq) * page_size > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  const long long q_blocks = attn ? (static_cast<long long>(max_q_len) + 127) / 128 : 0;
  const long long dec_runs = (static_cast<long long>(max_pages_per_seq) + 7) / 8;
  if (q_blocks * batch * heads > INT32_MAX || dec_runs * batch * heads > INT32_MAX ||
      static_cast<long long>(num_pool_pages) * page_size * heads > INT32_MAX)
    return MLA_ERR_UNSUPPORTED;
  if (attn && (rope_cos == nullptr) != (rope_sin == nullptr)) return MLA_ERR_NULL;
  if (attn && rope_cos != nullptr && rope_max_pos <= 0) return MLA_ERR_DIM;
  if (total_q == 0) return MLA_OK;
  if (!kv_cache || !page_table || !seq_lens || !workspace) return MLA_ERR_NULL;
  if (dec && (!w_uk || !w_uv)) return MLA_ERR_NULL;
  if (attn && (!q_c || !q_r || !cu_q || !out)) return MLA_ERR_NULL;
  const void* ptrs[] = {kv_cache, page_table, seq_lens, workspace};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MLA_ERR_ALIGN;
  if (dec && (!aligned16(w_uk) || !aligned16(w_uv))) return MLA_ERR_ALIGN;
  if (attn) {
    const void* aptrs[] = {q_c, q_r, cu_q, out};
    for (const void* p : aptrs)
      if (!aligned16(p)) return MLA_ERR_ALIGN;
    if (lse_out && !aligned16(lse_out)) return MLA_ERR_ALIGN;
    if (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) return MLA_ERR_ALIGN;
  }
  a->q_c = q_c;
  a->q_r = q_r;
  a->kv = kv_cache;
  a->page_table = page_table;
  a->seq_lens = seq_lens;
  a->cu_q = cu_q;
  a->rope_cos = rope_cos;
  a->rope_sin = rope_sin;
  a->rope_max_pos = rope_max_pos;
  a->w_uk = w_uk;
  a->w_uv = w_uv;
  a->workspace = workspace;
  a->out = out;
  a->lse_out = lse_out;
  a->batch = batch;
  a->total_q = total_q;
  a->max_pages = max_pages_per_seq;
  a->num_pool_pages = num_pool_pages;
  a->max_q_len = max_q_len;
  a->heads = heads;
  a->scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(d_hc + d_R));
  a->causal = causal != 0;
  return MLA_OK;
}

int mla_prefill_paged(const void* q_c, const void* q_r, const void* kv_cache,
                      const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                      const float* rope_cos, const float* rope_sin, int rope_max_pos,
                      const void* w_uk, const void* w_uv, void* workspace, void* out,
                      float* lse_out, int batch, int total_q, int max_pages_per_seq,
                      int num_pool_pages, int max_q_len, int heads, int groups, int d_hc,
                      int d_c, int d_R, int page_size, float softmax_scale, int causal, int dtype,
                      void* stream) {
  mla::PrefillArgs a{};
  const int st = prefill_validate(3, q_c, q_r, kv_cache, page_table, seq_lens, cu_q, rope_cos,
                                  rope_sin, rope_max_pos, w_uk, w_uv, workspace, out, lse_out,
                                  batch, total_q, max_pages_per_seq, num_pool_pages, max_q_len,
                                  heads, groups, d_hc, d_c, d_R, page_size, softmax_scale, causal,
                                  dtype, &a);
  if (st != MLA_OK || total_q == 0) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int sd = launch_status(mla::launch_decompress(a, s));
  if (sd != MLA_OK) return sd;
  return launch_status(mla::launch_prefill_attn(a, s));
}

int mla_decompress_kv(const void* kv_cache, const int32_t* page_table, const int32_t* seq_lens,
                      const void* w_uk, const void* w_uv, void* workspace, int batch,
                      int max_pages_per_seq, int num_pool_pages, int heads, int groups, int d_hc,
                      int d_c, int d_R, int page_size, int dtype, void* stream) {
  mla::PrefillArgs a{};
  const int st = prefill_validate(1, nullptr, nullptr, kv_cache, page_table, seq_lens, nullptr,
                                  nullptr, nullptr, 0, w_uk, w_uv, workspace, nullptr, nullptr,
                                  batch, 1, max_pages_per_seq, num_pool_pages, 0, heads, groups,
                                  d_hc, d_c, d_R, page_size, 0.f, 1, dtype, &a);
  if (st != MLA_OK) return st;
  return launch_status(mla::launch_decompress(a, static_cast<hipStream_t>(stream)));
}

int mla_prefill_attention(const void* q_c, const void* q_r, const void* kv_cache,
                          const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                          const float* rope_cos, const float* rope_sin, int rope_max_pos,
                          const void* workspace, void* out, float* lse_out, int batch,
                          int total_q, int max_pages_per_seq, int num_pool_pages, int max_q_len,
                          int heads, int groups, int d_hc, int d_c, int d_R, int page_size,
                          float softmax_scale, int causal, int dtype, void* stream) {
  mla::PrefillArgs a{};
  const int st = prefill_validate(2, q_c, q_r, kv_cache, page_table, seq_lens, cu_q, rope_cos,
                                  rope_sin, rope_max_pos, nullptr, nullptr,
                                  const_cast<void*>(workspace), out, lse_out, batch, total_q,
                                  max_pages_per_seq, num_pool_pages, max_q_len, heads, groups,
                                  d_hc, d_c, d_R, page_size, softmax_scale, causal, dtype, &a);
  if (st != MLA_OK || total_q == 0) return st;
  return launch_status(mla::launch_prefill_attn(a, static_cast<hipStream_t>(stream)));
}

size_t mla_fp8_page_bytes(int d_c, int d_R) {
  if (d_c <= 0 || d_R <= 0 || (d_R & 1)) return 0;
  return static_cast<size_t>(MLA_PAGE_SIZE) * (static_cast<size_t>(d_c) + 2 * d_R + 4);
}

int mla_append_kv_fp8(const void* c_kv_new, const void* k_r_new, void* kv_cache,
                      const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                      const float* rope_cos, const float* rope_sin, int rope_max_pos, int batch,
                      int total_q, int max_pages_per_seq, int num_pool_pages, int d_c, int d_R,
                      int page_size, void* stream) {
  if (total_q < 0 || batch <= 0 || d_c <= 0 || d_R <= 0 || (d_R & 1) || max_pages_per_seq <= 0 ||
      num_pool_pages <= 0 || page_size <= 0)
    return MLA_ERR_DIM;
  if (page_size != MLA_PAGE_SIZE) return MLA_ERR_UNSUPPORTED;
  if (d_c % 8 != 0 || d_R % 8 != 0 || d_c > 512 || d_R > 512) return MLA_ERR_UNSUPPORTED;
  if (static_cast<long long>(max_pages_per_seq) * page_size > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return MLA_ERR_NULL;
  if (rope_cos != nullptr && rope_max_pos <= 0) return MLA_ERR_DIM;
  if (total_q == 0) return MLA_OK;
  if (!c_kv_new || !k_r_new || !kv_cache || !page_table || !seq_lens || !cu_q) return MLA_ERR_NULL;
  const void* ptrs[] = {c_kv_new, k_r_new, kv_cache, page_table, seq_lens, cu_q};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MLA_ERR_ALIGN;
  if (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) return MLA_ERR_ALIGN;
  mla::AppendArgs a{};
  a.c_new = c_kv_new;
  a.k_new = k_r_new;
  a.kv = kv_cache;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.cu_q = cu_q;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.rope_max_pos = rope_max_pos;
  a.batch = batch;
  a.total_q = total_q;
  a.max_pages = max_pages_per_seq;
  a.num_pool_pages = num_pool_pages;
  a.d_c = d_c;
  a.d_R = d_R;
  a.page_size = page_size;
  return launch_status(mla::launch_append_kv_fp8(a, static_cast<hipStream_t>(stream)));
}

int mla_decode_paged_fp8(const void* q_abs, const void* q_r, const void* kv_cache,
                         const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                         const float* rope_cos, const float* rope_sin, int rope_max_pos,
                         void* o_part, float* lse_part, int batch, int total_q,
                         int max_pages_per_seq, int num_pool_pages, int heads, int groups, int d_hc,
                         int d_c, int d_R, int page_size, int num_splits, int pages_per_split,
                         float softmax_scale, int causal, void* stream) {
  mla::DecodeArgs a{};
  bool bf16 = false;
  int st = mla::decode_validate(q_abs, q_r, kv_cache, page_table, seq_lens, cu_q, rope_cos,
                                rope_sin, rope_max_pos, o_part, lse_part, batch, total_q,
                                max_pages_per_seq, num_pool_pages, heads, groups, d_hc, d_c, d_R,
                                page_size, num_splits, pages_per_split, softmax_scale, causal,
                                MLA_DTYPE_BF16, true, &a, &bf16);
  if (st != MLA_OK) return st;
  mla::DecodeArgs shape{};
  shape.heads = heads;
  shape.groups = groups;
  shape.d_c = d_c;
  shape.d_R = d_R;
  shape.page_size = page_size;
  if (!mla::decode_fp8_supported(shape)) return MLA_ERR_UNSUPPORTED;
  if (total_q == 0) return MLA_OK;
  const DecodeKernel choice = decode_kernel_choice();
  a.head_split = choice == DecodeKernel::kMfma32x128 ? 1 : choice == DecodeKernel::kMfma32x64 ? 2 : 0;
  const int hs = mla::decode_mfma_head_split(a, cu_count_of_current_device());
  if (static_cast<long long>(total_q) * num_splits * hs > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  return launch_status(mla::launch_decode_fp8(a, hs, static_cast<hipStream_t>(stream)));
}

size_t mla_mxfp4_page_bytes(int d_c, int d_R) {
  if (d_c <= 0 || d_R <= 0 || (d_R & 1) || d_c % 32 != 0) return 0;
  return static_cast<size_t>(MLA_PAGE_SIZE) * (static_cast<size_t>(d_c) / 2 + 2 * d_R + d_c / 32);
}

int mla_append_kv_mxfp4(const void* c_kv_new, const void* k_r_new, void* kv_cache,
                        const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                        const float* rope_cos, const float* rope_sin, int rope_max_pos, int batch,
                        int total_q, int max_pages_per_seq, int num_pool_pages, int d_c, int d_R,
                        int page_size, void* stream) {
  if (total_q < 0 || batch <= 0 || d_c <= 0 || d_R <= 0 || (d_R & 1) || max_pages_per_seq <= 0 ||
      num_pool_pages <= 0 || page_size <= 0)
    return MLA_ERR_DIM;
  if (page_size != MLA_PAGE_SIZE) return MLA_ERR_UNSUPPORTED;
  if (d_c % 32 != 0 || d_R % 8 != 0 || d_c > 512 || d_R > 512) return MLA_ERR_UNSUPPORTED;
  if (static_cast<long long>(max_pages_per_seq) * page_size > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return MLA_ERR_NULL;
  if (rope_cos != nullptr && rope_max_pos <= 0) return MLA_ERR_DIM;
  if (total_q == 0) return MLA_OK;
  if (!c_kv_new || !k_r_new || !kv_cache || !page_table || !seq_lens || !cu_q) return MLA_ERR_NULL;
  const void* ptrs[] = {c_kv_new, k_r_new, kv_cache, page_table, seq_lens, cu_q};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MLA_ERR_ALIGN;
  if (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) return MLA_ERR_ALIGN;
  mla::AppendArgs a{};
  a.c_new = c_kv_new;
  a.k_new = k_r_new;
  a.kv = kv_cache;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.cu_q = cu_q;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.rope_max_pos = rope_max_pos;
  a.batch = batch;
  a.total_q = total_q;
  a.max_pages = max_pages_per_seq;
  a.num_pool_pages = num_pool_pages;
  a.d_c = d_c;
  a.d_R = d_R;
  a.page_size = page_size;
  return launch_status(mla::launch_append_kv_mxfp4(a, static_cast<hipStream_t>(stream)));
}

int mla_decode_paged_mxfp4(const void* q_abs, const void* q_r, const void* kv_cache,
                           const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                           const float* rope_cos, const float* rope_sin, int rope_max_pos,
                           void* o_part, float* lse_part, int batch, int total_q,
                           int max_pages_per_seq, int num_pool_pages, int heads, int groups,
                           int d_hc, int d_c, int d_R, int page_size, int num_splits,
                           int pages_per_split, float softmax_scale, int causal, void* stream) {
  mla::DecodeArgs a{};
  bool bf16 = false;
  int st = mla::decode_validate(q_abs, q_r, kv_cache, page_table, seq_lens, cu_q, rope_cos,
                                rope_sin, rope_max_pos, o_part, lse_part, batch, total_q,
                                max_pages_per_seq, num_pool_pages, heads, groups, d_hc, d_c, d_R,
                                page_size, num_splits, pages_per_split, softmax_scale, causal,
                                MLA_DTYPE_BF16, true, &a, &bf16);
  if (st != MLA_OK) return st;
  mla::DecodeArgs shape{};
  shape.heads = heads;
  shape.groups = groups;
  shape.d_c = d_c;
  shape.d_R = d_R;
  shape.page_size = page_size;
  if (!mla::decode_fp8_supported(shape)) return MLA_ERR_UNSUPPORTED;  // the same shapes
  if (total_q == 0) return MLA_OK;
  const DecodeKernel choice = decode_kernel_choice();
  a.head_split = choice == DecodeKernel::kMfma32x128 ? 1 : choice == DecodeKernel::kMfma32x64 ? 2 : 0;
  const int hs = mla::decode_mfma_head_split(a, cu_count_of_current_device());
  if (static_cast<long long>(total_q) * num_splits * hs > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  return launch_status(mla::launch_decode_mxfp4(a, hs, static_cast<hipStream_t>(stream)));
}

int mla_combine(const void* o_part, const float* lse_part, void* o_latent, float* lse_out,
                int total_q, int heads, int groups, int d_c, int num_splits, int dtype,
                void* stream) {
  int st = check_dtype(dtype);
  if (st != MLA_OK) return st;
  if (total_q < 0 || num_splits <= 0) return MLA_ERR_DIM;
  if ((st = check_heads(heads, groups, d_c)) != MLA_OK) return st;
  if (num_splits > kMaxSplits) return MLA_ERR_UNSUPPORTED;
  if (total_q == 0) return MLA_OK;
  if (!o_part || !lse_part || !o_latent) return MLA_ERR_NULL;
  if (!aligned16(o_part) || !aligned16(lse_part) || !aligned16(o_latent) ||
      (lse_out && !aligned16(lse_out)))
    return MLA_ERR_ALIGN;
  const bool bf16 = dtype == MLA_DTYPE_BF16;
  return launch_status(mla::launch_combine(o_part, lse_part, o_latent, lse_out, total_q, heads,
                                           d_c / groups, num_splits, bf16,
                                           static_cast<hipStream_t>(stream)));
}

int mla_up_v(const void* o_latent, const void* w_uv, void* out, int total_q, int heads, int groups,
             int d_hc, int d_c, int dtype, void* stream) {
  int st = check_dtype(dtype);
  if (st != MLA_OK) return st;
  if (total_q < 0 || d_hc <= 0) return MLA_ERR_DIM;
  if ((st = check_heads(heads, groups, d_c)) != MLA_OK) return st;
  if (d_c / groups > kMaxGenericCols) return MLA_ERR_UNSUPPORTED;
  if (total_q == 0) return MLA_OK;
  if (!o_latent || !w_uv || !out) return MLA_ERR_NULL;
  if (!aligned16(o_latent) || !aligned16(w_uv) || !aligned16(out)) return MLA_ERR_ALIGN;
  const bool bf16 = dtype == MLA_DTYPE_BF16;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (mla::up_v_mfma_supported(d_hc, d_c / groups, bf16))
    return launch_status(mla::launch_up_v_mfma(o_latent, w_uv, out, total_q, heads, d_hc,
                                               d_c / groups, s));
  return launch_status(mla::launch_up_v_generic(o_latent, w_uv, out, total_q, heads, d_hc,
                                                d_c / groups, bf16, s));
}

int mla_combine_up_v_fused(int heads, int groups, int d_hc, int d_c, int num_splits, int dtype) {
  if (check_dtype(dtype) != MLA_OK || check_heads(heads, groups, d_c) != MLA_OK) return 0;
  return mla::merge_up_v_supported(d_hc, d_c / groups, num_splits, dtype == MLA_DTYPE_BF16) ? 1 : 0;
}

int mla_combine_up_v(const void* o_part, const float* lse_part, const void* w_uv, void* o_latent,
                     void* out, float* lse_out, int total_q, int heads, int groups, int d_hc,
                     int d_c, int num_splits, int dtype, void* stream) {
  int st = check_dtype(dtype);
  if (st != MLA_OK) return st;
  if (total_q < 0 || num_splits <= 0 || d_hc <= 0) return MLA_ERR_DIM;
  if ((st = check_heads(heads, groups, d_c)) != MLA_OK) return st;
  if (num_splits > kMaxSplits || d_c / groups > kMaxGenericCols) return MLA_ERR_UNSUPPORTED;
  const bool fused = mla_combine_up_v_fused(heads, groups, d_hc, d_c, num_splits, dtype) != 0;
  if (!fused && o_latent == nullptr) return MLA_ERR_UNSUPPORTED;
  if (total_q == 0) return MLA_OK;
  if (!o_part || !lse_part || !w_uv || !out) return MLA_ERR_NULL;
  if (!aligned16(o_part) || !aligned16(lse_part) || !aligned16(w_uv) || !aligned16(out) ||
      (o_latent && !aligned16(o_latent)) || (lse_out && !aligned16(lse_out)))
    return MLA_ERR_ALIGN;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (fused)
    return launch_status(mla::launch_merge_up_v(o_part, lse_part, w_uv, o_latent, out, lse_out,
                                                total_q, heads, d_hc, d_c / groups, num_splits, s));
  st = mla_combine(o_part, lse_part, o_latent, lse_out, total_q, heads, groups, d_c, num_splits,
                   dtype, stream);
  if (st != MLA_OK) return st;
  return mla_up_v(o_latent, w_uv, out, total_q, heads, groups, d_hc, d_c, dtype, stream);
}

}  // extern "C"
