/*
 * mla_kv.h -- C ABI of the MI355X (gfx950) absorbed-MLA decode library.
 *
 * One decode step of Multi-head Latent Attention over a paged latent cache,
 * split into four stream-ordered calls:
 *
 *   mla_absorb_q      q_abs[t,h,:] = q_c[t,h,:] . W_UK[h]            (absorption)
 *   mla_decode_paged  split-KV attention of q_abs / RoPE(q_R) against the
 *                     paged latent rows [c_KV | k_R]; per-split partial
 *                     outputs and log-sum-exp
 *   mla_combine       log-sum-exp merge of the splits -> o_latent
 *   mla_up_v          out[t,h,:] = W_UV[h] . o_latent[t,h,:]            (value up-projection)
 *
 * (mla_combine_up_v issues the last two as one launch where its fused kernel covers
 * the shape, with the same results),
 * plus mla_rope_table (the fp32 cos/sin table the decode call reads),
 * mla_append_kv (writes the new tokens' latent rows, with their rotated RoPE keys,
 * into the paged cache before the decode reads them), mla_decode_plan (host-only
 * split plan) and mla_status_string.  Further down: the quantized caches (FP8 and MXFP4
 * pages, with their own append and decode calls) and the decompressed branch.
 *
 * Sources, cited by page address and section:
 *   P3 = www.nxmr.cn/news/151634  (MLA operators: absorption, paged latent cache)
 *   P2 = m.xxqk.cn/news/443191    (attention from MHA to MoBA)
 *   P1 = www.hotelren.com/news/5324130 (from MLA to GLA)
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensors are dense, row-major, in device memory allocated and owned by
 *   the caller.  The library never allocates, frees or keeps a pointer after a
 *   call returns, and never synchronizes.  Work is enqueued on `stream`
 *   (a hipStream_t; NULL = the default stream) and runs asynchronously.
 *   Calls may be issued from several host threads.  The only state kept between
 *   calls is filled once per device and is safe under concurrent first calls: the
 *   device's compute-unit count and each decode kernel's dynamic-LDS limit.  The
 *   decode-kernel override MLA_KV_DECODE_KERNEL is read from the environment on
 *   every mla_decode_paged call.
 * - Every pointer must be 16-byte aligned (the pages' "misaligned address"
 *   failure of a vectorized gather, P3 §5).
 * - dtype selects the storage type of the non-float32 tensors: MLA_DTYPE_BF16
 *   (bfloat16 storage and MFMA operands, fp32 accumulation) or MLA_DTYPE_FP32.
 *   Softmax state and the log-sum-exp are always float32; split partial outputs
 *   are kept in the storage type (see mla_decode_paged).
 * - Indices: T = total query tokens of the batch (queries of all sequences
 *   packed back to back), H = heads, G = latent groups (1 = MLA; >1 = grouped
 *   latent attention, P1 §1), d_cg = d_c / G.  Head h belongs to group
 *   h / (H/G) and sees latent columns [g*d_cg, (g+1)*d_cg) plus the shared k_R.
 * - Return value: MLA_OK (0) or a negative MLA_ERR_* code.  Every code except
 *   MLA_ERR_LAUNCH is detected on the host before anything is enqueued.  A call
 *   with total_q == 0 validates nothing but its scalars and enqueues nothing.
 *
 * Memory-resident contents (page ids, sequence lengths, query offsets) are
 * trusted: the kernels clamp every index they derive from them so no access
 * leaves the buffers described here, but the result for out-of-range contents
 * is unspecified.
 */
#ifndef MLA_KV_H
#define MLA_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,        /* a required pointer is NULL */
  MLA_ERR_DIM = -2,         /* a size <= 0 (or < 0 where 0 is allowed), H % G, d_c % G, odd d_R */
  MLA_ERR_UNSUPPORTED = -3, /* valid but not implemented: page_size != 64, dims beyond limits */
  MLA_ERR_ALIGN = -4,       /* a pointer not 16-byte aligned */
  MLA_ERR_LAUNCH = -5,      /* the HIP runtime rejected a kernel launch */
  MLA_ERR_DTYPE = -6        /* dtype is not one of MLA_DTYPE_* */
};

enum mla_dtype {
  MLA_DTYPE_BF16 = 0,
  MLA_DTYPE_FP32 = 1
};

/* Only page size the library implements: 64 tokens per page (P3 §3: a 64-token
 * page of 576-element bf16 rows is about 72 KB; 16-token pages fragment the
 * page table and the transfers). */
#define MLA_PAGE_SIZE 64

/*
 * mla_absorb_q -- fold W_UK into the content query (P3 §1 intro and §4 path B:
 * q_abs = q_c W_UK, so scores are taken against the latent directly and K is
 * never re-expanded).
 *
 *   q_c    [T, H, d_hc]      dtype
 *   w_uk   [H, d_hc, d_cg]   dtype   ("hdc" order of P3 §4)
 *   q_abs  [T, H, d_cg]      dtype   output; q_abs[t,h,c] = sum_d q_c[t,h,d] w_uk[h,d,c],
 *                                    accumulated in fp32, rounded once to dtype
 */
int mla_absorb_q(const void* q_c, const void* w_uk, void* q_abs,
                 int total_q, int heads, int groups, int d_hc, int d_c,
                 int dtype, void* stream);

/*
 * mla_rope_table -- fp32 RoPE table for positions [0, max_pos) (P3 §3
 * rope_compute_dtype fp32; P3 §4: generate the table in FP32 and apply it with
 * FP32 multiply-adds, since an fp16 table shifts the phase).
 *
 *   cos_out, sin_out  [max_pos, d_R/2] float32 outputs:
 *     angle(p, k) = p * base^(-2k/d_R), evaluated in float64, then
 *     cos_out[p,k] = (float)cos(angle), sin_out[p,k] = (float)sin(angle).
 * The decode call rotates the interleaved pairs (q_R[2k], q_R[2k+1]) with it.
 */
int mla_rope_table(float* cos_out, float* sin_out, int max_pos, int d_R, double base,
                   void* stream);

/*
 * mla_decode_paged -- split-KV attention of the absorbed queries over the
 * paged latent cache (P3 §1: the cache row of a token is the 512-d c_KV plus
 * the 64-d decoupled RoPE key k_R; P3 §3: bf16 rows, page_size 64; P3 §4:
 * score = (q_abs . c_KV + q_R . k_R) * scale with scale = 1/sqrt(d_hc + d_R)).
 *
 * Inputs
 *   q_abs       [T, H, d_cg]  dtype    from mla_absorb_q
 *   q_r         [T, H, d_R]   dtype    RoPE query, before rotation
 *   kv_cache    [num_pool_pages, page_size, d_c + d_R] dtype; row = [c_KV | k_R],
 *               k_R already rotated at its own position
 *   page_table  [batch, max_pages_per_seq] int32: logical page p of sequence b
 *               lives in physical page page_table[b][p]
 *   seq_lens    [batch] int32: keys of sequence b, including its new tokens
 *   cu_q        [batch+1] int32: sequence b owns query rows cu_q[b] .. cu_q[b+1]-1
 *   rope_cos, rope_sin  [rope_max_pos, d_R/2] float32 from mla_rope_table, or
 *               both NULL for no rotation.  Query i of sequence b sits at
 *               position seq_lens[b] - q_len_b + i (clamped into the table).
 * Outputs (caller-allocated workspace)
 *   o_part      [T, H, num_splits, d_cg] in the storage type (bfloat16 for
 *               MLA_DTYPE_BF16, float32 for MLA_DTYPE_FP32): split s's
 *               softmax-normalised output, accumulated in float32 and rounded
 *               once on the way out (a normalised average of latent rows, so it
 *               cannot exceed the cache's own range)
 *   lse_part    [T, H, num_splits] float32: split s's natural-log log-sum-exp of the
 *               scaled scores; -INFINITY for an empty split, whose o_part rows
 *               are then left unwritten (mla_combine never reads them)
 * Split plan: sequence b has n_b = ceil(seq_lens[b] / page_size) pages, cut into
 * chunks of c_b pages: c_b = pages_per_split if pages_per_split > 0, else
 * ceil(n_b / num_splits).  Split s covers pages [s*c_b, (s+1)*c_b); the last
 * split (s = num_splits - 1) runs to the end of the sequence, so no key is ever
 * dropped whatever the two numbers are.  With causal != 0 query i sees keys
 * j <= its position; otherwise all keys.  softmax_scale <= 0 selects
 * 1/sqrt(d_hc + d_R).  total_q * num_splits above 2^31 - 1 is MLA_ERR_UNSUPPORTED.
 * Work split (no effect on the results beyond rounding order): with bf16 storage, 128
 * heads, d_c 512 and d_R 64 an MFMA kernel runs one workgroup of 128 heads per
 * (token, split) -- for one latent group the 32x32x16 kernel (four waves of 32 heads),
 * for two groups the 16x16x32 kernel -- or, with one latent group and
 * 2 * total_q * num_splits at most the device's compute-unit count, two 16x16x32
 * workgroups of 64 heads each.  The environment variable MLA_KV_DECODE_KERNEL
 * overrides the choice: "generic" (the shape-generic kernel), "mfma" (automatic MFMA
 * choice), "mfma128" / "mfma64" (16x16x32 kernel with the given heads per workgroup),
 * "mfma32" (32x32x16 kernel, one latent group, heads per workgroup chosen like the
 * automatic split), "mfma32-128" / "mfma32-64" (32x32x16 kernel with the given heads per
 * workgroup); an MFMA choice the shape does not support returns MLA_ERR_UNSUPPORTED.
 */
int mla_decode_paged(const void* q_abs, const void* q_r, const void* kv_cache,
                     const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                     const float* rope_cos, const float* rope_sin, int rope_max_pos,
                     void* o_part, float* lse_part,
                     int batch, int total_q, int max_pages_per_seq, int num_pool_pages,
                     int heads, int groups, int d_hc, int d_c, int d_R, int page_size,
                     int num_splits, int pages_per_split, float softmax_scale, int causal,
                     int dtype, void* stream);

/*
 * mla_append_kv -- write the latent-cache rows of a step's new tokens into their
 * pages, the step just before mla_decode_paged reads them (P3 §1: what one token
 * stores per layer is its latent c_KV followed by its decoupled RoPE key k_R, the
 * part that carries its position; P3 §3: 64-token pages, RoPE computed in fp32;
 * P3 §4: the fp32 table applied with fp32 multiply-adds).
 *
 * Inputs
 *   c_kv_new    [T, d_c]  dtype   latent of each new token (packed rows, as the queries)
 *   k_r_new     [T, d_R]  dtype   RoPE key of each new token, before rotation
 *   page_table, seq_lens, cu_q    as in mla_decode_paged; seq_lens[b] already counts
 *               the q_len_b new tokens, so new token i of sequence b (row cu_q[b] + i)
 *               sits at pos = seq_lens[b] - q_len_b + i, the position its query is
 *               rotated at
 *   rope_cos, rope_sin  [rope_max_pos, d_R/2] float32 from mla_rope_table, or both NULL
 *               for no rotation; positions past the table use its last row (as the decode)
 * In/out
 *   kv_cache    [num_pool_pages, page_size, d_c + d_R] dtype.  Slot pos % page_size of
 *               page page_table[b][pos / page_size] becomes
 *                 [c_kv_new[t] | RoPE(k_r_new[t], pos)],
 *               the latent copied bit for bit and each key pair (x0, x1) = (k[2k], k[2k+1])
 *               rotated in fp32 as y0 = x0 cos - x1 sin, y1 = x0 sin + x1 cos with the
 *               table's (pos, k) entry, rounded once to dtype (the arithmetic the decode
 *               applies to q_R).  No other slot is touched.
 * d_c and d_R must be multiples of 8 (bf16) or 4 (fp32): MLA_ERR_UNSUPPORTED otherwise.
 * Two new tokens that map to the same slot (overlapping page tables) race; a sequence
 * with seq_lens[b] < q_len_b writes only its rows at positions >= 0.
 */
int mla_append_kv(const void* c_kv_new, const void* k_r_new, void* kv_cache,
                  const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                  const float* rope_cos, const float* rope_sin, int rope_max_pos,
                  int batch, int total_q, int max_pages_per_seq, int num_pool_pages,
                  int d_c, int d_R, int page_size, int dtype, void* stream);

/*
 * mla_combine -- merge the split partials by their log-sum-exp.  No page describes
 * splitting the keys or merging partial results; this step is the library's own
 * reading, derived from the softmax definition alone (the softmax over the union of
 * disjoint key sets, written through each set's normaliser; P2 §2.5 names softmax
 * attention):
 *   M = max_s lse[s],  w_s = exp(lse[s] - M),
 *   o_latent = sum_s w_s o_part[s] / sum_s w_s,  lse = M + log(sum_s w_s).
 * A row whose splits are all empty gets o_latent = 0 and lse = -INFINITY.
 *
 *   o_part   [T, H, num_splits, d_cg] dtype (as written by mla_decode_paged),
 *   lse_part [T, H, num_splits] float32; the merge itself runs in float32
 *   o_latent [T, H, d_cg] dtype output
 *   lse_out  [T, H] float32 output, or NULL
 */
int mla_combine(const void* o_part, const float* lse_part, void* o_latent, float* lse_out,
                int total_q, int heads, int groups, int d_c, int num_splits,
                int dtype, void* stream);

/*
 * mla_up_v -- map the latent attention output back up to the value space
 * (P2 §2.4: the latent is mapped back up to full K/V when needed; P3 §1: K/V
 * are 128 heads x 128 dims):
 *   out[t,h,d] = sum_c w_uv[h,d,c] o_latent[t,h,c], fp32 accumulation.
 *
 *   o_latent [T, H, d_cg] dtype, w_uv [H, d_hc, d_cg] dtype, out [T, H, d_hc] dtype
 */
int mla_up_v(const void* o_latent, const void* w_uv, void* out,
             int total_q, int heads, int groups, int d_hc, int d_c,
             int dtype, void* stream);

/*
 * mla_combine_up_v -- mla_combine followed by mla_up_v (same arguments, same results bit
 * for bit), in one launch where a fused kernel covers the shape: bf16, d_hc a multiple
 * of 64, d_c / groups = 512 with num_splits <= 16 or 256 with num_splits <= 32
 * (mla_combine_up_v_fused tells).  The merged rows then stay on chip.
 *
 *   o_part, lse_part  as for mla_combine;  w_uv, out  as for mla_up_v
 *   o_latent [T, H, d_cg] dtype: optional output of the merged rows.  Required (as the
 *            two calls' intermediate) for a shape the fused kernel does not cover:
 *            MLA_ERR_UNSUPPORTED if it is NULL there.
 *   lse_out  [T, H] float32 output, or NULL
 */
int mla_combine_up_v(const void* o_part, const float* lse_part, const void* w_uv, void* o_latent,
                     void* out, float* lse_out, int total_q, int heads, int groups, int d_hc,
                     int d_c, int num_splits, int dtype, void* stream);

/* 1 when mla_combine_up_v runs this shape as one fused launch, else 0 (host only, no GPU
 * call). */
int mla_combine_up_v_fused(int heads, int groups, int d_hc, int d_c, int num_splits, int dtype);

/*
 * FP8 latent cache (P3 intro and §5: a quantized gather of the latent cache whose 16-byte
 * vector loads need 16-byte-aligned pages and offsets).  The page gives no format; the
 * one here is the library's reading on gfx950's native 8-bit float (E4M3: 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits, largest finite value 448, 0x7F/0xFF NaN,
 * no infinities):
 *   one page = { codes [64][d_c] uint8 E4M3 | k_R [64][d_R] bf16 | scale [64] float32 },
 *   mla_fp8_page_bytes(d_c, d_R) = 64 * (d_c + 2 d_R + 4) bytes (41216 for 512 / 64), pages
 *   back to back, a multiple of 16 bytes each.  Token j's latent is code_i * scale_j, the
 *   scale a power of two kept in a float32 slot; its k_R stays bf16 (P3 §4: reduced RoPE
 *   precision is what breaks the absorbed scores).
 */
size_t mla_fp8_page_bytes(int d_c, int d_R);

/*
 * mla_append_kv_fp8 -- mla_append_kv into an FP8 cache: the new token's latent row x gets
 * scale = 2^e, e the smallest integer with amax <= 448 * 2^e (amax = max |x_i|), clamped
 * to [-124, 117] (e = 0 for an all-zero row), and code_i = the E4M3 value nearest to
 * x_i / scale (an exact quotient; ties to the even code, saturating at 448); k_R is rotated
 * at the token's position and rounded to bf16 exactly as mla_append_kv does.  c_kv_new [T, d_c] and k_r_new [T, d_R] are bf16.
 * d_c and d_R must be multiples of 8 and at most 512 (MLA_ERR_UNSUPPORTED otherwise);
 * other arguments and errors as mla_append_kv.
 */
int mla_append_kv_fp8(const void* c_kv_new, const void* k_r_new, void* kv_cache,
                      const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                      const float* rope_cos, const float* rope_sin, int rope_max_pos,
                      int batch, int total_q, int max_pages_per_seq, int num_pool_pages,
                      int d_c, int d_R, int page_size, void* stream);

/*
 * mla_decode_paged_fp8 -- mla_decode_paged over an FP8 cache: same arguments, results
 * and split plan, with kv_cache the FP8 pages above, q_abs, q_r and o_part bf16 (the
 * storage type is bf16; there is no dtype argument): the result of mla_decode_paged on the
 * dequantized rows [code * scale | k_R].  Each code times its token's scale is converted to
 * bf16 exactly for the MFMAs; the scales must be powers of two, as the append writes them
 * (other scales are outside the format and their results unspecified).  Implemented for 128 heads, one latent group,
 * d_c 512 and d_R 64 (MLA_ERR_UNSUPPORTED otherwise); MLA_KV_DECODE_KERNEL "mfma32-128" /
 * "mfma32-64" force one or two workgroups per (token, split).
 */
int mla_decode_paged_fp8(const void* q_abs, const void* q_r, const void* kv_cache,
                         const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                         const float* rope_cos, const float* rope_sin, int rope_max_pos,
                         void* o_part, float* lse_part,
                         int batch, int total_q, int max_pages_per_seq, int num_pool_pages,
                         int heads, int groups, int d_hc, int d_c, int d_R, int page_size,
                         int num_splits, int pages_per_split, float softmax_scale, int causal,
                         void* stream);

/*
 * MXFP4 latent cache (P3 intro and §5: the page's quantized gather is of 4-bit values, two
 * per byte, loaded 16 bytes at a time; it names NVIDIA's NVFP4 and gives no layout).  The
 * format here is the library's reading on gfx950's native 4-bit format, OCP MXFP4:
 * elements E2M1 (1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes 0,
 * 0.5, 1, 1.5, 2, 3, 4, 6; no infinity or NaN), one E8M0 scale byte s (2^(s - 127)) per
 * 32 consecutive latent elements of a token:
 *   one page = { codes [64][d_c / 2] uint8 (byte j of a row: element 2j in the low nibble,
 *   2j + 1 in the high nibble) | k_R [64][d_R] bf16 | scales [64][d_c / 32] uint8 },
 *   mla_mxfp4_page_bytes(d_c, d_R) = 64 * (d_c / 2 + 2 d_R + d_c / 32) bytes (25600 for
 *   512 / 64), 0 when d_c is not a multiple of 32.  Element value = E2M1(code) * 2^(s - 127);
 *   k_R stays bf16 as in the FP8 cache.
 */
size_t mla_mxfp4_page_bytes(int d_c, int d_R);

/*
 * mla_append_kv_mxfp4 -- mla_append_kv into an MXFP4 cache.  Each 32-element block of the
 * new token's latent row x gets the shared exponent e = floor(log2 amax) - 2 (amax = the
 * block's max |x_i|; 2 is the exponent of E2M1's largest value), clamped to [-126, 127]
 * (-126 for an all-zero block), stored as the byte e + 127 (so 1 .. 254: the decode builds
 * the scale as a normal float32); code_i = the E2M1 value nearest to x_i * 2^-e (an exact
 * product), ties to the even code, magnitudes past 6 saturating to 6, with x_i's sign.
 * k_R is rotated and rounded as mla_append_kv does.  c_kv_new [T, d_c] and k_r_new
 * [T, d_R] are bf16.  d_c must be a multiple of 32 and d_R of 8, both at most 512
 * (MLA_ERR_UNSUPPORTED otherwise); other arguments and errors as mla_append_kv.
 */
int mla_append_kv_mxfp4(const void* c_kv_new, const void* k_r_new, void* kv_cache,
                        const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                        const float* rope_cos, const float* rope_sin, int rope_max_pos,
                        int batch, int total_q, int max_pages_per_seq, int num_pool_pages,
                        int d_c, int d_R, int page_size, void* stream);

/*
 * mla_decode_paged_mxfp4 -- mla_decode_paged over an MXFP4 cache: same arguments, results,
 * split plan and shapes as mla_decode_paged_fp8, with kv_cache the MXFP4 pages above: the
 * result of mla_decode_paged on the dequantized rows.  The codes times their block's scale
 * are converted to bf16 exactly for the MFMAs (a scale byte of 0 or 255, which the append
 * never writes, is outside the format: its block reads as zero or not a number).
 */
int mla_decode_paged_mxfp4(const void* q_abs, const void* q_r, const void* kv_cache,
                           const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                           const float* rope_cos, const float* rope_sin, int rope_max_pos,
                           void* o_part, float* lse_part,
                           int batch, int total_q, int max_pages_per_seq, int num_pool_pages,
                           int heads, int groups, int d_hc, int d_c, int d_R, int page_size,
                           int num_splits, int pages_per_split, float softmax_scale, int causal,
                           void* stream);

/*
 * Prefill/decode dispatch (P3 §3: kPrefillThresh = 256, the "absorption / decompression
 * switch-over threshold"; §6: prefill takes the decompressed branch and decode the
 * absorbed one, measured there at about 12 % end-to-end over absorbing everything on one
 * configuration, and to be re-measured per machine).
 *
 * mla_branch -- host-only: MLA_BRANCH_DECOMPRESSED when the batch's largest query count
 * (q_lens, host memory) is at least threshold, else MLA_BRANCH_ABSORBED.  A batch is
 * dispatched whole; a batch that mixes prompts and decode tokens takes the branch of its
 * largest member (split it to route each part).  MLA_ERR_NULL / MLA_ERR_DIM on a NULL
 * q_lens, batch or threshold <= 0, or a negative count.
 */
#define MLA_PREFILL_THRESHOLD 256
enum mla_branch_kind { MLA_BRANCH_ABSORBED = 0, MLA_BRANCH_DECOMPRESSED = 1 };
int mla_branch(const int32_t* q_lens, int batch, int threshold);

/*
 * mla_prefill_paged -- the decompressed branch (P3 §4 path A: K and V are expanded from
 * the latent, P2 §2.4): for every cache row j of every sequence b and every head h,
 *   K[j,h,:] = W_UK[h] c_j,  V[j,h,:] = W_UV[h] c_j     (fp32 accumulation, rounded to bf16)
 * into `workspace`, then per query row t (position p = seq_lens[b] - q_len_b + i) and head
 * h the softmax over the visible keys (j <= p with causal, else all) of
 *   (q_c[t,h] . K[j,h] + RoPE(q_R[t,h], p) . k_R[j]) * scale
 * applied to V[j,h], written to out[t,h,:] (the step's output: no mla_up_v after it).
 * The same result as the four absorbed calls, up to rounding.
 *
 *   q_c [T, H, d_hc], q_r [T, H, d_R], kv_cache, page_table, seq_lens, cu_q, rope tables:
 *               as mla_decode_paged (bf16)
 *   w_uk, w_uv  [H, d_hc, d_c] bf16
 *   workspace   caller-owned, mla_prefill_workspace_bytes(num_pool_pages, H, d_hc, dtype)
 *               bytes: K then V, each [num_pool_pages * 64, H, d_hc] bf16 (row = physical
 *               cache row page * 64 + slot; only the batch's pages are written)
 *   out         [T, H, d_hc] bf16 output;  lse_out [T, H] float32 (natural log) or NULL
 *   max_q_len   at least the largest query count of the batch (rows past it are not
 *               computed)
 * Implemented for bf16, one latent group, d_hc 128, d_c 512, d_R 64, page_size 64, any head
 * count (MLA_ERR_UNSUPPORTED otherwise).  Errors as mla_decode_paged.
 */
int mla_prefill_paged(const void* q_c, const void* q_r, const void* kv_cache,
                      const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                      const float* rope_cos, const float* rope_sin, int rope_max_pos,
                      const void* w_uk, const void* w_uv, void* workspace, void* out,
                      float* lse_out, int batch, int total_q, int max_pages_per_seq,
                      int num_pool_pages, int max_q_len, int heads, int groups, int d_hc,
                      int d_c, int d_R, int page_size, float softmax_scale, int causal,
                      int dtype, void* stream);

/*
 * The two halves of mla_prefill_paged, for callers that time or schedule them apart:
 * mla_decompress_kv writes the workspace (K and V of every cache row of the batch's
 * sequences, all heads), mla_prefill_attention reads it with the queries and the cache's
 * k_R rows and writes out / lse_out.  Arguments, limits and errors as mla_prefill_paged
 * (mla_decompress_kv takes no query arguments and always enqueues its kernel).
 */
int mla_decompress_kv(const void* kv_cache, const int32_t* page_table, const int32_t* seq_lens,
                      const void* w_uk, const void* w_uv, void* workspace, int batch,
                      int max_pages_per_seq, int num_pool_pages, int heads, int groups, int d_hc,
                      int d_c, int d_R, int page_size, int dtype, void* stream);
int mla_prefill_attention(const void* q_c, const void* q_r, const void* kv_cache,
                          const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                          const float* rope_cos, const float* rope_sin, int rope_max_pos,
                          const void* workspace, void* out, float* lse_out, int batch,
                          int total_q, int max_pages_per_seq, int num_pool_pages, int max_q_len,
                          int heads, int groups, int d_hc, int d_c, int d_R, int page_size,
                          float softmax_scale, int causal, int dtype, void* stream);

/* Bytes of mla_prefill_paged's workspace (0 on bad sizes or a dtype other than bf16):
 * 2 * num_pool_pages * 64 * heads * d_hc * 2. */
size_t mla_prefill_workspace_bytes(int num_pool_pages, int heads, int d_hc, int dtype);

/* Bytes of the o_part + lse_part workspace mla_decode_paged needs for this dtype
 * (0 on bad sizes or dtype): T*H*num_splits*(d_cg*elem + 4), elem = 2 for bf16. */
size_t mla_decode_workspace_bytes(int total_q, int heads, int groups, int d_c, int num_splits,
                                  int dtype);

/*
 * mla_decode_plan -- host-only choice of the split plan (num_splits, pages_per_split) for
 * mla_decode_paged.  The pages give no split plan; this is the library's own dispatch
 * model.  It touches no GPU, allocates nothing and keeps no state.
 *
 *   seq_lens  [batch] int32, HOST memory: keys of each sequence (incl. its new tokens)
 *   q_lens    [batch] int32, HOST memory: query rows of each sequence
 *   groups    latent groups of the decode (1 = MLA)
 *   cu_count  compute units of the device the decode will run on (256 on an MI355X),
 *             at most 4096
 *   num_splits, pages_per_split  outputs
 *
 * Model: a sequence of L keys has max(1, ceil(L / 64)) pages; a split of c pages costs
 * 2.5 + c page units (0.2 when it holds no page); the grid is launched split-fastest and
 * workgroup L goes to XCD L mod 8, whose CUs (cu_count / 8 of them) each take the next
 * workgroup when free.  Candidates are the shortest split length for each split count
 * of the longest sequence (at most 256 splits) and the lengths that give k workgroups
 * per CU (k = 1 .. 16), thinned to the 64 longest plus every (n/32)-th when there are
 * more than 96.  The plan is the candidate that finishes first, ties going to the fewer
 * workgroups and then the shorter split.  With groups == 1 a plan of at most 6 pages per
 * split is doubled in length when 2 * (sum of q_lens) * (the halved split count) <=
 * cu_count, so the decode runs two 64-head workgroups per (token, split).
 * Returns MLA_ERR_NULL for a NULL pointer, MLA_ERR_DIM for batch, groups or cu_count
 * <= 0 or a negative length, MLA_ERR_UNSUPPORTED for cu_count > 4096.
 */
int mla_decode_plan(const int32_t* seq_lens, const int32_t* q_lens, int batch, int groups,
                    int cu_count, int* num_splits, int* pages_per_split);

/*
 * mla_attend_noalloc -- for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the split-KV
 * decode followed by the log-sum-exp merge, i.e. mla_decode_paged then mla_combine with
 * the same arguments, the split partials kept in library-owned static device memory
 * instead of a caller workspace.  Same kernels, so the result is bitwise that of the
 * two calls.
 *
 *   arguments as mla_decode_paged, except that o_part / lse_part are replaced by the
 *   merge's outputs
 *   o_latent  [T, H, d_cg] dtype, output (required)
 *   lse_out   [T, H] float32, output, or NULL
 *
 * Scratch: one array of MLA_NOALLOC_SCRATCH_BYTES (64 MiB) per device, held from the
 * library's first call on that device until the process ends; its address is looked up
 * once per device.  The partials of a call, T*H*num_splits*(d_cg*elem + 4) bytes (the
 * LSEs 256-byte aligned after the outputs), must fit: larger calls return
 * MLA_ERR_UNSUPPORTED before anything is enqueued (batch 16 at 16 splits of 128 heads
 * and d_c 512 takes 32.1 MiB).  Nothing in the array needs to start at zero: the decode
 * writes every split's LSE and the merge reads only the partials of splits with keys.
 * Every call on a device shares that device's array, so calls that overlap on one
 * device (different streams, or different host threads) race; calls on one stream are
 * ordered.  The call allocates and frees nothing.  Errors as mla_decode_paged, plus
 * MLA_ERR_NULL for o_latent == NULL and MLA_ERR_ALIGN for a misaligned o_latent or
 * lse_out, all detected before anything is enqueued.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
int mla_attend_noalloc(const void* q_abs, const void* q_r, const void* kv_cache,
                       const int32_t* page_table, const int32_t* seq_lens, const int32_t* cu_q,
                       const float* rope_cos, const float* rope_sin, int rope_max_pos,
                       void* o_latent, float* lse_out,
                       int batch, int total_q, int max_pages_per_seq, int num_pool_pages,
                       int heads, int groups, int d_hc, int d_c, int d_R, int page_size,
                       int num_splits, int pages_per_split, float softmax_scale, int causal,
                       int dtype, void* stream);

/* Static text for a status code (never NULL). */
const char* mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_KV_H */
