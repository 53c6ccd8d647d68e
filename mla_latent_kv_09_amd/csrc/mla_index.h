// Integer index arithmetic of the paged decode, callable from host and device: the
// sequence that owns a packed query row, the key range of a split, and the maps from
// a workgroup id to the (query token, split, head half) it works on.  The kernels
// include this header; a host program compiled from the same header checks every map
// on the CPU (bijection, coverage, no overflow) under the address and
// undefined-behaviour sanitizers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// Sequence owning packed query row t: the largest b with cu_q[b] <= t.
__host__ __device__ inline int find_seq(const int32_t* __restrict__ cu_q, int batch, int t) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// The same lookup as the decode kernels' wave-wide form does it for batch <= 64 (lane l
// holds cu_q[l + 1]; the answer is the number of lanes l < batch - 1 with
// cu_q[l + 1] <= t), written as a loop over the lanes.
__host__ __device__ inline int find_seq_count(const int32_t* __restrict__ cu_q, int batch, int t) {
  int n = 0;
  for (int l = 0; l < 64; ++l)
    if (l < batch - 1 && cu_q[l + 1] <= t) ++n;
  return n;
}

// Where query row t sits and which keys split s of its sequence covers.
struct QueryWork {
  int b;       // sequence
  int L;       // keys of the sequence (clamped to the page-table capacity)
  int pos;     // absolute position of the query
  int k0, k1;  // key range [k0, k1) of this split, already clipped to the visible keys
};

// The key range of split `split` for query row t of sequence b, which starts at query
// row q0, has q_len query rows and L_raw keys.  Sequence b has n = ceil(L / page_size)
// pages cut into chunks of c pages (c = pages_per_split if > 0, else ceil(n / S)); split
// s covers pages [s c, (s + 1) c) and the last split runs to the end.
__host__ __device__ inline QueryWork split_work(int b, int q0, int q_len, int L_raw, int t,
                                                int split, int num_splits, int pages_per_split,
                                                int page_size, int max_pages, int causal) {
  QueryWork w;
  w.b = b;
  const long long cap = static_cast<long long>(max_pages) * page_size;
  const int L = L_raw < 0 ? 0 : (L_raw > cap ? static_cast<int>(cap) : L_raw);
  w.L = L;
  w.pos = L - q_len + (t - q0);
  int n_vis = causal ? (w.pos + 1 < L ? w.pos + 1 : L) : L;
  if (n_vis < 0) n_vis = 0;
  const int n_pages = (L + page_size - 1) / page_size;
  const int per_split = pages_per_split > 0 ? pages_per_split
                                            : (n_pages + num_splits - 1) / num_splits;
  // Key bounds in 64 bits: split * per_split * page_size can pass 2^31 for a long split
  // length, and every bound is then clipped to the visible keys.
  const long long step = static_cast<long long>(per_split) * page_size;
  const long long k0 = static_cast<long long>(split) * step;
  const long long k1 = split == num_splits - 1 ? n_vis : k0 + step;
  w.k0 = static_cast<int>(k0 < n_vis ? k0 : n_vis);
  w.k1 = static_cast<int>(k1 < n_vis ? k1 : n_vis);
  return w;
}

// What one workgroup of a decode launch works on.
struct Unit {
  int t;      // packed query row
  int split;  // split of its sequence
  int half;   // head half (0 or 1) when two workgroups share a (token, split) pair
};

// One workgroup per (token, split), split-fastest: workgroup L = t * S + split.
__host__ __device__ inline Unit unit_split_fastest(int L, int S) {
  Unit u;
  u.t = L / S;
  u.split = L - u.t * S;
  u.half = 0;
  return u;
}

// Two workgroups per (token, split), blocks of 8 pairs taking 16 consecutive
// workgroups: half h of pair 8k + i is workgroup 16k + 8h + i (in a last block of
// r < 8 pairs, 16k + r h + i).  The dispatcher deals workgroup L to XCD L mod 8, so the
// two halves of a pair in a full block share one XCD's L2.  Pairs are split-fastest.
__host__ __device__ inline Unit unit_pair_blocks(int L, int S, int T) {
  const int kb = L >> 4, base = kb * 8;
  const int r = (T * S - base) < 8 ? (T * S - base) : 8, off = L - 16 * kb;
  const int pair = base + off % r;
  Unit u;
  u.half = off / r;
  u.t = pair / S;
  u.split = pair - u.t * S;
  return u;
}

// Two workgroups per (token, split) of the 16x16x32 kernel: with T a multiple of 8 the
// 2 S workgroups of token t all go to XCD t mod 8 (workgroup L: XCD slot x = L mod 8,
// r = L / 8; token x + 8 (r / 2S), split (r mod 2S) / 2, half r mod 2), the two halves
// of a pair adjacent in that XCD's order; otherwise the pair blocks above.
__host__ __device__ inline Unit unit_mfma_half(int L, int S, int T) {
  if (T % 8 != 0) return unit_pair_blocks(L, S, T);
  const int x = L & 7, r = L >> 3;
  const int k = r / (2 * S), rem = r - k * 2 * S;
  Unit u;
  u.t = x + 8 * k;
  u.split = rem >> 1;
  u.half = rem & 1;
  return u;
}

// Non-empty splits of a sequence for its last query row, which sees every key: the
// splits s < num_splits with s * c * page_size < L (c and the clamp of L as in
// split_work).  Earlier rows of a causal multi-token sequence may find the last of them
// empty.
__host__ __device__ inline int active_splits(int L_raw, int num_splits, int pages_per_split,
                                             int page_size, int max_pages) {
  const long long cap = static_cast<long long>(max_pages) * page_size;
  const long long L = L_raw < 0 ? 0 : (L_raw > cap ? cap : L_raw);
  if (L == 0 || num_splits <= 0) return 0;
  const long long n_pages = (L + page_size - 1) / page_size;
  const long long per = pages_per_split > 0 ? pages_per_split : (n_pages + num_splits - 1) / num_splits;
  const long long step = per * page_size;
  const long long s = (L + step - 1) / step;
  return s < num_splits ? static_cast<int>(s) : num_splits;
}

// Unit v of the nq x cnt units (q0 + i, s_lo + j), i < nq, j < cnt: with one token in
// split order; with nq tokens, which read the same pages, blocks of 8 splits taking 8 nq
// consecutive units token-major, so the nq units of one split are 8 apart (one XCD,
// about the same time, when the block starts at a multiple of 8).
__host__ __device__ inline Unit unit_in_sequence(int v, int q0, int nq, int s_lo, int cnt) {
  Unit u;
  u.half = 0;
  if (nq <= 1) {
    u.t = q0;
    u.split = s_lo + v;
    return u;
  }
  const int blk = v / (8 * nq), r = v - blk * 8 * nq;
  const int k = (cnt - 8 * blk) < 8 ? (cnt - 8 * blk) : 8;
  u.t = q0 + r / k;
  u.split = s_lo + 8 * blk + (r - (r / k) * k);
  return u;
}

// Active-first launch order of the 32x32x16 kernel: first every sequence's non-empty
// splits (sequence order, unit_in_sequence within one), then every empty one.  The
// dispatcher deals the workgroups of an XCD round-robin to its shader engines and waits
// while the next one's engine is full, so short empty workgroups scattered through the
// order leave compute units idle until a long workgroup of that engine ends; at the end
// they cost nothing.  Reference form over the arrays (the kernel computes the same map
// with a wave-wide prefix sum).
__host__ __device__ inline Unit unit_active_first(int L, int S, int pages_per_split, int page_size,
                                                  int max_pages, const int32_t* cu_q,
                                                  const int32_t* seq_lens, int batch) {
  int base = 0;
  for (int pass = 0; pass < 2; ++pass)
    for (int b = 0; b < batch; ++b) {
      const int q0 = cu_q[b], nq = cu_q[b + 1] - cu_q[b];
      const int a = active_splits(seq_lens[b], S, pages_per_split, page_size, max_pages);
      const int lo = pass == 0 ? 0 : a, cnt = pass == 0 ? a : S - a;
      if (L < base + nq * cnt) return unit_in_sequence(L - base, q0, nq, lo, cnt);
      base += nq * cnt;
    }
  return unit_split_fastest(L, S);
}

// One workgroup per (token, split) of the 32x32x16 kernel.  The units of sequence b (its
// nq query tokens x S splits, first token q0) are the workgroups [q0 S, (q0 + nq) S).
// With one token they run in split order.  With nq tokens, which read the same pages,
// each block of 8 splits takes 8 nq consecutive workgroups, token-major: the nq
// workgroups of one split are 8 apart, so they land on one XCD at about the same time
// and its L2 serves the later reads of each page.  Workgroup L must belong to the
// sequence (q0 <= L / S < q0 + nq); a malformed cu_q that maps outside [0, T) x [0, S)
// falls back to split order.
__host__ __device__ inline Unit unit_m32(int L, int S, int q0, int nq, int T) {
  Unit u;
  u.half = 0;
  const int v = L - q0 * S;
  if (nq <= 1) {
    u.t = q0 + v / S;
    u.split = v - (v / S) * S;
  } else {
    const int blk = v / (8 * nq), r = v - blk * 8 * nq;
    const int k = (S - 8 * blk) < 8 ? (S - 8 * blk) : 8;
    if (k <= 0) {
      u.t = -1;
      u.split = -1;
    } else {
      u.t = q0 + r / k;
      u.split = 8 * blk + (r - (r / k) * k);
    }
  }
  if (u.t < 0 || u.t >= T || u.split < 0 || u.split >= S) u = unit_split_fastest(L, S);
  return u;
}

// Logical index of workgroup j in a grid of G that numbers each XCD's workgroups
// consecutively.  The dispatcher deals workgroup j to XCD j mod 8, so XCD x receives
// G / 8 workgroups, plus one if x < G mod 8.  It takes logical indices base_x, base_x + 1,
// ... in its dispatch order, with base_x = x (G / 8) + min(x, G mod 8).  A bijection of
// [0, G).
__host__ __device__ inline int xcd_grouped(int j, int G) {
  const int x = j & 7, per = G >> 3, extra = G & 7;
  return x * per + (x < extra ? x : extra) + (j >> 3);
}

}  // namespace mla
