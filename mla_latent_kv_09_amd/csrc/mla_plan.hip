// Host-only split planner of the paged decode (mla_decode_plan in include/mla_kv.h):
// picks the split length whose grid finishes first under a model of how the device
// dispatches workgroups.  Touches no GPU and allocates nothing (fixed arrays on the
// stack).
#include <stdint.h>

#include <algorithm>
#include <functional>

#include "mla_kv.h"

namespace {

// Cost of one split in units of one page (streaming 72 KB and computing 128 heads over
// it): a fixed part for the prologue (queries fetched, first page in flight) and the
// epilogue (the split's partial written), fitted at about 4 pages to the decode times of
// ragged_b64's candidate plans on MI355X, plus one unit per page.  A split with no keys
// exits at once.
constexpr double kSplitOverheadPages = 4.0;
constexpr double kEmptySplitPages = 0.2;
constexpr int kXcds = 8;
constexpr int kEngines = 4;  // shader engines per XCD
constexpr int kMaxSplits = 256;
constexpr int kMaxCusPerXcd = 512;
// Longest split (pages) for which two 64-head workgroups per (token, split) pay off: the
// half-head workgroups run a page at about 0.66 of a full page's time, so twice the
// pages cost about 1.3x, and the split count halves, which halves the partial output
// the decode writes and the merge reads.  Measured on 4096-key sequences at batch 16
// (4 pages per full-head split): 58.1 against 61.4 us per step; at 1024 pages per
// sequence (64 per split) the head split loses (383 against 348 us).
constexpr int kHeadSplitMaxPages = 6;

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

int pages_of(int32_t L) { return L <= 64 ? 1 : static_cast<int>(ceil_div(L, 64)); }

// One workgroup of the model: the XCD deals its k-th workgroup to shader engine
// k mod engines, to the engine's first CU to come free, never before the XCD's previous
// workgroup started (a workgroup whose engine is full holds back the ones behind it).
struct XcdQueue {
  double free_at[kEngines][kMaxCusPerXcd / kEngines];  // per_engine <= 512 / 4
  double last_start = 0.0;
  long long k = 0;
  void place(int engines, int per_engine, double cost) {
    double* f = free_at[k % engines];
    int c = 0;
    for (int i = 1; i < per_engine; ++i)
      if (f[i] < f[c]) c = i;
    const double start = std::max(last_start, f[c]);
    f[c] = start + cost;
    last_start = start;
    ++k;
  }
};

// Finish time, in page units, of the decode grid with splits of `pps` pages.  The grid
// runs every sequence's non-empty splits first (sequence, token, split order), then the
// empty ones; the dispatcher deals workgroup L to XCD L mod 8 (XcdQueue above).
double makespan(const int32_t* seq_lens, const int32_t* q_lens, int batch, int pps, int cu_count) {
  int n_splits = 1;
  for (int b = 0; b < batch; ++b)
    n_splits = std::max(n_splits, static_cast<int>(ceil_div(pages_of(seq_lens[b]), pps)));
  const int per_xcd = std::max(1, cu_count / kXcds);
  const int engines = std::min(kEngines, per_xcd);
  const int per_engine = std::max(1, per_xcd / engines);
  XcdQueue q[kXcds];  // 32 KB on the stack
  for (int x = 0; x < kXcds; ++x) {
    for (int e = 0; e < engines; ++e)
      for (int c = 0; c < per_engine; ++c) q[x].free_at[e][c] = 0.0;
    q[x].last_start = 0.0;
    q[x].k = 0;
  }
  long long wg = 0;
  for (int pass = 0; pass < 2; ++pass)
    for (int b = 0; b < batch; ++b) {
      const int p = pages_of(seq_lens[b]);
      const long long active = ceil_div(p, pps);
      for (int i = 0; i < q_lens[b]; ++i) {
        if (pass == 0) {
          for (long long y = 0; y < active; ++y) {
            const long long work = std::min<long long>(pps, p - y * pps);
            q[wg % kXcds].place(engines, per_engine, kSplitOverheadPages + static_cast<double>(work));
            ++wg;
          }
        } else {
          for (long long y = active; y < n_splits; ++y) {
            q[wg % kXcds].place(engines, per_engine, kEmptySplitPages);
            ++wg;
          }
        }
      }
    }
  double m = 0.0;
  for (int x = 0; x < kXcds; ++x)
    for (int e = 0; e < engines; ++e)
      for (int c = 0; c < per_engine; ++c) m = std::max(m, q[x].free_at[e][c]);
  return m;
}

}  // namespace

extern "C" int mla_decode_plan(const int32_t* seq_lens, const int32_t* q_lens, int batch,
                               int groups, int cu_count, int* num_splits, int* pages_per_split) {
  if (!seq_lens || !q_lens || !num_splits || !pages_per_split) return MLA_ERR_NULL;
  if (batch <= 0 || groups <= 0 || cu_count <= 0) return MLA_ERR_DIM;
  if (cu_count > kXcds * kMaxCusPerXcd) return MLA_ERR_UNSUPPORTED;
  long long total = 0, total_q = 0;
  int max_p = 1;
  for (int b = 0; b < batch; ++b) {
    if (seq_lens[b] < 0 || q_lens[b] < 0) return MLA_ERR_DIM;
    max_p = std::max(max_p, pages_of(seq_lens[b]));
    total += static_cast<long long>(pages_of(seq_lens[b])) * q_lens[b];
    total_q += q_lens[b];
  }
  // Candidate split lengths: the shortest length for each split count of the longest
  // sequence, and the lengths that give k workgroups per CU for k = 1 .. 16; only those
  // that need at most 256 splits.
  int cands[kMaxSplits + 16];
  int n = 0;
  for (int s = 1; s <= std::min(kMaxSplits, max_p); ++s) cands[n++] = static_cast<int>(ceil_div(max_p, s));
  for (int k = 1; k <= 16; ++k)
    cands[n++] = static_cast<int>(std::max<long long>(1, ceil_div(total, static_cast<long long>(cu_count) * k)));
  std::sort(cands, cands + n);
  n = static_cast<int>(std::unique(cands, cands + n) - cands);
  int m = 0;
  for (int i = 0; i < n; ++i)
    if (ceil_div(max_p, cands[i]) <= kMaxSplits) cands[m++] = cands[i];
  n = m;
  // Keep the evaluation cheap: the 64 longest lengths plus an even spread of the rest.
  if (n > 96) {
    int kept[kMaxSplits + 16];
    int k = 0;
    const int stride = std::max(1, n / 32);
    for (int i = 0; i < n; i += stride) kept[k++] = cands[i];
    for (int i = n - 64; i < n; ++i) kept[k++] = cands[i];
    std::sort(kept, kept + k);
    k = static_cast<int>(std::unique(kept, kept + k) - kept);
    std::copy(kept, kept + k, cands);
    n = k;
  }
  // The length with the earliest finish; a tie goes to the fewer workgroups (less
  // partial output to merge), then to the shorter split.
  double best_t = 0.0;
  long long best_wg = 0;
  int best = -1;
  for (int i = 0; i < n; ++i) {
    const int pps = cands[i];
    long long n_wg = 0;
    for (int b = 0; b < batch; ++b) n_wg += static_cast<long long>(q_lens[b]) * ceil_div(pages_of(seq_lens[b]), pps);
    const double t = makespan(seq_lens, q_lens, batch, pps, cu_count);
    if (best < 0 || t < best_t || (t == best_t && n_wg < best_wg)) {
      best = pps;
      best_t = t;
      best_wg = n_wg;
    }
  }
  int pps = best;
  int S = static_cast<int>(std::max<long long>(1, ceil_div(max_p, pps)));
  // With one latent group a short plan is doubled in length when the halved split count
  // lets the decode run two 64-head workgroups per (token, split) (2 T S <= CUs).
  if (groups == 1 && S >= 2 && pps <= kHeadSplitMaxPages) {
    const int pps2 = 2 * pps;
    const int S2 = static_cast<int>(std::max<long long>(1, ceil_div(max_p, pps2)));
    if (2 * total_q * S2 <= cu_count) {
      pps = pps2;
      S = S2;
    }
  }
  *num_splits = S;
  *pages_per_split = pps;
  return MLA_OK;
}
