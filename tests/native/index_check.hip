// CPU check of the paged decode's integer index code (mla_index.h, the header the
// kernels include), built for the host under the address and undefined-behaviour
// sanitizers.  For random batches it checks:
//  - the wave-wide sequence lookup equals the binary search over cu_q;
//  - each launch-order map is a bijection from workgroup ids onto
//    (query token, split[, head half]) and keeps its locality promise (the tokens of a
//    split 8 workgroups apart, the halves of a pair on one XCD, a token's workgroups on
//    XCD t mod 8); the active-first order puts every non-empty split before every empty
//    one, and its count of non-empty splits agrees with split_work;
//  - split_work's key ranges tile the visible keys of every query exactly, for any
//    split count and split length up to INT32_MAX, without signed overflow.
// Prints one line per section and exits non-zero on the first failure.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <climits>
#include <random>
#include <vector>

#include "mla_index.h"

using mla::Unit;

static int failures = 0;
#define CHECK(cond, ...)                                 \
  do {                                                   \
    if (!(cond)) {                                       \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                      \
      fprintf(stderr, "\n");                             \
      if (++failures > 20) exit(1);                      \
    }                                                    \
  } while (0)

static std::vector<int32_t> make_cu(std::mt19937& g, int B, bool allow_empty, int max_q) {
  std::vector<int32_t> cu(B + 1, 0);
  std::uniform_int_distribution<int> q(allow_empty ? 0 : 1, max_q);
  for (int b = 0; b < B; ++b) cu[b + 1] = cu[b] + q(g);
  if (cu[B] == 0) {  // at least one query row
    cu[B] = 1;
  }
  return cu;
}

static void check_lookup(std::mt19937& g) {
  int n = 0;
  for (int it = 0; it < 400; ++it) {
    const int B = 1 + static_cast<int>(g() % 64);
    const std::vector<int32_t> cu = make_cu(g, B, true, 3);
    for (int t = 0; t < cu[B]; ++t, ++n) {
      const int b = mla::find_seq(cu.data(), B, t);
      CHECK(b >= 0 && b < B && cu[b] <= t && t < cu[b + 1], "find_seq B=%d t=%d -> %d", B, t, b);
      CHECK(mla::find_seq_count(cu.data(), B, t) == b, "wave lookup B=%d t=%d", B, t);
    }
  }
  printf("lookup: %d rows ok\n", n);
}

static void check_m32(std::mt19937& g) {
  int n = 0;
  for (int it = 0; it < 600; ++it) {
    const int B = 1 + static_cast<int>(g() % 12);
    const int S = 1 + static_cast<int>(g() % 40);
    const std::vector<int32_t> cu = make_cu(g, B, true, 3);
    const int T = cu[B];
    std::vector<int> where(static_cast<size_t>(T) * S, -1);
    for (int L = 0; L < T * S; ++L, ++n) {
      const int b = mla::find_seq(cu.data(), B, L / S);
      const Unit u = mla::unit_m32(L, S, cu[b], cu[b + 1] - cu[b], T);
      CHECK(u.t >= 0 && u.t < T && u.split >= 0 && u.split < S, "m32 range L=%d", L);
      if (u.t < 0 || u.t >= T || u.split < 0 || u.split >= S) continue;
      int& w = where[static_cast<size_t>(u.t) * S + u.split];
      CHECK(w < 0, "m32 (t=%d, s=%d) hit twice", u.t, u.split);
      w = L;
    }
    for (int b = 0; b < B; ++b) {
      const int q0 = cu[b], nq = cu[b + 1] - cu[b];
      for (int s = 0; s < S; ++s) {
        if (nq == 1) {
          CHECK(where[static_cast<size_t>(q0) * S + s] == q0 * S + s, "m32 split order");
        } else if (nq > 1 && s < 8 * (S / 8)) {
          for (int i = 0; i < nq; ++i)
            CHECK(where[static_cast<size_t>(q0 + i) * S + s] - where[static_cast<size_t>(q0) * S + s] == 8 * i,
                  "m32 tokens of a split 8 apart");
        }
      }
    }
  }
  printf("m32 launch order: %d workgroups ok\n", n);
}

static void check_active_first(std::mt19937& g) {
  long long n = 0;
  for (int it = 0; it < 500; ++it) {
    const int B = 1 + static_cast<int>(g() % 150);
    const int S = 1 + static_cast<int>(g() % 40);
    const int page = 64;
    const std::vector<int32_t> cu = make_cu(g, B, true, 3);
    const int T = cu[B];
    std::vector<int32_t> lens(B);
    for (int b = 0; b < B; ++b) lens[b] = static_cast<int32_t>(g() % 6000) - (g() % 20 == 0 ? 10 : 0);
    const int max_pages = 1 + static_cast<int>(g() % 100);
    const int pps = g() % 3 == 0 ? 0 : 1 + static_cast<int>(g() % 40);
    std::vector<int> where(static_cast<size_t>(T) * S, -1);
    int last_active = -1, first_empty = T * S;
    for (int L = 0; L < T * S; ++L, ++n) {
      const Unit u = mla::unit_active_first(L, S, pps, page, max_pages, cu.data(), lens.data(), B);
      const bool ok = u.t >= 0 && u.t < T && u.split >= 0 && u.split < S;
      CHECK(ok, "active-first range L=%d", L);
      if (!ok) continue;
      int& w = where[static_cast<size_t>(u.t) * S + u.split];
      CHECK(w < 0, "active-first (t=%d, s=%d) hit twice", u.t, u.split);
      w = L;
      const int b = mla::find_seq(cu.data(), B, u.t);
      const int a = mla::active_splits(lens[b], S, pps, page, max_pages);
      if (u.split < a) last_active = L; else if (L < first_empty) first_empty = L;
      // active_splits agrees with split_work for the sequence's last row
      const int nq = cu[b + 1] - cu[b];
      const mla::QueryWork wk = mla::split_work(b, cu[b], nq, lens[b], cu[b + 1] - 1, u.split, S, pps, page,
                                                max_pages, 1);
      CHECK((wk.k0 < wk.k1) == (u.split < a), "active_splits vs split_work (L=%d s=%d a=%d)", lens[b], u.split, a);
    }
    CHECK(last_active < first_empty, "an empty unit before an active one");
    for (int b = 0; b < B; ++b) {
      const int q0 = cu[b], nq = cu[b + 1] - cu[b];
      const int a = mla::active_splits(lens[b], S, pps, page, max_pages);
      for (int s = 1; s < a && nq == 1; ++s)
        CHECK(where[static_cast<size_t>(q0) * S + s] == where[static_cast<size_t>(q0) * S + s - 1] + 1,
              "active splits of a one-token sequence in order");
      for (int s = 0; s < 8 * (a / 8) && nq > 1; ++s)
        for (int i = 1; i < nq; ++i)
          CHECK(where[static_cast<size_t>(q0 + i) * S + s] - where[static_cast<size_t>(q0) * S + s] == 8 * i,
                "tokens of an active split 8 apart");
    }
  }
  printf("active-first launch order: %lld workgroups ok\n", n);
}

static void check_halves(std::mt19937& g, bool mfma_form) {
  int n = 0;
  for (int it = 0; it < 400; ++it) {
    const int T = 1 + static_cast<int>(g() % 48);
    const int S = 1 + static_cast<int>(g() % 12);
    std::vector<int> where(static_cast<size_t>(2) * T * S, -1);
    for (int L = 0; L < 2 * T * S; ++L, ++n) {
      const Unit u = mfma_form ? mla::unit_mfma_half(L, S, T) : mla::unit_pair_blocks(L, S, T);
      const bool ok = u.t >= 0 && u.t < T && u.split >= 0 && u.split < S && (u.half == 0 || u.half == 1);
      CHECK(ok, "half map range L=%d T=%d S=%d", L, T, S);
      if (!ok) continue;
      int& w = where[(static_cast<size_t>(u.t) * S + u.split) * 2 + u.half];
      CHECK(w < 0, "half map hit twice");
      w = L;
    }
    for (int t = 0; t < T; ++t)
      for (int s = 0; s < S; ++s) {
        const int w0 = where[(static_cast<size_t>(t) * S + s) * 2], w1 = where[(static_cast<size_t>(t) * S + s) * 2 + 1];
        const bool full_block = (t * S + s) < 8 * (T * S / 8);
        if ((mfma_form && T % 8 == 0) || full_block) CHECK(w0 % 8 == w1 % 8, "halves on one XCD");
        if (mfma_form && T % 8 == 0) CHECK(w0 % 8 == t % 8, "token on XCD t mod 8");
      }
  }
  printf("%s: %d workgroups ok\n", mfma_form ? "16x16x32 head-split order" : "pair-block order", n);
}

static void check_splits(std::mt19937& g) {
  long long n = 0;
  const int pps_big[] = {INT_MAX, INT_MAX - 1, 1 << 30, 33554432, 33554433};
  for (int it = 0; it < 3000; ++it) {
    const int page = 64;
    const int L = static_cast<int>(g() % 200000);
    const int max_pages = (L + page - 1) / page + static_cast<int>(g() % 3);
    if (max_pages == 0) continue;
    const int q_len = 1 + static_cast<int>(g() % 3);
    const int S = 1 + static_cast<int>(g() % 256);
    int pps;
    switch (g() % 4) {
      case 0: pps = 0; break;
      case 1: pps = 1 + static_cast<int>(g() % 100); break;
      case 2: pps = pps_big[g() % 5]; break;
      default: pps = 1 + static_cast<int>(g() % (max_pages + 1)); break;
    }
    const int causal = static_cast<int>(g() % 2);
    for (int i = 0; i < q_len; ++i) {
      int next = 0, n_vis = -1;
      for (int s = 0; s < S; ++s, ++n) {
        const mla::QueryWork w = mla::split_work(0, 0, q_len, L, i, s, S, pps, page, max_pages, causal);
        if (n_vis < 0) n_vis = causal ? (w.pos + 1 < w.L ? (w.pos + 1 > 0 ? w.pos + 1 : 0) : w.L) : w.L;
        CHECK(w.k0 <= w.k1, "k0 > k1 (L=%d S=%d pps=%d s=%d)", L, S, pps, s);
        if (w.k0 < w.k1) {
          CHECK(w.k0 == next, "gap or overlap at split %d (L=%d S=%d pps=%d): k0=%d want %d", s, L, S, pps,
                w.k0, next);
          next = w.k1;
        }
        CHECK(w.k1 <= n_vis, "split past the visible keys");
        if (s < S - 1 && w.k0 < w.k1) {
          const long long per = pps > 0 ? pps : ((L + page - 1) / page + S - 1) / S;
          CHECK(w.k0 % page == 0 && static_cast<long long>(w.k0) == static_cast<long long>(s) * per * page,
                "split start not on its page boundary");
        }
      }
      CHECK(next == n_vis, "keys not covered (L=%d S=%d pps=%d): %d of %d", L, S, pps, next, n_vis);
    }
  }
  printf("split_work: %lld key ranges ok\n", n);
}

// The XCD-grouped logical order: a bijection of [0, G), and each XCD's logical indices
// form one consecutive range taken in that XCD's dispatch order.
static void check_xcd(std::mt19937& g) {
  long long n = 0;
  for (int k = 0; k < 400; ++k) {
    const int G = k < 200 ? 1 + k : 1 + static_cast<int>(g() % 100000);
    std::vector<int> seen(G, -1);
    std::vector<int> last(8, -1);
    for (int j = 0; j < G; ++j, ++n) {
      const int L = mla::xcd_grouped(j, G);
      CHECK(L >= 0 && L < G, "xcd_grouped range G=%d j=%d -> %d", G, j, L);
      if (L < 0 || L >= G) continue;
      CHECK(seen[L] < 0, "xcd_grouped G=%d: logical %d hit twice", G, L);
      seen[L] = j;
      const int x = j & 7;
      CHECK(last[x] < 0 || L == last[x] + 1, "xcd_grouped G=%d: XCD %d not consecutive", G, x);
      last[x] = L;
    }
  }
  printf("xcd_grouped: %lld indices ok\n", n);
}

int main() {
  std::mt19937 g(20261203);
  check_lookup(g);
  check_m32(g);
  check_active_first(g);
  check_halves(g, false);
  check_halves(g, true);
  check_splits(g);
  check_xcd(g);
  if (failures) {
    printf("%d failures\n", failures);
    return 1;
  }
  printf("all index checks passed\n");
  return 0;
}
