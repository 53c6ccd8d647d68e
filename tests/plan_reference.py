"""Reference transcription, in Python, of the library's host-only split planner
(``mla_decode_plan``): the tests check the C planner against it on the five workloads
and on random ragged batches, and use its dispatch model to check the plan's
properties.  Test infrastructure: the product calls the C planner only."""
import heapq
import math

PAGE_SIZE = 64


# Cost of one split in units of one page (streaming 72 KB and computing 128 heads
# over it): a fixed part for the prologue (queries fetched, first page in flight) and
# the epilogue (bf16 partial written, 128 KB), fitted at about 4 pages to the decode
# times of ragged_b64's candidate plans on MI355X, plus one unit per page.  A split with
# no keys exits at once.
SPLIT_OVERHEAD_PAGES = 4.0
EMPTY_SPLIT_PAGES = 0.2
XCDS = 8
ENGINES = 4  # shader engines per XCD


def plan_makespan(pages, q_lens, pages_per_split: int, cu_count: int = 256) -> float:
    """Finish time, in page units, of the decode grid under the cost model above.  The
    grid runs every sequence's non-empty splits first (sequence, token, split order),
    then the empty ones; the dispatcher deals workgroup L to XCD L mod 8, and each XCD
    deals its k-th workgroup to shader engine k mod 4, to the first of that engine's
    CUs to come free, never before the XCD's previous workgroup started (a workgroup
    whose engine is full holds back the ones behind it)."""
    n_splits = max(math.ceil(p / pages_per_split) for p in pages)
    per_xcd = max(1, cu_count // XCDS)
    engines = min(ENGINES, per_xcd)
    per_engine = max(1, per_xcd // engines)
    costs, empties = [], 0
    for p, n in zip(pages, q_lens):
        active = math.ceil(p / pages_per_split)
        for _ in range(n):
            costs += [SPLIT_OVERHEAD_PAGES + min(pages_per_split, p - y * pages_per_split)
                      for y in range(active)]
        empties += n * (n_splits - active)
    costs += [EMPTY_SPLIT_PAGES] * empties
    span = 0.0
    for x in range(XCDS):
        free = [[0.0] * per_engine for _ in range(engines)]
        last_start = 0.0
        for k, c in enumerate(costs[x::XCDS]):
            f = free[k % engines]
            heapq.heapify(f)
            start = max(last_start, f[0])
            heapq.heapreplace(f, start + c)
            last_start = start
        span = max([span] + [max(f) for f in free])
    return span


# Longest split (pages) for which two 64-head workgroups per (token, split) pay off: the
# half-head workgroups run a page at about 0.66 of a full page's time, so twice the
# pages cost about 1.3x; in exchange the split count halves, which halves the partial
# output the decode writes and the merge reads.  Measured on 4096-key sequences at
# batch 16 (4 pages per full-head split): 58.1 against 61.4 us per step; at 1024
# pages per sequence (64 per split) the head split loses (383 against 348 us).
HEAD_SPLIT_MAX_PAGES = 6


def head_split(total_q: int, num_splits: int, groups: int, cu_count: int = 256) -> int:
    """Workgroups per (token, split) pair of the MFMA decode kernel: 2 (64 heads each)
    for one latent group when 2 * total_q * num_splits <= cu_count, else 1 (128 heads).
    The library applies the same rule to the device's compute-unit count."""
    return 2 if groups == 1 and 2 * total_q * num_splits <= cu_count else 1


def split_plan(seq_lens_host, q_lens_host, cu_count: int = 256, groups: int = 1):
    """(num_splits, pages_per_split) for a batch: the split length whose grid finishes
    first under plan_makespan's model, among at most 256 splits per sequence.  The
    candidates are the shortest split lengths for each split count of the longest
    sequence and the lengths that give k workgroups per CU for small k; a tie goes
    to the fewer workgroups (less partial output to merge).  With one latent group, a
    plan of at most HEAD_SPLIT_MAX_PAGES pages per split is then doubled in length
    when the halved split count lets the kernel run two 64-head workgroups per
    (token, split) (head_split)."""
    pages = [max(1, math.ceil(int(L) / PAGE_SIZE)) for L in seq_lens_host]
    q = [int(x) for x in q_lens_host]
    max_p = max(pages)
    total = sum(p * n for p, n in zip(pages, q))
    cands = {math.ceil(max_p / s) for s in range(1, min(256, max_p) + 1)}
    cands |= {max(1, math.ceil(total / (cu_count * k))) for k in range(1, 17)}
    cands = sorted(c for c in cands if math.ceil(max_p / c) <= 256)
    if len(cands) > 96:  # keep the evaluation cheap: the longest splits plus a spread
        cands = sorted(set(cands[-64:]) | set(cands[:: max(1, len(cands) // 32)]))
    best = None
    for pps in cands:
        n_wg = sum(n * math.ceil(p / pps) for p, n in zip(pages, q))
        key = (plan_makespan(pages, q, pps, cu_count), n_wg)
        if best is None or key < best[0]:
            best = (key, pps)
    pps = best[1]
    S = max(1, math.ceil(max_p / pps))
    if groups == 1 and S >= 2 and pps <= HEAD_SPLIT_MAX_PAGES:
        pps2 = 2 * pps
        S2 = max(1, math.ceil(max_p / pps2))
        if head_split(sum(q), S2, groups, cu_count) == 2:
            return S2, pps2
    return S, pps
