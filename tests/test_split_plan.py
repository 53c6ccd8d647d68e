"""Host-side split planning (CPU only): coverage, the split-count limit, one workgroup
per CU on uniform batches, and the dispatch model it optimises."""
import math

import numpy as np
import pytest

from mla_latent_kv_09_amd import mla
from mla_latent_kv_09_amd import workloads as wl


def _lens(cfg):
    if cfg.seq_len_range is not None:
        lo, hi = cfg.seq_len_range
        L = wl._rng(cfg.seed, "lengths").integers(lo, hi + 1, size=cfg.batch)
    else:
        L = np.full(cfg.batch, cfg.seq_len)
    q = np.full(cfg.batch, cfg.q_len)
    if cfg.q_len_mix:
        q = np.ones(cfg.batch, dtype=np.int64)
        q[wl._rng(cfg.seed, "q_lens").permutation(cfg.batch)[: cfg.batch // 2]] = 2
    return [int(x) for x in L], [int(x) for x in q]


@pytest.mark.parametrize("name", ["dsv3_b16_l4096", "long_b16_l65536", "ragged_b64",
                                  "gla2_b32_l16384"])
def test_plan_covers_every_page_within_the_split_limit(name):
    L, q = _lens(wl.CONFIGS[name])
    S, pps = mla.split_plan(L, q)
    pages = [math.ceil(x / mla.PAGE_SIZE) for x in L]
    assert 1 <= S <= 256 and pps >= 1
    assert S * pps >= max(pages)               # the last split never has to take extra pages
    assert (S - 1) * pps < max(pages)          # and no split is empty for the longest sequence


@pytest.mark.parametrize("name,expect,hs", [("dsv3_b16_l4096", (8, 8), 2),
                                            ("long_b16_l65536", (16, 64), 1),
                                            ("gla2_b32_l16384", (8, 32), 1)])
def test_uniform_batches_get_one_workgroup_per_cu(name, expect, hs):
    """16 x 4096 keys: 16 splits of 4 pages would fill the 256 CUs, and that short a
    split is doubled so two 64-head workgroups per (token, split) fill them instead."""
    cfg = wl.CONFIGS[name]
    L, q = _lens(cfg)
    S, pps = mla.split_plan(L, q, groups=cfg.groups)
    assert (S, pps) == expect
    T = sum(q)
    assert mla.head_split(T, S, cfg.groups) == hs
    assert T * S * hs == 256


def test_head_split_rule():
    # one latent group: two workgroups per pair while the doubled grid fits the CUs
    assert mla.head_split(16, 8, 1) == 2
    assert mla.head_split(16, 9, 1) == 1
    assert mla.head_split(1, 128, 1) == 2 and mla.head_split(1, 129, 1) == 1
    assert mla.head_split(16, 8, 1, cu_count=128) == 1
    # two latent groups: never
    assert mla.head_split(1, 1, 2) == 1


@pytest.mark.parametrize("B,L,groups", [(16, 2048, 1), (16, 4096, 1), (32, 4096, 1), (16, 4096, 2),
                                        (4, 1000, 1), (64, 300, 1)])
def test_head_split_only_doubles_short_splits(B, L, groups):
    """The head split doubles a plan's split length only when that length is at most
    HEAD_SPLIT_MAX_PAGES and the halved split count then gets two workgroups per pair;
    otherwise the plan is the one-workgroup plan.  Either way every page is covered."""
    lens, q = [L] * B, [1] * B
    S, pps = mla.split_plan(lens, q, groups=groups)
    S1, pps1 = mla.split_plan(lens, q, groups=2)      # the plan without a head split
    pages = math.ceil(L / mla.PAGE_SIZE)
    assert S * pps >= pages and (S - 1) * pps < pages
    if groups == 2:
        assert mla.head_split(B, S, groups) == 1
    elif (S, pps) != (S1, pps1):
        assert pps == 2 * pps1 and pps1 <= mla.HEAD_SPLIT_MAX_PAGES
        assert mla.head_split(B, S, groups) == 2
    else:
        assert pps1 > mla.HEAD_SPLIT_MAX_PAGES or S1 == 1 or mla.head_split(
            B, math.ceil(pages / (2 * pps1)), groups) == 1 or mla.head_split(B, S, groups) == 2


def test_makespan_model_by_hand():
    one = mla.SPLIT_OVERHEAD_PAGES + 4
    # 8 CUs = one per XCD.  Two sequences of 8 pages, splits of 4 pages: workgroups
    # 0..3 go to XCDs 0..3 and run side by side.
    assert mla.plan_makespan([8, 8], [1, 1], 4, cu_count=8) == pytest.approx(one)
    # nine splits of one sequence: workgroup 8 is dealt to XCD 0 again and queues there
    # although the other seven XCDs are idle.
    assert mla.plan_makespan([36], [1], 4, cu_count=8) == pytest.approx(2 * one)
    # with two CUs per XCD it runs next to workgroup 0 instead
    assert mla.plan_makespan([36], [1], 4, cu_count=16) == pytest.approx(one)
    # an empty split (short sequence past its pages) costs only the early exit
    assert mla.plan_makespan([8, 1], [1, 1], 4, cu_count=8) == pytest.approx(one)
    # a query length of 2 runs the sequence's splits once per query token
    assert mla.plan_makespan([8], [2], 4, cu_count=8) == pytest.approx(one)
    assert mla.plan_makespan([4] * 9, [1] * 9, 4, cu_count=8) == pytest.approx(2 * one)


def test_ragged_plan_no_worse_than_any_candidate_length():
    L, q = _lens(wl.CONFIGS["ragged_b64"])
    pages = [math.ceil(x / mla.PAGE_SIZE) for x in L]
    S, pps = mla.split_plan(L, q)
    best = mla.plan_makespan(pages, q, pps)
    for other in (4, 8, 16, 24, 28, 32, 48, 64, 128):
        if math.ceil(max(pages) / other) <= 256:
            assert best <= mla.plan_makespan(pages, q, other) + 1e-9


def _launch_unit(L, S, cu_q):
    """The 32x32x16 decode kernel's launch order (one workgroup per (token, split)),
    written out: the units of sequence b are workgroups [cu_q[b] S, cu_q[b+1] S); one
    token runs in split order, n tokens in blocks of 8 splits x n tokens, token-major."""
    t0 = L // S
    b = max(i for i in range(len(cu_q) - 1) if cu_q[i] <= t0)
    q0, n = cu_q[b], cu_q[b + 1] - cu_q[b]
    u = L - q0 * S
    if n <= 1:
        return q0 + u // S, u % S
    blk, r = divmod(u, 8 * n)
    k = min(8, S - 8 * blk)
    return q0 + r // k, 8 * blk + r % k


@pytest.mark.parametrize("seed", range(20))
def test_launch_order_is_a_bijection_that_groups_tokens_of_a_split(seed):
    rng = np.random.default_rng(seed)
    B, S = int(rng.integers(1, 10)), int(rng.integers(1, 40))
    q_lens = rng.choice([1, 1, 2, 3], size=B)
    cu = np.concatenate([[0], np.cumsum(q_lens)]).tolist()
    T = cu[-1]
    where = {}
    for L in range(T * S):
        t, s = _launch_unit(L, S, cu)
        assert 0 <= t < T and 0 <= s < S and (t, s) not in where
        where[(t, s)] = L
    assert len(where) == T * S
    for b in range(B):
        q0, n = cu[b], cu[b + 1] - cu[b]
        for s in range(S):
            if n == 1:
                assert where[(q0, s)] == q0 * S + s          # split order, as before
            elif s < 8 * (S // 8):                           # full blocks: 8 apart, one XCD
                assert all(where[(q0 + i, s)] - where[(q0, s)] == 8 * i for i in range(n))


def _find_seq_binary(cu_q, batch, t):
    lo, hi = 0, batch - 1
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if cu_q[mid] <= t:
            lo = mid
        else:
            hi = mid - 1
    return lo


def _find_seq_wave(cu_q, batch, t):
    """The decode kernels' wave-wide lookup for batch <= 64: lane l holds cu_q[l + 1];
    the sequence is the number of lanes l < batch - 1 with cu_q[l + 1] <= t."""
    return sum(1 for lane in range(64) if lane < batch - 1 and cu_q[lane + 1] <= t)


@pytest.mark.parametrize("seed", range(40))
def test_wave_sequence_lookup_matches_binary_search(seed):
    rng = np.random.default_rng(seed)
    batch = int(rng.choice([1, 2, 3, 16, 63, 64]))
    q_lens = rng.choice([0, 1, 1, 2, 3], size=batch)
    q_lens[int(rng.integers(batch))] = max(1, q_lens[0])
    cu = np.concatenate([[0], np.cumsum(q_lens)]).tolist()
    for t in range(cu[-1]):
        b = _find_seq_wave(cu, batch, t)
        assert b == _find_seq_binary(cu, batch, t)
        assert cu[b] <= t < cu[b + 1]  # the row belongs to a non-empty sequence


def _k2_half_unit(L, S, T):
    """The 16x16x32 decode kernel's launch order with two workgroups per (token, split),
    written out: (token, split, half) of workgroup L."""
    if T % 8 == 0:
        x, r = L & 7, L >> 3
        k, rem = divmod(r, 2 * S)
        return x + 8 * k, rem >> 1, rem & 1
    kb = L >> 4
    base = kb * 8
    r = min(8, T * S - base)
    off = L - 16 * kb
    pair = base + off % r
    return pair // S, pair % S, off // r


@pytest.mark.parametrize("T", [1, 3, 8, 16, 24, 40])
@pytest.mark.parametrize("S", [1, 2, 5, 8])
def test_head_split_launch_order_is_a_bijection_with_halves_on_one_xcd(T, S):
    where = {}
    for L in range(2 * T * S):
        t, s, h = _k2_half_unit(L, S, T)
        assert 0 <= t < T and 0 <= s < S and h in (0, 1) and (t, s, h) not in where
        where[(t, s, h)] = L
    assert len(where) == 2 * T * S
    for t in range(T):
        for s in range(S):
            full_block = (t * S + s) < 8 * (T * S // 8)
            if T % 8 == 0 or full_block:                       # halves share an L2
                assert where[(t, s, 0)] % 8 == where[(t, s, 1)] % 8
            if T % 8 == 0:                                     # a token's units share one
                assert where[(t, s, 0)] % 8 == t % 8
