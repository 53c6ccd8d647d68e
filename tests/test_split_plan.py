"""Host-side split planning and index arithmetic (CPU only).

The library's planner (``mla_decode_plan``, called through ``mla.split_plan``) is checked
against its Python transcription in ``plan_reference`` on the five workloads and on
random ragged batches, and the plan's properties (coverage, the split-count limit, one
workgroup per CU on uniform batches, optimality under the dispatch model) are checked
on the C result.  The kernels' own index code (``csrc/mla_index.h``: sequence lookup,
split key ranges, launch orders) is checked by a host program compiled from that header
under the address and undefined-behaviour sanitizers.
"""
import math
import os
import subprocess

import numpy as np
import pytest

import plan_reference as pr
from mla_latent_kv_09_amd import build_lib, mla
from mla_latent_kv_09_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


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
    pages = [math.ceil(x / pr.PAGE_SIZE) for x in L]
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
    assert pr.head_split(T, S, cfg.groups) == hs
    assert T * S * hs == 256


def test_head_split_rule():
    # one latent group: two workgroups per pair while the doubled grid fits the CUs
    assert pr.head_split(16, 8, 1) == 2
    assert pr.head_split(16, 9, 1) == 1
    assert pr.head_split(1, 128, 1) == 2 and pr.head_split(1, 129, 1) == 1
    assert pr.head_split(16, 8, 1, cu_count=128) == 1
    # two latent groups: never
    assert pr.head_split(1, 1, 2) == 1


@pytest.mark.parametrize("B,L,groups", [(16, 2048, 1), (16, 4096, 1), (32, 4096, 1), (16, 4096, 2),
                                        (4, 1000, 1), (64, 300, 1)])
def test_head_split_only_doubles_short_splits(B, L, groups):
    """The head split doubles a plan's split length only when that length is at most
    HEAD_SPLIT_MAX_PAGES and the halved split count then gets two workgroups per pair;
    otherwise the plan is the one-workgroup plan.  Either way every page is covered."""
    lens, q = [L] * B, [1] * B
    S, pps = mla.split_plan(lens, q, groups=groups)
    S1, pps1 = mla.split_plan(lens, q, groups=2)      # the plan without a head split
    pages = math.ceil(L / pr.PAGE_SIZE)
    assert S * pps >= pages and (S - 1) * pps < pages
    if groups == 2:
        assert pr.head_split(B, S, groups) == 1
    elif (S, pps) != (S1, pps1):
        assert pps == 2 * pps1 and pps1 <= pr.HEAD_SPLIT_MAX_PAGES
        assert pr.head_split(B, S, groups) == 2
    else:
        assert pps1 > pr.HEAD_SPLIT_MAX_PAGES or S1 == 1 or pr.head_split(
            B, math.ceil(pages / (2 * pps1)), groups) == 1 or pr.head_split(B, S, groups) == 2


def test_makespan_model_by_hand():
    one = pr.SPLIT_OVERHEAD_PAGES + 4
    # 8 CUs = one per XCD.  Two sequences of 8 pages, splits of 4 pages: workgroups
    # 0..3 go to XCDs 0..3 and run side by side.
    assert pr.plan_makespan([8, 8], [1, 1], 4, cu_count=8) == pytest.approx(one)
    # nine splits of one sequence: workgroup 8 is dealt to XCD 0 again and queues there
    # although the other seven XCDs are idle.
    assert pr.plan_makespan([36], [1], 4, cu_count=8) == pytest.approx(2 * one)
    # with two CUs per XCD it runs next to workgroup 0 instead
    assert pr.plan_makespan([36], [1], 4, cu_count=16) == pytest.approx(one)
    # an empty split (short sequence past its pages) costs only the early exit
    assert pr.plan_makespan([8, 1], [1, 1], 4, cu_count=8) == pytest.approx(one)
    # a query length of 2 runs the sequence's splits once per query token
    assert pr.plan_makespan([8], [2], 4, cu_count=8) == pytest.approx(one)
    assert pr.plan_makespan([4] * 9, [1] * 9, 4, cu_count=8) == pytest.approx(2 * one)


def test_makespan_model_engine_blocking_and_empty_splits_last():
    over = pr.SPLIT_OVERHEAD_PAGES
    # 64 CUs: per XCD 4 shader engines of 2 CUs.  65 one-split sequences; XCD 0 gets
    # sequences 0, 8, .., 64 and deals them to engines 0, 1, 2, 3, 0, 1, 2, 3, 0.  The
    # two on engine 0 before the last are 20 pages long, every other one 1 page: the
    # last waits for engine 0 (it may not pass to the idle engines), so the XCD ends at
    # (over + 20) + (over + 1), not at over + 20.
    pages = [20 if j in (0, 32) else 1 for j in range(65)]
    assert pr.plan_makespan(pages, [1] * 65, 20, cu_count=64) == pytest.approx(2 * over + 21)
    # Empty splits run after every non-empty one: one CU per XCD, sequence 0's eight
    # 1-page splits take XCDs 0..7, sequence 1's one page XCD 0 again, and its seven
    # empty splits (0.2 each) come last, on XCDs 1..7.
    assert pr.plan_makespan([8, 1], [1, 1], 1, cu_count=8) == pytest.approx(2 * (over + 1))


def test_ragged_plan_no_worse_than_any_candidate_length():
    L, q = _lens(wl.CONFIGS["ragged_b64"])
    pages = [math.ceil(x / pr.PAGE_SIZE) for x in L]
    S, pps = mla.split_plan(L, q)
    best = pr.plan_makespan(pages, q, pps)
    for other in (4, 8, 16, 24, 28, 32, 48, 64, 128):
        if math.ceil(max(pages) / other) <= 256:
            assert best <= pr.plan_makespan(pages, q, other) + 1e-9




@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mla.LIB_PATH):
        build_lib.build()
    return mla.load()


@pytest.mark.parametrize("name", wl.CONFIG_ORDER)
def test_c_planner_equals_reference_on_the_workloads(lib, name):
    cfg = wl.CONFIGS[name]
    L, q = _lens(cfg)
    assert mla.split_plan(L, q, groups=cfg.groups) == pr.split_plan(L, q, groups=cfg.groups)


@pytest.mark.parametrize("seed", range(40))
def test_c_planner_equals_reference_on_random_batches(lib, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 80))
    hi = int(rng.choice([64, 700, 5000, 40000, 140000]))
    L = rng.integers(0, hi + 1, size=B).tolist()
    q = rng.choice([1, 1, 2, 3], size=B).tolist()
    groups = int(rng.choice([1, 2]))
    cus = int(rng.choice([256, 256, 128, 304, 8]))
    assert mla.split_plan(L, q, cu_count=cus, groups=groups) == pr.split_plan(
        L, q, cu_count=cus, groups=groups), (L, q, cus, groups)


def test_native_index_code_under_sanitizers():
    """Build tests/native/index_check.hip (host code around csrc/mla_index.h) with
    AddressSanitizer and UBSan (host side only) and run it: launch-order bijections and
    locality, the wave-wide sequence lookup, and split key ranges that tile the visible
    keys for any split count and split length, with no signed overflow."""
    out = os.path.join(ROOT, "_build", "index_check")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    src = os.path.join(ROOT, "tests", "native", "index_check.hip")
    cmd = [build_lib.hipcc(), "-x", "hip", f"--offload-arch={build_lib.ARCH}", "-O1", "-g",
           "-std=c++17", f"-I{build_lib.CSRC}",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([out], capture_output=True, text=True, timeout=120,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all index checks passed" in r.stdout
