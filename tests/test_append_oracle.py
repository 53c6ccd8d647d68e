"""Pins for the oracle's latent-cache append: facts fixed by the pages or by mathematics.

What a cache row holds (www.nxmr.cn/news/151634 §1): the token's latent c_KV followed
by its decoupled RoPE key k_R, the part that carries the token's position; §3 fixes
64-token pages.  The pins: positions and page slots of a worked example derived by
hand, the key rotation written independently as complex multiplication, the relative
-position property the rotation exists for, untouched slots, and planted mistakes that
each of these catches.
"""
import numpy as np
import pytest

import oracle.mla_oracle as om


def _rotate_complex(x, pos, base):
    """RoPE as complex multiplication: (x0 + i x1) * exp(i pos theta_k), theta_k = base^(-2k/d)."""
    d = len(x)
    z = np.array([complex(x[2 * k], x[2 * k + 1]) for k in range(d // 2)])
    th = np.array([base ** (-2.0 * k / d) for k in range(d // 2)])
    z = z * np.exp(1j * pos * th)
    out = np.empty(d)
    out[0::2], out[1::2] = z.real, z.imag
    return out


# Worked example, derived by hand.  Four sequences with lengths 130, 64, 1, 300 and
# query lengths 2, 1, 1, 2 (seq_lens count the new tokens):
#   seq 0: new tokens at 128, 129 -> logical page 2, slots 0 and 1
#   seq 1: new token at 63        -> logical page 0, slot 63
#   seq 2: new token at 0         -> logical page 0, slot 0
#   seq 3: new tokens at 298, 299 -> logical page 4, slots 42 and 43
SEQ_LENS = np.array([130, 64, 1, 300])
CU_Q = np.array([0, 2, 3, 4, 6])
POSITIONS = [128, 129, 63, 0, 298, 299]
PAGE_TABLE = np.array([[5, 2, 7, -1, -1],
                       [1, -1, -1, -1, -1],
                       [3, -1, -1, -1, -1],
                       [9, 0, 4, 6, 8]])
SLOTS = [(7, 0), (7, 1), (1, 63), (3, 0), (8, 42), (8, 43)]  # (physical page, slot) per new token


def _example(d_c=8, d_R=4, seed=5):
    rng = np.random.default_rng(seed)
    T = len(POSITIONS)
    c_new = rng.standard_normal((T, d_c))
    k_new = rng.standard_normal((T, d_R))
    pool = np.arange(10 * 64 * (d_c + d_R), dtype=np.float64).reshape(10, 64, d_c + d_R)
    return c_new, k_new, pool


def test_positions_worked_example():
    assert om.new_token_positions(SEQ_LENS, CU_Q).tolist() == POSITIONS


def test_placement_worked_example_and_untouched_slots():
    c_new, k_new, pool = _example()
    out = om.append_to_pool(pool, PAGE_TABLE, SEQ_LENS, CU_Q, c_new, k_new, None)
    touched = np.zeros(pool.shape[:2], bool)
    for t, (page, slot) in enumerate(SLOTS):
        assert np.array_equal(out[page, slot, :8], c_new[t])
        assert np.array_equal(out[page, slot, 8:], k_new[t])  # no table: key unrotated
        touched[page, slot] = True
    assert np.array_equal(out[~touched], pool[~touched])
    assert np.array_equal(pool, np.arange(pool.size, dtype=np.float64).reshape(pool.shape))  # input kept


def test_key_rotation_is_complex_multiplication_at_own_position():
    c_new, k_new, pool = _example(d_c=8, d_R=16)
    base = 10000.0
    out = om.append_to_pool(pool, PAGE_TABLE, SEQ_LENS, CU_Q, c_new, k_new, base)
    for t, (page, slot) in enumerate(SLOTS):
        assert np.array_equal(out[page, slot, :8], c_new[t])  # latent copied bit for bit
        np.testing.assert_allclose(out[page, slot, 8:], _rotate_complex(k_new[t], POSITIONS[t], base),
                                   rtol=0, atol=1e-12)
        assert abs(np.linalg.norm(out[page, slot, 8:]) - np.linalg.norm(k_new[t])) < 1e-12


def test_appended_key_scores_depend_only_on_relative_position():
    # A query rotated at m against a key appended at n scores as the query rotated at
    # m - n against the unrotated key: what storing the key rotated is for (P3 section 1).
    rng = np.random.default_rng(9)
    d_R, base = 64, 10000.0
    k = rng.standard_normal((1, d_R))
    q = rng.standard_normal(d_R)
    for n, m in ((0, 0), (5, 17), (4095, 4095), (1000, 65535)):
        row = om.append_rows(np.zeros((1, 8)), k, [n + 1], [0, 1], base)[0, 8:]
        lhs = _rotate_complex(q, m, base) @ row
        rhs = _rotate_complex(q, m - n, base) @ k[0]
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))


def test_no_new_tokens_is_a_no_op():
    _, _, pool = _example()
    out = om.append_to_pool(pool, PAGE_TABLE, np.array([3, 4]), np.array([0, 0, 0]),
                            np.zeros((0, 8)), np.zeros((0, 4)), 10000.0)
    assert np.array_equal(out, pool)


# ---------------------------------------------------------------- pins have teeth

def _mutant(kind):
    def positions(seq_lens, cu_q):
        p = om.new_token_positions(seq_lens, cu_q)
        return p + 1 if kind == "position_off_by_one" else p

    def append(pool, page_table, seq_lens, cu_q, c_new, k_new, base):
        out = np.array(pool, np.float64, copy=True)
        pos = positions(seq_lens, cu_q)
        for b in range(len(seq_lens)):
            for t in range(int(cu_q[b]), int(cu_q[b + 1])):
                p = int(pos[t])
                if kind == "slot_from_page_index":
                    page, slot = int(page_table[b][p % 64]) if p % 64 < page_table.shape[1] else 0, p // 64
                else:
                    page, slot = int(page_table[b][p // 64]), p % 64
                key = np.asarray(k_new[t], np.float64)
                if base is not None:
                    key = om.rope_rotate(key, -p if kind == "rotation_sign" else p, base)
                if kind == "pairs_split_halves" and base is not None:
                    h = len(key) // 2
                    halves = np.empty_like(key)
                    halves[0::2], halves[1::2] = key[:h], key[h:]
                    key = om.rope_rotate(halves, p, base)
                out[page, slot] = np.concatenate([c_new[t], key])
        return out
    return append


@pytest.mark.parametrize("kind", ["position_off_by_one", "slot_from_page_index", "rotation_sign",
                                  "pairs_split_halves"])
def test_planted_mistakes_are_caught(kind):
    c_new, k_new, pool = _example(d_c=8, d_R=16)
    bad = _mutant(kind)(pool, PAGE_TABLE, SEQ_LENS, CU_Q, c_new, k_new, 10000.0)
    caught = False
    for t, (page, slot) in enumerate(SLOTS):
        want = np.concatenate([c_new[t], _rotate_complex(k_new[t], POSITIONS[t], 10000.0)])
        if not np.allclose(bad[page, slot], want, rtol=0, atol=1e-9):
            caught = True
    assert caught
