"""Pins for the split-KV oracle (oracle/splitkv.py): the partial results over key ranges, their
logsumexp merge, and the pages' num_splits rule.

What pins what:
  * merging the partials of any partition of the keys reproduces the plain definition
    (oracle/attention.py, a separate code path that never splits), for partitions with empty
    ranges, ragged ends, causal rows whose range lies past the diagonal, and every order;
  * closed forms: a one-key range gives O_s = V_j and L_s = S_ij; a range of keys the causal
    mask hides gives O_s = 0, L_s = -inf; two equal partials merge to the same O and L + ln 2;
  * no overflow for L_s near 1000 (a merge without the max shift returns inf or NaN there);
  * the heuristic on cases worked out by hand below, and its defining property;
  * split_ranges covers every block exactly once, in order.
Planted mistakes in the merge must fail at least one of the merge pins.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import attention_fp64
from oracle.splitkv import (attention_keyrange_fp64, combine_fp64, num_splits_heuristic,
                            split_ranges, utilisation)


def _qkv(B, H, N, d, seed, sigma=1.0):
    g = np.random.default_rng(seed)
    return tuple(g.standard_normal((B, H, N, d)) * s for s in (sigma, sigma, 1.0))


def _merge_matches_definition(combine, q, k, v, causal, bounds):
    scale = 1.0 / math.sqrt(q.shape[-1])
    parts = [attention_keyrange_fp64(q, k, v, lo, hi, causal, scale) for lo, hi in bounds]
    O, L = combine(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    O_ref, L_ref = attention_fp64(q, k, v, causal, scale)
    return np.abs(O - O_ref).max() < 1e-12 and np.abs(L - L_ref).max() < 1e-12


PARTITIONS = [
    (37, [(0, 37)]),                                  # one range: the plain definition itself
    (37, [(0, 16), (16, 32), (32, 37)]),              # ragged last range
    (37, [(0, 5), (5, 5), (5, 37)]),                  # an empty range
    (40, [(0, 1), (1, 39), (39, 40)]),                # one-key ranges at both ends
    (64, [(48, 64), (0, 16), (16, 48)]),              # out of order
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,bounds", PARTITIONS)
def test_merge_of_any_partition_is_the_definition(N, bounds, causal):
    q, k, v = _qkv(2, 2, N, 8, seed=N)
    assert _merge_matches_definition(combine_fp64, q, k, v, causal, bounds)


def test_one_key_range_closed_form():
    q, k, v = _qkv(1, 1, 9, 4, seed=3)
    scale = 0.37
    O, L = attention_keyrange_fp64(q, k, v, 4, 5, causal=False, scale=scale)
    assert np.allclose(O[0, 0], np.broadcast_to(v[0, 0, 4], (9, 4)), rtol=0, atol=1e-15)
    assert np.allclose(L[0, 0], scale * (q[0, 0] @ k[0, 0, 4]), rtol=0, atol=1e-14)


def test_range_hidden_by_the_causal_mask():
    q, k, v = _qkv(1, 2, 12, 4, seed=5)
    O, L = attention_keyrange_fp64(q, k, v, 8, 12, causal=True)
    # rows 0..7 see none of the keys 8..11; row 8 sees key 8 only
    assert np.all(np.isneginf(L[:, :, :8])) and np.all(O[:, :, :8] == 0)
    assert np.allclose(O[:, :, 8], v[:, :, 8], rtol=0, atol=1e-15)


def test_equal_partials_closed_form():
    g = np.random.default_rng(7)
    Os, Ls = g.standard_normal((3, 5)), g.standard_normal(3)
    O, L = combine_fp64(np.stack([Os, Os]), np.stack([Ls, Ls]))
    assert np.allclose(O, Os, rtol=0, atol=1e-15)
    assert np.allclose(L, Ls + math.log(2.0), rtol=0, atol=1e-15)


def test_empty_range_contributes_nothing():
    g = np.random.default_rng(8)
    Os, Ls = g.standard_normal((4, 6)), g.standard_normal(4)
    O, L = combine_fp64(np.stack([np.zeros_like(Os), Os]), np.stack([np.full(4, -np.inf), Ls]))
    assert np.array_equal(O, Os) and np.array_equal(L, Ls)


def test_large_partial_lse_does_not_overflow():
    # L = 1001 + ln(1 + e^-1); O = (e^-1 * O_0 + O_1) / (1 + e^-1)
    O0, O1 = np.array([[1.0, -2.0]]), np.array([[3.0, 0.5]])
    O, L = combine_fp64(np.stack([O0, O1]), np.array([[1000.0], [1001.0]]))
    w0 = math.exp(-1.0) / (1.0 + math.exp(-1.0))
    assert np.allclose(L, 1001.0 + math.log1p(math.exp(-1.0)), rtol=0, atol=1e-12)
    assert np.allclose(O, w0 * O0 + (1 - w0) * O1, rtol=0, atol=1e-12)


# ---- planted mistakes: each broken merge must fail a pin above -----------------------------
def _no_max_shift(Op, Lp):
    w = np.exp(Lp)
    return (w[..., None] * Op).sum(0) / w.sum(0)[..., None], np.log(w.sum(0))


def _unnormalised(Op, Lp):
    m = Lp.max(0)
    w = np.exp(Lp - m)
    return (w[..., None] * Op).sum(0), m + np.log(w.sum(0))


def _mean_lse(Op, Lp):
    m = Lp.max(0)
    w = np.exp(Lp - m)
    return (w[..., None] * Op).sum(0) / w.sum(0)[..., None], m + np.log(w.mean(0))


def _max_only(Op, Lp):
    i = Lp.argmax(0)
    return np.take_along_axis(Op, i[None, ..., None], 0)[0], Lp.max(0)


@pytest.mark.parametrize("broken", [_no_max_shift, _unnormalised, _mean_lse, _max_only])
def test_every_planted_merge_mistake_is_caught(broken):
    caught = False
    try:
        O0, O1 = np.array([[1.0, -2.0]]), np.array([[3.0, 0.5]])
        with np.errstate(all="ignore"):
            O, L = broken(np.stack([O0, O1]), np.array([[1000.0], [1001.0]]))
        w0 = math.exp(-1.0) / (1.0 + math.exp(-1.0))
        caught |= not (np.allclose(L, 1001.0 + math.log1p(math.exp(-1.0)), atol=1e-12)
                       and np.allclose(O, w0 * O0 + (1 - w0) * O1, atol=1e-12))
    except (FloatingPointError, ValueError):
        caught = True
    q, k, v = _qkv(1, 2, 37, 8, seed=11)
    with np.errstate(all="ignore"):
        caught |= not _merge_matches_definition(broken, q, k, v, True, [(0, 16), (16, 32), (32, 37)])
    assert caught


# ---- the num_splits rule ---------------------------------------------------------------------
# Worked by hand with util(s) = (items*s/slots) / ceil(items*s/slots):
#  * 64 items on 512 slots, up to 8 splits: util = s/8 for s <= 8, so only s = 8 reaches 1.0.
#  * 4096 items on 512 slots: s = 1 already gives 8 full rounds (util 1.0).
#  * 100 items on 512 slots, up to 8: util(1..8) = .195 .391 .586 .781 .977 .586 .684 .781;
#    best .977 at s = 5, threshold .928 -> 5.
#  * 300 items on 512 slots, up to 4: util(1..4) = .586 .586 .879 .781; best .879 at s = 3,
#    threshold .835 -> 3.
#  * 10 items on 512 slots, up to 4 (few KV blocks): util = 10s/512, best at s = 4 -> 4.
@pytest.mark.parametrize("items,slots,max_splits,expected", [
    (64, 512, 8, 8), (4096, 512, 64, 1), (100, 512, 8, 5), (300, 512, 4, 3), (10, 512, 4, 4),
    (1, 1, 1, 1),
])
def test_num_splits_hand_worked(items, slots, max_splits, expected):
    assert num_splits_heuristic(items, slots, max_splits) == expected


def test_num_splits_defining_property():
    for items in (1, 7, 64, 100, 257, 1000):
        for max_splits in (1, 3, 16, 64):
            s = num_splits_heuristic(items, 512, max_splits)
            best = max(utilisation(items * t, 512) for t in range(1, max_splits + 1))
            assert 1 <= s <= max_splits
            assert utilisation(items * s, 512) >= 0.95 * best
            assert all(utilisation(items * t, 512) < 0.95 * best for t in range(1, s))


@pytest.mark.parametrize("n_blocks,s", [(1, 1), (1, 4), (7, 3), (16, 4), (17, 4), (5, 8)])
def test_split_ranges_partition(n_blocks, s):
    r = split_ranges(n_blocks, s)
    assert len(r) == s and r[0][0] == 0 and r[-1][1] == n_blocks
    assert all(a <= b for a, b in r) and all(r[i][1] == r[i + 1][0] for i in range(s - 1))


# ---- query and key lengths that differ (bottom-right causal alignment) ----------------------
@pytest.mark.parametrize("Nq,Nk,bounds", [(5, 40, [0, 13, 27, 40]), (40, 12, [0, 5, 12]),
                                          (1, 64, [0, 32, 64]), (33, 33, [0, 16, 33])])
@pytest.mark.parametrize("causal", [False, True])
def test_merge_with_different_lengths_is_the_definition(Nq, Nk, bounds, causal):
    g = np.random.default_rng(Nq * 100 + Nk)
    q = g.standard_normal((1, 2, Nq, 8))
    k, v = g.standard_normal((2, 1, 2, Nk, 8))
    parts = [attention_keyrange_fp64(q, k, v, lo, hi, causal, 0.5) for lo, hi in zip(bounds, bounds[1:])]
    O, L = combine_fp64([p[0] for p in parts], [p[1] for p in parts])
    Oref, Lref = attention_fp64(q, k, v, causal=causal, scale=0.5)
    np.testing.assert_allclose(O, Oref, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.isfinite(L), np.isfinite(Lref))
    fin = np.isfinite(Lref)
    np.testing.assert_allclose(L[fin], Lref[fin], rtol=0, atol=1e-13)


def test_rows_that_see_no_key_merge_to_zero_and_minus_infinity():
    q = np.ones((1, 1, 6, 4))
    k = v = np.ones((1, 1, 2, 4))
    parts = [attention_keyrange_fp64(q, k, v, lo, hi, True, 1.0) for lo, hi in ((0, 1), (1, 2))]
    O, L = combine_fp64([p[0] for p in parts], [p[1] for p in parts])
    # rows 0..3 see no key (j > i + 2 - 6 for every j); row 4 sees key 0, row 5 both
    assert np.all(O[0, 0, :4] == 0.0) and np.all(L[0, 0, :4] == -np.inf)
    np.testing.assert_allclose(L[0, 0, 4:], [4.0, 4.0 + math.log(2.0)], rtol=0, atol=1e-14)
    np.testing.assert_allclose(O[0, 0, 4:], 1.0, rtol=0, atol=1e-15)
