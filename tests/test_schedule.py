"""The kernels' work schedules, checked on the CPU through the library's host-side
schedule queries (fa2_schedule_map, fa2_schedule_blocks, fa2_bwd_block_map), which
run the same integer functions the kernels compile (csrc/fa2_schedule.h).

Forward (the pages' grid of one thread block per (query block, batch, head), page
"FlashAttention学习笔记(2)", section "V2中的thread blocks排布"), run as a persistent
grid: every work item must be processed by exactly one workgroup, each workgroup's
items must occupy positions 0..n-1 of its sequence, every XCD (workgroup id % 8) must
own one contiguous range of items, and the causal training and long workloads must
give every workgroup the same number of K/V blocks.  The total number of blocks is
checked against an independent count from the definition (a query block visits every
K/V block up to the one holding the last key its last row sees).

Backward: the logical block of each workgroup id must be a bijection on [0, G), with
each XCD taking one contiguous range.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np
import pytest

from exact_attention_62_amd import fa2 as F

pytestmark = pytest.mark.skipif(not os.path.exists(F.library_path()),
                                reason="libfa2.so not built (python -m exact_attention_62_amd.build)")

i32p = ctypes.POINTER(ctypes.c_int32)
i64p = ctypes.POINTER(ctypes.c_int64)


def _lib():
    lib = F.load_library()
    lib.fa2_schedule_map.argtypes = [ctypes.c_int64, ctypes.c_int64, i32p, i32p, i32p]
    lib.fa2_schedule_map.restype = ctypes.c_int
    lib.fa2_schedule_blocks.argtypes = [ctypes.c_int64] * 5 + [ctypes.c_int, ctypes.c_int,
                                                               ctypes.c_int, ctypes.c_int64,
                                                               i64p, i64p]
    lib.fa2_schedule_blocks.restype = ctypes.c_int
    lib.fa2_bwd_block_map.argtypes = [ctypes.c_int64, i32p]
    lib.fa2_bwd_block_map.restype = ctypes.c_int
    return lib


def schedule_map(items: int, grid: int):
    visits = np.full(items, -1, dtype=np.int32)
    wg = np.full(items, -1, dtype=np.int32)
    pos = np.full(items, -1, dtype=np.int32)
    st = _lib().fa2_schedule_map(items, grid, visits.ctypes.data_as(i32p),
                                 wg.ctypes.data_as(i32p), pos.ctypes.data_as(i32p))
    assert st == F.FA2_OK, F.fa2_last_error()
    return visits, wg, pos


def schedule_blocks(B, H, Nq, Nk, d, causal, grid, num_splits=0, dtype=F.FA2_BF16):
    blocks = np.full(grid, -1, dtype=np.int64)
    items = ctypes.c_int64(-1)
    st = _lib().fa2_schedule_blocks(B, H, Nq, Nk, d, dtype, int(causal), num_splits, grid,
                                    blocks.ctypes.data_as(i64p), ctypes.byref(items))
    assert st == F.FA2_OK, F.fa2_last_error()
    return blocks, items.value


ITEMS = sorted(set(range(1, 131)) | {255, 256, 257, 511, 512, 513, 1000, 2047, 2048, 4096,
                                     8191, 65535, 65539})
GRIDS = sorted(set(range(1, 17)) | {31, 32, 33, 63, 64, 100, 255, 256, 257, 511, 512})


@pytest.mark.parametrize("grid", GRIDS)
def test_every_item_exactly_once(grid):
    for items in ITEMS:
        visits, wg, pos = schedule_map(items, grid)
        assert np.all(visits == 1), (items, grid, np.flatnonzero(visits != 1)[:8])
        assert wg.min() >= 0 and wg.max() < grid
        # each workgroup's items sit at positions 0 .. n-1 of its sequence
        for g in np.unique(wg):
            p = np.sort(pos[wg == g])
            assert np.array_equal(p, np.arange(p.size)), (items, grid, g)
        # each XCD (id % 8, or id % grid below 8 workgroups) owns one contiguous range
        nx = min(grid, 8)
        xcd = wg % nx
        starts = [np.flatnonzero(xcd == x) for x in range(nx)]
        for idx in starts:
            if idx.size:
                assert idx[-1] - idx[0] + 1 == idx.size, (items, grid)
        firsts = [idx[0] for idx in starts if idx.size]
        assert firsts == sorted(firsts)


def test_snake_order_pairs_heavy_and_light():
    # 32 workgroups on one XCD's share: round k deals slot s position s (k even) or
    # P-1-s (k odd), so slot s takes items s and 2P-1-s of the first two rounds.
    visits, wg, pos = schedule_map(8 * 64, 8 * 32)
    for g in (0, 8, 8 * 31):
        mine = np.flatnonzero(wg == g)
        x, s = g % 8, g // 8
        base = x * 64
        assert list(mine - base) == sorted([s, 63 - s])


def _definition_blocks(B, H, Nq, Nk, kBM, BN, causal):
    """K/V blocks all work items visit, from the definition: every block up to the one
    holding the last key the last row of the query block sees (causal, aligned
    bottom-right), or every block; at least one block per query block."""
    nkb = math.ceil(Nk / BN)
    total = 0
    for m in range(math.ceil(Nq / kBM)):
        if not causal:
            total += nkb
            continue
        last_row = min((m + 1) * kBM, Nq) - 1
        last_key = last_row + Nk - Nq
        total += 1 if last_key < 0 else min(last_key // BN + 1, nkb)
    return B * H * total


@pytest.mark.parametrize("name,shape,causal", [
    ("train", (16, 16, 2048, 2048, 128), True),
    ("train", (16, 16, 2048, 2048, 128), False),
    ("long", (1, 16, 16384, 16384, 128), True),
    ("long", (1, 16, 16384, 16384, 128), False),
])
def test_block_balance_on_the_benchmark_shapes(name, shape, causal):
    """The eight-wavefront d = 128 form on 256 CUs (one workgroup per CU): every
    workgroup gets the same number of K/V blocks (the snake order pairs the heavy and
    light causal query blocks), and the blocks add up to the definition's count."""
    B, H, Nq, Nk, d = shape
    kBM = F.fa2_launch_shape(B, H, Nq, d)[0]
    assert kBM == 256
    items = B * H * math.ceil(Nq / kBM)
    grid = min(items, 256)
    blocks, n = schedule_blocks(B, H, Nq, Nk, d, causal, grid)
    assert n == items
    assert blocks.sum() == _definition_blocks(B, H, Nq, Nk, kBM, 64, causal)
    assert blocks.max() == blocks.min(), (name, causal, blocks.min(), blocks.max())


@pytest.mark.parametrize("shape,causal,grid", [
    ((2, 16, 8191, 8191, 256), True, 256),    # ragged d = 256: 32-key blocks
    ((1, 16, 2048, 2048, 128), True, 512),    # four wavefronts, one item each
    ((3, 5, 777, 1500, 64), True, 512),        # Nq != Nk, bottom-right mask
    ((1, 2, 1300, 700, 96), True, 7),          # rows that see no key; grid below 8
])
def test_block_totals_match_the_definition(shape, causal, grid):
    B, H, Nq, Nk, d = shape
    kBM = F.fa2_launch_shape(B, H, Nq, d)[0]
    BN = 32 if d == 256 else 64
    items = B * H * math.ceil(Nq / kBM)
    blocks, n = schedule_blocks(B, H, Nq, Nk, d, causal, min(grid, items))
    assert n == items
    assert blocks.sum() == _definition_blocks(B, H, Nq, Nk, kBM, BN, causal)


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 128])
def test_split_ranges_partition_each_query_block(splits):
    """With num_splits parts, the parts of a query block cover its blocks exactly once:
    the workgroups' blocks add up to the unsplit count."""
    B, H, Nq, Nk, d = 2, 3, 300, 5000, 128
    blocks, n = schedule_blocks(B, H, Nq, Nk, d, True, 200, num_splits=splits)
    assert n == B * H * math.ceil(Nq / 128) * splits
    assert blocks.sum() == _definition_blocks(B, H, Nq, Nk, 128, 64, True)


def test_schedule_queries_reject_bad_arguments():
    lib = _lib()
    v = np.zeros(4, dtype=np.int32)
    assert lib.fa2_schedule_map(0, 4, v.ctypes.data_as(i32p), None, None) == F.FA2_EINVAL
    assert lib.fa2_schedule_map(4, 0, v.ctypes.data_as(i32p), None, None) == F.FA2_EINVAL
    assert lib.fa2_schedule_map(4, 4, None, None, None) == F.FA2_EINVAL
    b = np.zeros(4, dtype=np.int64)
    n = ctypes.c_int64()
    assert lib.fa2_schedule_blocks(1, 1, 64, 64, 64, F.FA2_FP32, 0, 0, 4,
                                   b.ctypes.data_as(i64p), ctypes.byref(n)) == F.FA2_ENOTSUP
    assert lib.fa2_schedule_blocks(1, 1, 64, 0, 64, F.FA2_BF16, 0, 0, 4,
                                   b.ctypes.data_as(i64p), ctypes.byref(n)) == F.FA2_EINVAL
    assert lib.fa2_schedule_blocks(1, 1, 64, 64, 48, F.FA2_BF16, 0, 0, 4,
                                   b.ctypes.data_as(i64p), ctypes.byref(n)) == F.FA2_ENOTSUP
    assert lib.fa2_bwd_block_map(0, v.ctypes.data_as(i32p)) == F.FA2_EINVAL


@pytest.mark.parametrize("G", list(range(1, 300)) + [511, 512, 513, 2048, 4095, 65539])
def test_backward_block_order_is_a_bijection_with_contiguous_xcd_ranges(G):
    logical = np.full(G, -1, dtype=np.int32)
    assert _lib().fa2_bwd_block_map(G, logical.ctypes.data_as(i32p)) == F.FA2_OK
    assert np.array_equal(np.sort(logical), np.arange(G))
    ids = np.arange(G)
    prev_end = 0
    for x in range(8):
        mine = np.sort(logical[ids % 8 == x])
        if mine.size:
            assert mine[0] == prev_end and mine[-1] - mine[0] + 1 == mine.size, (G, x)
            prev_end = mine[-1] + 1
    assert prev_end == G
