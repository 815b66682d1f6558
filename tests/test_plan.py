"""Host planning: front/back chunk pairing (and, below, HDP sharding and the balance scheduler).

The pairing pins are the pages' claim that 2N chunks handed out in front/back pairs balance the
causal mask: with 2N | s every rank's visible pairs over the whole ring are equal (counted by
the library's closed form and, independently, by the oracle's brute-force enumeration)."""
import pytest

import oracle
from variable_length_attention_amd import _lib, ops


def rank_pairs_library(s, N, k):
    """Visible causal pairs of rank k's two query chunks against every chunk of the ring."""
    mine = ops.hdp_pair_chunks(s, N, k)
    allc = [c for r in range(N) for c in ops.hdp_pair_chunks(s, N, r)]
    total = 0
    for qo, ql in mine:
        for ko, kl in allc:
            total += ops.hdp_chunk_flops(ql, kl, qo, ko, True, 1, 1) // 4   # 4 H D per pair
    return total


@pytest.mark.parametrize("s,N", [(0, 3), (1, 1), (10, 4), (4096, 16), (131072, 16), (1000, 7), (37, 5)])
def test_pair_chunks_tile_the_sequence(s, N):
    pieces = sorted(c for k in range(N) for c in ops.hdp_pair_chunks(s, N, k))
    pos = 0
    for off, ln in pieces:
        assert off == pos and ln >= 0
        pos += ln
    assert pos == s
    for k in range(N):
        (o0, l0), (o1, l1) = ops.hdp_pair_chunks(s, N, k)
        assert o0 <= o1 and abs(l0 - s // (2 * N)) <= 1 and abs(l1 - s // (2 * N)) <= 1


@pytest.mark.parametrize("s,N", [(64, 4), (96, 3), (128, 8), (4096, 16)])
def test_front_back_pairs_equalise_causal_work(s, N):
    per_rank = [rank_pairs_library(s, N, k) for k in range(N)]
    assert len(set(per_rank)) == 1
    assert sum(per_rank) == s * (s + 1) // 2
    # contiguous slicing of the same ring is far from it: the last rank does (2N-1)x the first
    c = s // N
    contiguous = [oracle.count_pairs(c, s, k * c, 0, True) for k in range(N)]
    assert contiguous[-1] > contiguous[0] * (2 * N - 2)


def test_front_back_pair_counts_match_brute_force():
    s, N = 48, 3
    for k in range(N):
        mine = ops.hdp_pair_chunks(s, N, k)
        brute = sum(oracle.count_pairs(ql, s, qo, 0, True) for qo, ql in mine)
        assert brute == rank_pairs_library(s, N, k)


def test_pair_chunks_validation():
    L = _lib.lib()
    import ctypes
    a = (ctypes.c_int64 * 2)()
    b = (ctypes.c_int64 * 2)()
    pa, pb = ctypes.addressof(a), ctypes.addressof(b)
    assert L.hdp_pair_chunks(-1, 4, 0, pa, pb) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_pair_chunks(10, 0, 0, pa, pb) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_pair_chunks(10, 4, 4, pa, pb) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_pair_chunks(10, 4, 1, None, pb) == _lib.HDP_ERR_INVALID_ARG


@pytest.mark.parametrize("s,N,k", [(1 << 60, 4, 1), ((1 << 63) - 1, 2 ** 31 - 1, 2 ** 31 - 2),
                                   ((1 << 62) + 12345, 2 ** 30 + 7, 5), (10 ** 18, 3, 2)])
def test_pair_chunks_bounds_exact_at_int64_limits(s, N, k):
    # c * s exceeds 64 bits here: the bounds floor(c s / 2N) must still be exact
    (o0, l0), (o1, l1) = ops.hdp_pair_chunks(s, N, k)
    n2 = 2 * N
    assert (o0, l0) == (k * s // n2, (k + 1) * s // n2 - k * s // n2)
    c = n2 - 1 - k
    assert (o1, l1) == (c * s // n2, (c + 1) * s // n2 - c * s // n2)


# ---------------------------------------------------------------------- HDP sharding

K = 1024


def test_figure2_layout_exactly():
    # Five sequences (32K, 16K, 8K, 4K, 4K) on a pool of eight ranks of C = 8K (digest §3.1,
    # Figure 2b): ranks 0-3 ring of 4 for S0, ranks 4-5 ring of 2 for S1, S2 alone on rank 6,
    # S3 and S4 packed on rank 7.
    plan = ops.hdp_plan_shard([32 * K, 16 * K, 8 * K, 4 * K, 4 * K], 8 * K)
    assert plan.units() == [
        (0, [(0, 0, 8 * K)]), (0, [(0, 8 * K, 8 * K)]), (0, [(0, 16 * K, 8 * K)]), (0, [(0, 24 * K, 8 * K)]),
        (1, [(1, 0, 8 * K)]), (1, [(1, 8 * K, 8 * K)]),
        (-1, [(2, 0, 8 * K)]),
        (-1, [(3, 0, 4 * K), (4, 0, 4 * K)]),
    ]
    cost = ops.hdp_plan_unit_flops(plan, 32, 128)
    ranks, load = ops.hdp_plan_balance(cost, plan.ring, 8)
    assert ranks == list(range(8))                       # one unit per rank, in Figure 2's order
    # the ring units hold the ring's causal work, summed back to the sequence's FLOPs
    assert sum(cost[0:4]) == ops.hdp_seq_flops(32 * K, 32, 128)
    assert sum(cost[4:6]) == ops.hdp_seq_flops(16 * K, 32, 128)
    assert cost[7] == ops.hdp_seq_flops(4 * K, 32, 128) * 2


@pytest.mark.parametrize("s,C,ranks", [
    (2048 * K, 8 * K, 256),      # a 2M-token sequence at C = 8K needs 256 ranks
    (8 * K, 8 * K, 1),           # an 8K one needs one
    (16 * K, 8 * K, 2),          # a 16K one only two
    (312 * K, 8 * K, 39),        # the measured HDP ring: 312K on 39 ranks
    (768 * K, 8 * K, 96),        # 768K needs 96 ranks
    (1024 * K, 8 * K, 128),      # a 1M context at 8K per GPU: d_cp = 128
])
def test_ring_sizes_are_ceil_s_over_C(s, C, ranks):
    plan = ops.hdp_plan_shard([s], C)
    units = plan.units()
    assert len(units) == ranks
    assert all(len(p) == 1 and p[0][2] <= C for _, p in units)
    if ranks > 1:
        assert all(r == 0 for r, _ in units)
    else:
        assert units == [(-1, [(0, 0, s)])]


def test_768k_and_32_8k_sequences_fill_128_ranks():
    # At C = 8K a 768K sequence takes 96 ranks; on 128 ranks the other 32 hold an 8K sequence
    # each (digest §3.1).
    plan = ops.hdp_plan_shard([768 * K] + [8 * K] * 32, 8 * K)
    units = plan.units()
    assert len(units) == 128
    assert [r for r, _ in units[:96]] == [0] * 96
    assert [p for _, p in units[96:]] == [[(i, 0, 8 * K)] for i in range(1, 33)]


def test_paired_ring_units_have_equal_work():
    s, C = 64 * K, 8 * K
    plan = ops.hdp_plan_shard([s], C, pair=True)
    units = plan.units()
    assert len(units) == 8 and all(len(p) == 2 for _, p in units)
    cost = ops.hdp_plan_unit_flops(plan, 32, 128)
    assert len(set(cost)) == 1 and sum(cost) == ops.hdp_seq_flops(s, 32, 128)
    contiguous = ops.hdp_plan_unit_flops(ops.hdp_plan_shard([s], C), 32, 128)
    assert max(contiguous) > 10 * min(contiguous)


def test_best_fit_packing_is_tight_and_complete():
    import numpy as np
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(1, 3000, size=60)]
    C = 4096
    plan = ops.hdp_plan_shard(lens, C)
    seen = []
    for ring, pieces in plan.units():
        assert ring == -1 and sum(p[2] for p in pieces) <= C
        seen += [p[0] for p in pieces]
    assert sorted(seen) == list(range(60))
    # best fit leaves at most one unit half empty or less
    fills = [sum(p[2] for p in pieces) for _, pieces in plan.units()]
    assert sum(f <= C // 2 for f in fills) <= 1


# ------------------------------------------------------------------ balance scheduler

def test_balance_equal_time_with_unequal_counts():
    # Units of equal tokens but unequal work (Figure 4): 2 long (6), 4 medium (3), 12 short (1)
    # on 4 ranks.  Equal counts (4-5 each) cannot meet; the scheduler ends every rank at 9.
    cost = [6] * 2 + [3] * 4 + [1] * 12
    ranks, load = ops.hdp_plan_balance(cost, [-1] * len(cost), 4)
    assert load == [9, 9, 9, 9]
    counts = [ranks.count(r) for r in range(4)]
    assert sum(counts) == 18 and max(counts) > min(counts)


def test_balance_keeps_rings_on_distinct_ranks_and_conserves_work():
    import numpy as np
    lens = [40 * K, 24 * K, 9 * K] + [int(x) for x in np.random.default_rng(9).integers(200, 8 * K, 70)]
    plan = ops.hdp_plan_shard(lens, 8 * K)
    cost = ops.hdp_plan_unit_flops(plan, 32, 128)
    for delta in (0, 10 ** 11):
        ranks, load = ops.hdp_plan_balance(cost, plan.ring, 16, delta)
        assert sum(load) == sum(cost)
        for r in range(16):
            assert load[r] == sum(c for c, u in zip(cost, ranks) if u == r)
        for seq in set(x for x in plan.ring if x >= 0):
            members = [ranks[j] for j in range(len(ranks)) if plan.ring[j] == seq]
            assert len(set(members)) == len(members)
        assert max(load) - min(load) <= delta + max(cost)


def test_planner_validation():
    import ctypes
    L = _lib.lib()
    n = ctypes.c_int32(0)
    lens = (ctypes.c_int64 * 2)(5, -1)
    assert L.hdp_plan_shard(ctypes.addressof(lens), 2, 8, 0, 0, 0, ctypes.addressof(n),
                            ctypes.addressof(n), None, None, None, None, None) == _lib.HDP_ERR_INVALID_ARG
    lens = (ctypes.c_int64 * 2)(5, 7)
    assert L.hdp_plan_shard(ctypes.addressof(lens), 2, 0, 0, 0, 0, ctypes.addressof(n),
                            ctypes.addressof(n), None, None, None, None, None) == _lib.HDP_ERR_INVALID_ARG
    m = ctypes.c_int32(0)
    assert L.hdp_plan_shard(ctypes.addressof(lens), 2, 8, 0, 0, 0, ctypes.addressof(n),
                            ctypes.addressof(m), None, None, None, None, None) == _lib.HDP_ERR_OVERFLOW
    assert (n.value, m.value) == (2, 2)          # 7 and 5 do not share a unit of 8
    cost = (ctypes.c_uint64 * 3)(1, 1, 1)
    ring = (ctypes.c_int32 * 3)(0, 0, 0)
    ur = (ctypes.c_int32 * 3)()
    load = (ctypes.c_uint64 * 2)()
    assert L.hdp_plan_balance(ctypes.addressof(cost), ctypes.addressof(ring), 3, 2, 0,
                              ctypes.addressof(ur), ctypes.addressof(load)) == _lib.HDP_ERR_INVALID_ARG
