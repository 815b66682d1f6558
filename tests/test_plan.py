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
    assert L.hdp_pair_chunks(1 << 60, 4, 1, pa, pb) == _lib.HDP_ERR_OVERFLOW
