"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

The pages print no attention values for a worked example, so each part of the oracle is pinned
by closed forms, invariants the pages state, an independent dense formulation built on scipy's
softmax / logsumexp, brute-force mask enumeration and finite differences.  Each pin is chosen
so that a plausible slip (wrong scale, off-by-one in the causal mask, wrong head group, log2
instead of ln, a dropped term in the merge or in the backward) fails at least one of them.

"Digest" = the research-digest page "ByteScale: Communication-Efficient Scaling of LLM Training
with a 2048K Context Length on 16384 GPUs".
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- closed forms


def test_single_token_sequence_returns_its_value_row():
    # s = 1: the only visible key is the row itself, so out = v_0 and lse = scale <q_0, k_0>.
    H, Hkv, D, scale = 4, 2, 8, 0.37
    q, k, v = rnd(1, 1, H, D), rnd(2, 1, Hkv, D), rnd(3, 1, Hkv, D)
    out, lse = oracle.varlen_fwd(q, k, v, [0, 1], scale)
    for h in range(H):
        g = h // (H // Hkv)
        np.testing.assert_allclose(out[0, h], v[0, g], rtol=0, atol=1e-15)
        assert lse[0, h] == pytest.approx(scale * float(q[0, h] @ k[0, g]), abs=1e-14)


def test_zero_query_gives_causal_prefix_mean_and_log_count():
    # q = 0: all scores are 0, so row r averages v_0..v_r of its own sequence and
    # lse_r = ln(r + 1) (natural log).  Distinct values per K/V head catch a wrong head map.
    lengths = [5, 1, 7]
    cu = np.cumsum([0] + lengths)
    T, H, Hkv, D = cu[-1], 6, 3, 4
    q = np.zeros((T, H, D))
    k = rnd(4, T, Hkv, D)
    v = rnd(5, T, Hkv, D) + 10.0 * np.arange(Hkv)[None, :, None]
    out, lse = oracle.varlen_fwd(q, k, v, cu, 0.5)
    for i, s in enumerate(lengths):
        a = cu[i]
        for r in range(s):
            for h in range(H):
                g = h // 2
                np.testing.assert_allclose(out[a + r, h], v[a:a + r + 1, g].mean(axis=0),
                                           rtol=0, atol=1e-13)
                assert lse[a + r, h] == pytest.approx(math.log(r + 1), abs=1e-14)


def test_equal_keys_give_prefix_mean_and_shifted_log_count():
    # Every key of a head equal to kappa: scores are constant per row, so out is the prefix
    # mean and lse_r = scale <q_r, kappa> + ln(r + 1).
    T, H, Hkv, D, scale = 9, 2, 1, 5, 0.8
    q = rnd(6, T, H, D)
    kappa = rnd(7, D)
    k = np.broadcast_to(kappa, (T, Hkv, D)).copy()
    v = rnd(8, T, Hkv, D)
    out, lse = oracle.varlen_fwd(q, k, v, [0, T], scale)
    for r in range(T):
        for h in range(H):
            np.testing.assert_allclose(out[r, h], v[:r + 1, 0].mean(axis=0), atol=1e-13)
            assert lse[r, h] == pytest.approx(scale * float(q[r, h] @ kappa) + math.log(r + 1),
                                              abs=1e-12)


def test_constant_values_are_reproduced():
    T, H, Hkv, D = 12, 4, 4, 3
    q, k = rnd(9, T, H, D), rnd(10, T, Hkv, D)
    c = np.array([1.5, -2.0, 0.25])
    v = np.broadcast_to(c, (T, Hkv, D)).copy()
    out, _ = oracle.varlen_fwd(q, k, v, [0, 4, 12], 0.3)
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), atol=1e-14)


def test_key_shift_leaves_output_and_moves_lse_by_query_projection():
    # Adding u to every key of a sequence adds scale <q_r, u> to every score of row r.
    T, H, Hkv, D, scale = 10, 2, 2, 4, 0.6
    q, k, v = rnd(11, T, H, D), rnd(12, T, Hkv, D), rnd(13, T, Hkv, D)
    u = rnd(14, D)
    out0, lse0 = oracle.varlen_fwd(q, k, v, [0, T], scale)
    out1, lse1 = oracle.varlen_fwd(q, k + u, v, [0, T], scale)
    np.testing.assert_allclose(out1, out0, atol=1e-12)
    np.testing.assert_allclose(lse1 - lse0, scale * np.einsum("thd,d->th", q, u), atol=1e-12)


# ------------------------------------------------- independent dense formulation


def dense_reference(q, k, v, cu, scale):
    """T x T scores with a block-diagonal causal mask, softmax and logsumexp from scipy."""
    T, H, D = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    seq = np.zeros(T, np.int64)
    for i in range(len(cu) - 1):
        seq[cu[i]:cu[i + 1]] = i
    idx = np.arange(T)
    allowed = (seq[:, None] == seq[None, :]) & (idx[None, :] <= idx[:, None])
    out = np.zeros_like(q)
    lse = np.zeros((T, H))
    for h in range(H):
        kh, vh = k[:, h // G, :], v[:, h // G, :]
        s = scale * (q[:, h, :] @ kh.T)
        s = np.where(allowed, s, -np.inf)
        out[:, h, :] = softmax(s, axis=1) @ vh
        lse[:, h] = logsumexp(s, axis=1)
    return out, lse


@pytest.mark.parametrize("lengths,H,Hkv,D", [([17, 64, 100, 75], 4, 4, 8),
                                             ([1, 2, 3, 30, 0, 9], 8, 2, 16),
                                             ([40], 2, 1, 32)])
def test_matches_dense_masked_softmax(lengths, H, Hkv, D):
    cu = np.cumsum([0] + lengths)
    T = cu[-1]
    q, k, v = rnd(20, T, H, D), rnd(21, T, Hkv, D), rnd(22, T, Hkv, D)
    scale = 1 / math.sqrt(D)
    out, lse = oracle.varlen_fwd(q, k, v, cu, scale)
    ro, rl = dense_reference(q, k, v, cu, scale)
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


def test_packed_equals_each_sequence_alone_bitwise():
    # "a query attends only to its own sequence" (Digest §3.2).
    lengths = [3, 20, 1, 11]
    cu = np.cumsum([0] + lengths)
    T, H, Hkv, D = cu[-1], 4, 2, 8
    q, k, v = rnd(30, T, H, D), rnd(31, T, Hkv, D), rnd(32, T, Hkv, D)
    out, lse = oracle.varlen_fwd(q, k, v, cu, 0.3)
    for i in range(len(lengths)):
        a, b = cu[i], cu[i + 1]
        o1, l1 = oracle.varlen_fwd(q[a:b], k[a:b], v[a:b], [0, b - a], 0.3)
        assert np.array_equal(o1, out[a:b]) and np.array_equal(l1, lse[a:b])


def test_row_selection_and_thread_count_do_not_change_results():
    lengths = [50, 13, 64]
    cu = np.cumsum([0] + lengths)
    T, H, Hkv, D = cu[-1], 4, 1, 16
    q, k, v = rnd(33, T, H, D), rnd(34, T, Hkv, D), rnd(35, T, Hkv, D)
    o1, l1 = oracle.varlen_fwd(q, k, v, cu, 0.25, nthreads=1)
    o8, l8 = oracle.varlen_fwd(q, k, v, cu, 0.25, nthreads=8)
    assert np.array_equal(o1, o8) and np.array_equal(l1, l8)
    rows = [126, 0, 63, 50, 49]
    orow, lrow = oracle.varlen_fwd(q, k, v, cu, 0.25, rows=rows)
    assert np.array_equal(orow, o1[rows]) and np.array_equal(lrow, l1[rows])


def test_zero_length_sequences_are_allowed():
    cu = [0, 0, 5, 5, 9, 9]
    T, H, D = 9, 2, 4
    q, k, v = rnd(36, T, H, D), rnd(37, T, 1, D), rnd(38, T, 1, D)
    out, lse = oracle.varlen_fwd(q, k, v, cu, 0.5)
    o2, l2 = oracle.varlen_fwd(q, k, v, [0, 5, 9], 0.5)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


# ------------------------------------------------------ ring chunks and the merge


def test_whole_sequence_chunk_equals_varlen_bitwise():
    # A sequence of at most C tokens needs no partner (Digest §2): one chunk at offset 0 over
    # the whole sequence is exactly the local attention.
    s, H, Hkv, D = 33, 4, 2, 8
    q, k, v = rnd(40, s, H, D), rnd(41, s, Hkv, D), rnd(42, s, Hkv, D)
    o, l = oracle.chunk_partial(q, k, v, 0, 0, True, 0.4)
    o2, l2 = oracle.varlen_fwd(q, k, v, [0, s], 0.4)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_non_causal_chunk_is_plain_softmax():
    Lq, Lk, H, Hkv, D = 5, 7, 2, 1, 4
    q, k, v = rnd(43, Lq, H, D), rnd(44, Lk, Hkv, D), rnd(45, Lk, Hkv, D)
    o, l = oracle.chunk_partial(q, k, v, 1000, 0, False, 0.5)
    for h in range(H):
        s = 0.5 * q[:, h] @ k[:, 0].T
        np.testing.assert_allclose(o[:, h], softmax(s, axis=1) @ v[:, 0], atol=1e-13)
        np.testing.assert_allclose(l[:, h], logsumexp(s, axis=1), atol=1e-13)


def test_future_chunk_rows_are_empty():
    # Keys at positions after every query: nothing visible, out = 0, lse = -inf.
    q, k, v = rnd(46, 4, 2, 4), rnd(47, 6, 2, 4), rnd(48, 6, 2, 4)
    o, l = oracle.chunk_partial(q, k, v, 10, 14, True, 0.5)
    assert np.all(o == 0.0) and np.all(l == -np.inf)
    # partially visible: row r sees keys j with 14 + j <= 10 + r, i.e. j <= r - 4
    q2 = rnd(49, 8, 2, 4)
    o2, l2 = oracle.chunk_partial(q2, k, v, 10, 14, True, 0.5)
    assert np.all(l2[:4] == -np.inf) and np.all(np.isfinite(l2[4:]))


def test_merge_with_empty_partial_is_identity():
    o, l = rnd(50, 3, 2, 4), rnd(51, 3, 2)
    empty_o, empty_l = np.zeros((3, 2, 4)), np.full((3, 2), -np.inf)
    mo, ml = oracle.lse_merge(o, l, empty_o, empty_l)
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    mo, ml = oracle.lse_merge(empty_o, empty_l, o, l)
    assert np.array_equal(mo, o) and np.array_equal(ml, l)
    mo, ml = oracle.lse_merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(ml == -np.inf) and np.all(mo == 0) and not np.any(np.isnan(mo))


def test_merge_is_commutative():
    o1, l1, o2, l2 = rnd(52, 4, 3, 5), rnd(53, 4, 3), rnd(54, 4, 3, 5), rnd(55, 4, 3)
    a = oracle.lse_merge(o1, l1, o2, l2)
    b = oracle.lse_merge(o2, l2, o1, l1)
    np.testing.assert_allclose(a[0], b[0], atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], atol=1e-15)


@pytest.mark.parametrize("order", ["forward", "reverse", "shuffled"])
def test_ring_partials_merged_equal_full_causal_attention(order):
    # Ring attention (Digest §3.2): the slice of a long sequence attends to one K/V chunk per
    # step; merging the per-step partials by log-sum-exp gives full causal attention.
    chunk, n_chunks, H, Hkv, D = 6, 5, 4, 2, 8
    L = chunk * n_chunks
    q, k, v = rnd(56, L, H, D), rnd(57, L, Hkv, D), rnd(58, L, Hkv, D)
    full_o, full_l = oracle.varlen_fwd(q, k, v, [0, L], 0.35)
    steps = list(range(n_chunks))
    if order == "reverse":
        steps.reverse()
    elif order == "shuffled":
        np.random.default_rng(7).shuffle(steps)
    for qi in range(n_chunks):
        qs = q[qi * chunk:(qi + 1) * chunk]
        acc_o, acc_l = np.zeros((chunk, H, D)), np.full((chunk, H), -np.inf)
        for kj in steps:
            po, pl = oracle.chunk_partial(qs, k[kj * chunk:(kj + 1) * chunk],
                                          v[kj * chunk:(kj + 1) * chunk], qi * chunk,
                                          kj * chunk, True, 0.35)
            acc_o, acc_l = oracle.lse_merge(acc_o, acc_l, po, pl)
        np.testing.assert_allclose(acc_o, full_o[qi * chunk:(qi + 1) * chunk], atol=1e-12)
        np.testing.assert_allclose(acc_l, full_l[qi * chunk:(qi + 1) * chunk], atol=1e-12)


# ------------------------------------------------------------------- backward


def loss(q, k, v, do, cu, scale):
    out, _ = oracle.varlen_fwd(q, k, v, cu, scale)
    return float(np.sum(do * out))


@pytest.mark.parametrize("lengths,H,Hkv,D", [([5, 3], 2, 2, 3), ([8], 4, 2, 4), ([1, 6], 2, 1, 2)])
def test_backward_matches_central_differences(lengths, H, Hkv, D):
    cu = np.cumsum([0] + lengths)
    T = cu[-1]
    q, k, v, do = rnd(60, T, H, D), rnd(61, T, Hkv, D), rnd(62, T, Hkv, D), rnd(63, T, H, D)
    scale = 0.7
    dq, dk, dv = oracle.varlen_bwd(q, k, v, do, cu, scale)
    eps = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"], do, cu, scale)
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"], do, cu, scale)
            num[idx] = (lp - lm) / (2 * eps)
        err = np.max(np.abs(num - g)) / max(1.0, np.max(np.abs(num)))
        assert err < 1e-7, (name, err)


def test_backward_group_identities_and_row_selection():
    # Per sequence and K/V head: sum_j dK_j = 0 (softmax rows are shift invariant) and
    # sum_j dV_j = sum over the group's heads and rows of dO_r.
    lengths = [9, 4, 12]
    cu = np.cumsum([0] + lengths)
    T, H, Hkv, D = cu[-1], 4, 2, 5
    q, k, v, do = rnd(64, T, H, D), rnd(65, T, Hkv, D), rnd(66, T, Hkv, D), rnd(67, T, H, D)
    dq, dk, dv = oracle.varlen_bwd(q, k, v, do, cu, 0.45)
    for i in range(len(lengths)):
        a, b = cu[i], cu[i + 1]
        for g in range(Hkv):
            np.testing.assert_allclose(dk[a:b, g].sum(axis=0), 0.0, atol=1e-12)
            np.testing.assert_allclose(dv[a:b, g].sum(axis=0),
                                       do[a:b, 2 * g:2 * g + 2].sum(axis=(0, 1)), atol=1e-12)
    qrows, krows = [24, 3, 9], [0, 13, 24, 12]
    dq2, dk2, dv2 = oracle.varlen_bwd(q, k, v, do, cu, 0.45, qrows=qrows, krows=krows)
    assert np.array_equal(dq2, dq[qrows])
    assert np.array_equal(dk2, dk[krows]) and np.array_equal(dv2, dv[krows])


# ------------------------------------------------------- ring-chunk backward

@pytest.mark.parametrize("cuts_q,cuts_k", [([0, 13], [0, 5, 13]), ([0, 6, 13], [0, 9, 13]),
                                           ([0, 4, 9, 13], [0, 4, 9, 13])])
def test_chunk_backward_over_a_ring_partition_sums_to_the_full_backward(cuts_q, cuts_k):
    # One causal sequence of 13 tokens, its rows cut into slices and its keys into chunks.
    # Given the full forward's out and lse, every slice x chunk step adds its share: dQ of a
    # slice is the sum over chunks, dK/dV of a chunk the sum over slices (ring reading of the
    # pages' long-sequence path; the reference is the separately written packed backward).
    S, H, Hkv, D, scale = 13, 4, 2, 5, 0.6
    q, k, v, do = rnd(80, S, H, D), rnd(81, S, Hkv, D), rnd(82, S, Hkv, D), rnd(83, S, H, D)
    cu = np.array([0, S])
    out, lse = oracle.varlen_fwd(q, k, v, cu, scale)
    dq_ref, dk_ref, dv_ref = oracle.varlen_bwd(q, k, v, do, cu, scale)
    dq = np.zeros_like(dq_ref)
    dk = np.zeros_like(dk_ref)
    dv = np.zeros_like(dv_ref)
    for a, b in zip(cuts_q[:-1], cuts_q[1:]):
        for c, e in zip(cuts_k[:-1], cuts_k[1:]):
            gq, gk, gv = oracle.chunk_bwd(q[a:b], k[c:e], v[c:e], a, c, True, scale,
                                          out[a:b], lse[a:b], do[a:b])
            dq[a:b] += gq
            dk[c:e] += gk
            dv[c:e] += gv
    np.testing.assert_allclose(dq, dq_ref, atol=1e-12)
    np.testing.assert_allclose(dk, dk_ref, atol=1e-12)
    np.testing.assert_allclose(dv, dv_ref, atol=1e-12)


def test_future_chunk_backward_is_zero():
    # A chunk entirely after the slice contributes nothing (every pair masked).
    H, Hkv, D = 2, 1, 3
    q, k, v, do = rnd(84, 4, H, D), rnd(85, 5, Hkv, D), rnd(86, 5, Hkv, D), rnd(87, 4, H, D)
    out, lse = rnd(88, 4, H, D), rnd(89, 4, H)
    dq, dk, dv = oracle.chunk_bwd(q, k, v, 10, 14, True, 0.5, out, lse, do)
    assert not dq.any() and not dk.any() and not dv.any()


def test_chunk_backward_row_selection():
    H, Hkv, D = 2, 1, 4
    q, k, v, do = rnd(94, 20, H, D), rnd(95, 15, Hkv, D), rnd(96, 15, Hkv, D), rnd(97, 20, H, D)
    out, lse = rnd(98, 20, H, D), rnd(99, 20, H)
    a = oracle.chunk_bwd(q, k, v, 5, 3, True, 0.5, out, lse, do)
    b = oracle.chunk_bwd(q, k, v, 5, 3, True, 0.5, out, lse, do, qrows=[3, 19, 0], krows=[14, 2])
    assert np.array_equal(a[0][[3, 19, 0]], b[0])
    assert np.array_equal(a[1][[14, 2]], b[1]) and np.array_equal(a[2][[14, 2]], b[2])


def test_non_causal_chunk_backward_matches_central_differences():
    # Non-causal slice x chunk: L = sum(dO * out) with out from the oracle's chunk partial;
    # the analytic gradients must match central differences of L.
    Lq, Lk, H, Hkv, D, scale = 3, 4, 2, 1, 3, 0.8
    q, k, v, do = rnd(90, Lq, H, D), rnd(91, Lk, Hkv, D), rnd(92, Lk, Hkv, D), rnd(93, Lq, H, D)

    def L(qq, kk, vv):
        o, _ = oracle.chunk_partial(qq, kk, vv, 7, 2, False, scale)
        return float(np.sum(do * o))

    out, lse = oracle.chunk_partial(q, k, v, 7, 2, False, scale)
    dq, dk, dv = oracle.chunk_bwd(q, k, v, 7, 2, False, scale, out, lse, do)
    eps = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args[name] = xp
            lp = L(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = L(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * eps)
        assert np.max(np.abs(num - g)) < 1e-7 * max(1.0, np.max(np.abs(num))), name


# ----------------------------------------------------------------------- FLOPs


@pytest.mark.parametrize("s", [0, 1, 2, 7, 64, 100, 511, 512])
def test_pair_count_is_the_triangle_number(s):
    # Causal: row r sees r + 1 keys, so s (s + 1) / 2 pairs; without the mask, s^2.
    assert oracle.count_pairs(s, s, 0, 0, True) == s * (s + 1) // 2
    assert oracle.count_pairs(s, s, 0, 0, False) == s * s


def test_chunk_pair_counts_tile_the_triangle():
    s, c = 96, 32
    total = sum(oracle.count_pairs(c, c, qi * c, kj * c, True)
                for qi in range(s // c) for kj in range(s // c))
    assert total == s * (s + 1) // 2


def test_flop_conventions():
    # fwd 4D per pair per head (two length-D contractions), bwd 10D (five).
    assert oracle.attn_flops(3, 3, 0, 0, True, 2, 8, 0) == 6 * 2 * 32
    assert oracle.attn_flops(3, 3, 0, 0, True, 2, 8, 1) == 6 * 2 * 80
    assert oracle.attn_flops(3, 3, 0, 0, True, 2, 8, 2) == 6 * 2 * 112
