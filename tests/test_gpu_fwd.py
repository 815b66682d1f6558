"""GPU parity of the forward paths against the fp64 oracle, through the C ABI.

Small cases and the 8K packed slice compare every element; the 32K micro-batches and the ring
share compare a deterministic row sample (every 8th row, both sides of every tile edge and the
first and last row of every sequence, all heads) that the oracle evaluates row by row.  Exactness properties of the packing (a query attends only to
its own sequence) are checked bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TOL_BF16_LSE, TOL_BF16_OUT, TOL_F32, boundary_rows, lse_close, max_abs,
                      sample_rows, to_gpu)
from variable_length_attention_amd import ops, synth

pytestmark = pytest.mark.gpu


def varlen_case(lengths, H, Hkv, D, seed, dtype="bf16"):
    w = synth.Workload("case", "varlen", H, Hkv, D, dtype, list(lengths), seed)
    q, k, v = synth.varlen_tensors(w)
    cu = synth.cu_seqlens(w.lengths)
    return w, q, k, v, cu


def run_fwd(q, k, v, cu, scale):
    qg, kg, vg = to_gpu(q, k, v)
    cug = torch.from_numpy(cu).to("cuda")
    out, lse = ops.hdp_attn_varlen_fwd(qg, kg, vg, cug, scale)
    torch.cuda.synchronize()
    return out, lse


def test_tiny_fp32_pack_full():
    w = synth.tiny_fp32_pack()
    q, k, v = synth.varlen_tensors(w)
    cu = synth.cu_seqlens(w.lengths)
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale)
    qg, kg, vg = to_gpu(q, k, v)
    out, lse = ops.hdp_attn_varlen_fwd_f32(qg, kg, vg, torch.from_numpy(cu).cuda(), w.scale)
    torch.cuda.synchronize()
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print("%s: all %d rows, max|dout|=%.3g max|dlse|=%.3g" % (w.name, int(cu[-1]), e_out, e_lse))
    assert e_out <= TOL_F32
    assert e_lse <= TOL_F32


@pytest.mark.parametrize("lengths,H,Hkv,D", [([1, 5, 37, 0, 260, 33], 8, 2, 128),
                                             ([3, 100, 64, 131], 6, 3, 64),
                                             ([300, 7, 0, 257, 129], 4, 4, 64)])
def test_fp32_ragged_pack_full(lengths, H, Hkv, D):
    # grouped heads, empty and single-token sequences, rows past one row block, key counts that
    # are not multiples of the kernel's 4-key blocks, and sequences whose keys span more than one
    # LDS chunk (128 keys at D = 128, 256 at D = 64)
    w, q, k, v, cu = varlen_case(lengths, H, Hkv, D, 23, dtype="f32")
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale)
    qg, kg, vg = to_gpu(q, k, v)
    out, lse = ops.hdp_attn_varlen_fwd_f32(qg, kg, vg, torch.from_numpy(cu).cuda(), w.scale)
    torch.cuda.synchronize()
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print("fp32 lengths=%s H=%d Hkv=%d D=%d max|dout|=%.3g max|dlse|=%.3g" % (lengths, H, Hkv, D, e_out, e_lse))
    assert e_out <= TOL_F32
    assert e_lse <= TOL_F32


RAGGED = [1, 17, 64, 65, 127, 128, 129, 300, 0, 513, 31]


@pytest.mark.parametrize("H,Hkv,D", [(32, 8, 128), (8, 8, 64), (4, 2, 128), (16, 2, 64),
                                     (6, 2, 64), (32, 8, 64)])
def test_bf16_ragged_pack_full(H, Hkv, D):
    w, q, k, v, cu = varlen_case(RAGGED, H, Hkv, D, seed=11)
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale)
    out, lse = run_fwd(q, k, v, cu, w.scale)
    e_out = max_abs(out, ro)
    e_lse = max_abs(lse, rl)
    print("H=%d Hkv=%d D=%d max|dout|=%.3g max|dlse|=%.3g" % (H, Hkv, D, e_out, e_lse))
    assert e_out <= TOL_BF16_OUT and e_lse <= TOL_BF16_LSE


def test_packed_slice_8k_every_row():
    # One rank's whole 8192-token slice (9 sequences): every row and head against the oracle.
    # This is the digest's §3.1-§3.2 rule in full: each packed sequence attends only to itself.
    w = synth.packed_slice_8k()
    q, k, v = synth.varlen_tensors(w)
    cu = synth.cu_seqlens(w.lengths)
    out, lse = run_fwd(q, k, v, cu, w.scale)
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale)
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print("%s: all %d rows, max|dout|=%.3g max|dlse|=%.3g" % (w.name, int(cu[-1]), e_out, e_lse))
    assert e_out <= TOL_BF16_OUT and e_lse <= TOL_BF16_LSE


@pytest.mark.parametrize("make", [synth.microbatch_32k_short, synth.microbatch_32k_long])
def test_microbatch_32k_sampled(make):
    # Every 8th packed row, both sides of every 64-row tile edge and the first and last row of
    # every sequence, all heads.
    w = make()
    q, k, v = synth.varlen_tensors(w)
    cu = synth.cu_seqlens(w.lengths)
    out, lse = run_fwd(q, k, v, cu, w.scale)
    rows = np.union1d(sample_rows(cu, 8), boundary_rows(int(cu[-1]), 8))
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    e_out = max_abs(out[idx], ro)
    e_lse = max_abs(lse[idx], rl)
    print("%s: %d sampled rows, max|dout|=%.3g max|dlse|=%.3g" % (w.name, len(rows), e_out, e_lse))
    assert e_out <= TOL_BF16_OUT and e_lse <= TOL_BF16_LSE
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_rows_depend_only_on_their_own_sequence_bitwise():
    # Perturb one sequence (including NaN) and check every other row is bit-identical.
    lengths = [100, 257, 64, 3, 190]
    w, q, k, v, cu = varlen_case(lengths, 32, 8, 128, seed=12)
    out0, lse0 = run_fwd(q, k, v, cu, w.scale)
    a, b = int(cu[1]), int(cu[2])
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[a:b] = float("nan")
    k2[a:b] = 3.0
    v2[a:b] = float("nan")
    out1, lse1 = run_fwd(q2, k2, v2, cu, w.scale)
    keep = torch.ones(int(cu[-1]), dtype=torch.bool)
    keep[a:b] = False
    keep = keep.cuda()
    assert torch.equal(out0[keep].view(torch.int16), out1[keep].view(torch.int16))
    assert torch.equal(lse0[keep].view(torch.int32), lse1[keep].view(torch.int32))


def test_sequence_permutation_permutes_rows_bitwise():
    lengths = [100, 257, 64, 3, 190, 1]
    w, q, k, v, cu = varlen_case(lengths, 32, 8, 128, seed=13)
    out0, lse0 = run_fwd(q, k, v, cu, w.scale)
    perm = [4, 2, 0, 5, 1, 3]
    spans = [(int(cu[i]), int(cu[i + 1])) for i in range(len(lengths))]
    idx = np.concatenate([np.arange(*spans[p]) for p in perm])
    cu2 = synth.cu_seqlens([lengths[p] for p in perm])
    out1, lse1 = run_fwd(q[idx], k[idx], v[idx], cu2, w.scale)
    ig = torch.from_numpy(idx).cuda()
    assert torch.equal(out0[ig].view(torch.int16), out1.view(torch.int16))
    assert torch.equal(lse0[ig].view(torch.int32), lse1.view(torch.int32))


def many_lengths(n=150, seed=21):
    """n ragged sequences (empty ones included) with long ones at index 64 (the first sequence
    whose span the work queue reads from memory rather than from registers) and later on."""
    rng = np.random.default_rng(seed)
    lengths = [int(x) for x in rng.integers(0, 90, size=n)]
    lengths[64] = 700
    lengths[100] = 450
    lengths[n - 1] = 333
    for i in (3, 70, 120):
        lengths[i] = 0
    return lengths


def test_more_than_64_sequences_full():
    lengths = many_lengths()
    w, q, k, v, cu = varlen_case(lengths, 8, 2, 128, seed=22)
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale)
    out, lse = run_fwd(q, k, v, cu, w.scale)
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print("%d sequences, %d tokens: max|dout|=%.3g max|dlse|=%.3g" % (len(lengths), int(cu[-1]), e_out, e_lse))
    assert e_out <= TOL_BF16_OUT and e_lse <= TOL_BF16_LSE


@pytest.mark.parametrize("D", [128, 64])
def test_many_items_per_workgroup_full(D):
    # 300 short sequences at 32 query heads (8 head blocks, one queue per XCD): each queue holds
    # sum ceil(len / 64) ~ 450 items, at least 8 per workgroup on 256 CUs, so every workgroup
    # holds one item in reserve and issues the next item's first loads under its output stores.
    # Every row of every head against the oracle.
    rng = np.random.default_rng(31)
    lengths = [int(x) for x in rng.integers(1, 129, size=300)]
    lengths[7], lengths[150] = 0, 1
    w, q, k, v, cu = varlen_case(lengths, 32, 8, D, seed=31)
    items_per_queue = sum((n + 63) // 64 for n in lengths)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    reserve = items_per_queue >= 8 * max(1, cus // 8)
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale)
    out, lse = run_fwd(q, k, v, cu, w.scale)
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print("%d sequences, %d tokens, %d items per queue (reserve %s): max|dout|=%.3g max|dlse|=%.3g"
          % (len(lengths), int(cu[-1]), items_per_queue, reserve, e_out, e_lse))
    assert e_out <= TOL_BF16_OUT and e_lse <= TOL_BF16_LSE


@pytest.mark.parametrize("lengths", [[4096, 17, 0, 300], [4097, 5, 64]])
def test_work_queue_level_boundary_sampled(lengths):
    # with 4 query heads per key/value head an item spans 64 rows: a 4096-token sequence has 64
    # tile levels (the last that the per-lane level table holds), 4097 tokens have 65
    w, q, k, v, cu = varlen_case(lengths, 8, 2, 128, seed=23)
    out, lse = run_fwd(q, k, v, cu, w.scale)
    rows = sample_rows(cu, 7)
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    e_out, e_lse = max_abs(out[idx], ro), max_abs(lse[idx], rl)
    print("lengths=%s: %d sampled rows, max|dout|=%.3g max|dlse|=%.3g" % (lengths, len(rows), e_out, e_lse))
    assert e_out <= TOL_BF16_OUT and e_lse <= TOL_BF16_LSE
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()


def test_every_row_is_written_and_runs_are_deterministic():
    w, q, k, v, cu = varlen_case([5, 700, 64, 0, 129], 32, 8, 128, seed=14)
    qg, kg, vg = to_gpu(q, k, v)
    cug = torch.from_numpy(cu).cuda()
    out = torch.full_like(qg, float("nan"))
    lse = torch.full((qg.shape[0], 32), float("nan"), device="cuda")
    ops.hdp_attn_varlen_fwd(qg, kg, vg, cug, w.scale, out=out, lse=lse)
    out2, lse2 = ops.hdp_attn_varlen_fwd(qg, kg, vg, cug, w.scale)
    torch.cuda.synchronize()
    assert not torch.isnan(out.float()).any() and not torch.isnan(lse).any()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))


def test_empty_and_single_token_sequences():
    w, q, k, v, cu = varlen_case([0, 1, 0, 0, 1, 2, 0], 32, 8, 128, seed=15)
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale)
    out, lse = run_fwd(q, k, v, cu, w.scale)
    assert max_abs(out, ro) <= TOL_BF16_OUT and max_abs(lse, rl) <= TOL_BF16_LSE


# ------------------------------------------------------------------ ring chunks


CHUNK_CASES = [
    # (Lq, Lk, q_offset, kv_offset, causal)
    (200, 192, 0, 0, True),        # diagonal chunk
    (200, 192, 1000, 0, True),     # fully visible chunk
    (200, 192, 0, 500, True),      # chunk in the future: nothing visible
    (200, 192, 100, 150, True),    # partly visible, some rows empty
    (130, 70, 0, 1000, False),     # no mask
    (33, 65, 7, 3, True),          # ragged sizes
    (64, 0, 0, 0, True),           # empty chunk
]


@pytest.mark.parametrize("Lq,Lk,q_off,kv_off,causal", CHUNK_CASES)
@pytest.mark.parametrize("D", [128, 64])
def test_chunk_partial_full(Lq, Lk, q_off, kv_off, causal, D):
    H, Hkv = 32, 8
    rng = np.random.default_rng(21)
    q = synth.normal(rng, (Lq, H, D), "bf16")
    k = synth.normal(rng, (Lk, Hkv, D), "bf16")
    v = synth.normal(rng, (Lk, Hkv, D), "bf16")
    scale = 1 / math.sqrt(D)
    ro, rl = oracle.chunk_partial(q, k, v, q_off, kv_off, causal, scale)
    qg, kg, vg = to_gpu(q, k, v)
    o, lse = ops.hdp_attn_chunk_partial(qg, kg, vg, q_off, kv_off, causal, scale)
    torch.cuda.synchronize()
    assert max_abs(o, ro) <= TOL_BF16_OUT
    lse_close(lse, rl, TOL_BF16_LSE)


def test_ring_128k_share_merged_equals_full_causal_attention_sampled():
    # One rank's share of a 16-rank ring over a 131072-token sequence: its 8192 queries at
    # offset 122880 attend to 16 chunks of 8192 keys; merged partials = full causal attention.
    w = synth.ring_chunks_128k()
    q, k, v = synth.ring_tensors(w)
    qg, kg, vg = to_gpu(q, k, v)
    L = w.chunk_len
    acc_o, acc_l = ops.hdp_attn_chunk_partial(qg, kg[:L], vg[:L], w.q_offset, 0, True, w.scale)
    part_o = torch.empty_like(acc_o)
    part_l = torch.empty_like(acc_l)
    out_bf16 = torch.empty(acc_o.shape, dtype=torch.bfloat16, device="cuda")
    keep = {}
    for c in range(1, w.n_chunks):
        ops.hdp_attn_chunk_partial(qg, kg[c * L:(c + 1) * L], vg[c * L:(c + 1) * L], w.q_offset,
                                   c * L, True, w.scale, o_partial=part_o, lse=part_l)
        if c in (3, 15):
            keep[c] = (part_o.clone(), part_l.clone())
        ops.hdp_lse_merge(acc_o, acc_l, part_o, part_l,
                          out_bf16=out_bf16 if c == w.n_chunks - 1 else None)
    torch.cuda.synchronize()
    # every 8th row and both sides of every 64-row tile edge of the slice, all heads
    rows = boundary_rows(w.q_len, 8, extra=(1, 2))
    idx = torch.from_numpy(rows).cuda()
    ro, rl = oracle.chunk_partial(q, k, v, w.q_offset, 0, True, w.scale, rows=rows)
    e_o = max_abs(acc_o[idx], ro)
    e_b = max_abs(out_bf16[idx], ro)
    e_l = max_abs(acc_l[idx], rl)
    print("ring merged: rows=%d max|do|=%.3g max|dbf16|=%.3g max|dlse|=%.3g" % (len(rows), e_o, e_b, e_l))
    assert e_o <= TOL_BF16_OUT and e_b <= TOL_BF16_OUT and e_l <= TOL_BF16_LSE
    for c, (po, pl) in keep.items():
        co, cl = oracle.chunk_partial(q, k[c * L:(c + 1) * L], v[c * L:(c + 1) * L], w.q_offset,
                                      c * L, True, w.scale, rows=rows)
        assert max_abs(po[idx], co) <= TOL_BF16_OUT
        lse_close(pl[idx], cl, TOL_BF16_LSE)


# ------------------------------------------------------------------------ merge


@pytest.mark.parametrize("D", [64, 128])
def test_lse_merge_matches_oracle_including_empty_partials(D):
    L, H = 300, 4
    rng = np.random.default_rng(31)
    o1 = rng.standard_normal((L, H, D)).astype(np.float32)
    o2 = rng.standard_normal((L, H, D)).astype(np.float32)
    l1 = (rng.standard_normal((L, H)) * 5).astype(np.float32)
    l2 = (rng.standard_normal((L, H)) * 5).astype(np.float32)
    l1[:20] = -np.inf
    o1[:20] = 0
    l2[10:30] = -np.inf
    o2[10:30] = 0
    ro, rl = oracle.lse_merge(o1, l1, o2, l2)
    go, gl, po, pl = (torch.from_numpy(x).cuda() for x in (o1, l1, o2, l2))
    bf = torch.empty(go.shape, dtype=torch.bfloat16, device="cuda")
    ops.hdp_lse_merge(go, gl, po, pl, out_bf16=bf)
    torch.cuda.synchronize()
    assert max_abs(go, ro) <= 1e-5
    lse_close(gl, rl, 1e-5)
    ref_bf = torch.from_numpy(ro).float().to(torch.bfloat16).double().numpy()
    assert max_abs(bf, ref_bf) <= TOL_BF16_OUT
    assert not torch.isnan(go).any()


# ------------------------------------------------------------------ fused ring step


def ring_reference(q, k, v, q_off, pieces, causal, scale, rows=None):
    """The oracle's merge of the pieces' partials in ring order (fp64)."""
    acc_o = acc_l = None
    for ko, kl in pieces:
        o, l = oracle.chunk_partial(q, k[ko:ko + kl], v[ko:ko + kl], q_off, ko, causal, scale, rows=rows)
        if acc_o is None:
            acc_o, acc_l = o, l
        else:
            acc_o, acc_l = oracle.lse_merge(acc_o, acc_l, o, l)
    return acc_o, acc_l


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("Lq,q_off,pieces,causal", [
    (200, 300, [(0, 192), (192, 150), (342, 64)], True),    # past, diagonal-crossing, future-ish chunks
    (130, 0, [(0, 70), (70, 70), (500, 30)], True),         # rows with no key in some chunks, one empty chunk
    (77, 1000, [(0, 33), (33, 129)], False),                # no mask
    (64, 64, [(64, 64), (0, 64), (128, 0)], True),          # tile-exact, out of order, empty chunk
])
def test_chunk_merge_equals_partials_merged_by_the_oracle(Lq, q_off, pieces, causal, D):
    # The fused ring step merges each chunk's partial into the running result; starting from
    # lse_acc = -inf with garbage (NaN) in o_acc, the result must equal the oracle's partials
    # merged in the same order, and the bf16 copy must be that result rounded.
    H, Hkv = 8, 2
    rng = np.random.default_rng(170 + Lq)
    S = max(o + l for o, l in pieces)
    q = synth.normal(rng, (Lq, H, D), "bf16")
    k = synth.normal(rng, (S, Hkv, D), "bf16")
    v = synth.normal(rng, (S, Hkv, D), "bf16")
    scale = 1 / math.sqrt(D)
    qg, kg, vg = to_gpu(q, k, v)
    o_acc = torch.full((Lq, H, D), float("nan"), device="cuda")
    l_acc = torch.full((Lq, H), -float("inf"), device="cuda")
    ob = torch.empty((Lq, H, D), dtype=torch.bfloat16, device="cuda")
    for i, (ko, kl) in enumerate(pieces):
        ops.hdp_attn_chunk_merge(qg, kg[ko:ko + kl], vg[ko:ko + kl], q_off, ko, o_acc, l_acc, causal, scale,
                                 out_bf16=ob if i == len(pieces) - 1 else None)
    torch.cuda.synchronize()
    ro, rl = ring_reference(q, k, v, q_off, pieces, causal, scale)
    # rows that saw no key at all: 0 and -inf
    ro = np.where(np.isneginf(rl)[:, :, None], 0.0, ro)
    assert max_abs(o_acc, ro) <= TOL_BF16_OUT
    lse_close(l_acc, rl, TOL_BF16_LSE)
    assert max_abs(ob, ro) <= TOL_BF16_OUT
    assert torch.equal(ob.view(torch.int16), o_acc.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("D", [128, 64])
def test_chunk_modes_with_an_item_in_reserve_sampled(D):
    # A 20,000-row slice gives 313 row tiles per head block (one queue per XCD): at least 8 items
    # per workgroup, so the chunk and fused-merge kernels hold one item in reserve and issue the
    # next item's first loads under the current item's output (and merge) traffic.  One chunk
    # fully in the past, one crossing the slice's first rows (digest ring model, §3.2).
    H, Hkv, Lq, q_off = 32, 8, 20000, 20000
    pieces = [(0, 300), (19900, 400)]
    rng = np.random.default_rng(181 + D)
    S = max(o + l for o, l in pieces)
    q = synth.normal(rng, (Lq, H, D), "bf16")
    k = synth.normal(rng, (S, Hkv, D), "bf16")
    v = synth.normal(rng, (S, Hkv, D), "bf16")
    scale = 1 / math.sqrt(D)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert (Lq + 63) // 64 >= 8 * max(1, cus // 8)               # reserve mode in both kernels
    qg, kg, vg = to_gpu(q, k, v)
    rows = boundary_rows(Lq, 37, extra=(1, 2, 99, 100, 101))
    idx = torch.from_numpy(rows).cuda()
    # chunk partial (no merge) of the crossing chunk
    ko, kl = pieces[1]
    o, lse = ops.hdp_attn_chunk_partial(qg, kg[ko:ko + kl], vg[ko:ko + kl], q_off, ko, True, scale)
    # fused ring steps over both chunks
    o_acc = torch.full((Lq, H, D), float("nan"), device="cuda")
    l_acc = torch.full((Lq, H), -float("inf"), device="cuda")
    ob = torch.empty((Lq, H, D), dtype=torch.bfloat16, device="cuda")
    for i, (po, pl) in enumerate(pieces):
        ops.hdp_attn_chunk_merge(qg, kg[po:po + pl], vg[po:po + pl], q_off, po, o_acc, l_acc, True, scale,
                                 out_bf16=ob if i == len(pieces) - 1 else None)
    torch.cuda.synchronize()
    co, cl = oracle.chunk_partial(q, k[ko:ko + kl], v[ko:ko + kl], q_off, ko, True, scale, rows=rows)
    e_o, e_l = max_abs(o[idx], co), lse_close(lse[idx], cl, TOL_BF16_LSE)
    ro, rl = ring_reference(q, k, v, q_off, pieces, True, scale, rows=rows)
    e_m = max_abs(o_acc[idx], ro)
    e_ml = lse_close(l_acc[idx], rl, TOL_BF16_LSE)
    print("D=%d, %d sampled rows: partial max|do|=%.3g max|dlse|=%.3g; merged max|do|=%.3g max|dlse|=%.3g"
          % (D, len(rows), e_o, e_l, e_m, e_ml))
    assert e_o <= TOL_BF16_OUT and e_m <= TOL_BF16_OUT
    assert max_abs(ob[idx], ro) <= TOL_BF16_OUT


def test_chunk_merge_agrees_with_partial_then_merge():
    # Fused and unfused ring steps compute the same merge in a different arithmetic order.
    H, Hkv, D, Lq = 32, 8, 128, 300
    rng = np.random.default_rng(180)
    q = synth.normal(rng, (Lq, H, D), "bf16").cuda()
    k = synth.normal(rng, (900, Hkv, D), "bf16").cuda()
    v = synth.normal(rng, (900, Hkv, D), "bf16").cuda()
    scale = 1 / math.sqrt(D)
    pieces = [(0, 300), (300, 300), (600, 300)]
    a_o, a_l = ops.hdp_attn_chunk_partial(q, k[:300], v[:300], 600, 0, True, scale)
    b_o, b_l = a_o.clone(), a_l.clone()
    for ko, kl in pieces[1:]:
        po, pl = ops.hdp_attn_chunk_partial(q, k[ko:ko + kl], v[ko:ko + kl], 600, ko, True, scale)
        ops.hdp_lse_merge(a_o, a_l, po, pl)
        ops.hdp_attn_chunk_merge(q, k[ko:ko + kl], v[ko:ko + kl], 600, ko, b_o, b_l, True, scale)
    torch.cuda.synchronize()
    assert float((a_o - b_o).abs().max()) <= 1e-5
    assert float((a_l - b_l).abs().max()) <= 1e-5


def test_ring_128k_share_fused_merge_equals_full_causal_attention_sampled():
    # The ring share of the 128K sequence as 16 fused steps from an empty accumulator.
    w = synth.ring_chunks_128k()
    q, k, v = synth.ring_tensors(w)
    qg, kg, vg = to_gpu(q, k, v)
    L = w.chunk_len
    o_acc = torch.zeros((w.q_len, w.H, w.D), device="cuda")
    l_acc = torch.full((w.q_len, w.H), -float("inf"), device="cuda")
    ob = torch.empty((w.q_len, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    for c in range(w.n_chunks):
        ops.hdp_attn_chunk_merge(qg, kg[c * L:(c + 1) * L], vg[c * L:(c + 1) * L], w.q_offset, c * L, o_acc, l_acc,
                                 True, w.scale, out_bf16=ob if c == w.n_chunks - 1 else None)
    torch.cuda.synchronize()
    rows = boundary_rows(w.q_len, 16, extra=(1, 2))
    idx = torch.from_numpy(rows).cuda()
    ro, rl = oracle.chunk_partial(q, k, v, w.q_offset, 0, True, w.scale, rows=rows)
    e_o, e_b, e_l = max_abs(o_acc[idx], ro), max_abs(ob[idx], ro), max_abs(l_acc[idx], rl)
    print("fused ring: rows=%d max|do|=%.3g max|dbf16|=%.3g max|dlse|=%.3g" % (len(rows), e_o, e_b, e_l))
    assert e_o <= TOL_BF16_OUT and e_b <= TOL_BF16_OUT and e_l <= TOL_BF16_LSE
