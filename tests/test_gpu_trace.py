"""GPU: the forward's workgroup and per-item timelines (measurement helpers hdp_set_trace and
hdp_set_item_trace) account for every work item exactly once.

The work items of the packed forward are the query-row tiles of every sequence times the head
blocks, each visiting the 32-key units up to its last row (causal); their cost grows with the
square of the sequence length (research digest "ByteScale: Communication-Efficient Scaling of LLM
Training with a 2048K Context Length on 16384 GPUs", §2, "Imbalanced computation"), which is
what the longest-first queue balances.  Whatever workgroup takes an item, the items recorded
over all workgroups must be exactly the items of the batch: their number and their units add up
to the host-side count, each record's timestamps are ordered, and the result is still correct.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16_LSE, TOL_BF16_OUT, lse_close, max_abs
from variable_length_attention_amd import ops, synth

pytestmark = pytest.mark.gpu

ROWS = 64           # query rows per item (256 row-heads over 4 query heads per item)
UNIT = 32           # keys per unit


def expected_items(lengths, H, heads_per_item=4):
    """Host count of the forward's items and their units (causal: up to the item's last row)."""
    units = []
    for L in lengths:
        for t in range(math.ceil(L / ROWS)):
            last_row = min(L, (t + 1) * ROWS) - 1
            units += [last_row // UNIT + 1] * (H // heads_per_item)
    return len(units), sum(units)


@pytest.mark.parametrize("lengths", [None, [1, 2, 63, 64, 65, 700, 5, 1500, 31, 128, 129]])
def test_item_trace_accounts_for_every_item_once(lengths):
    if lengths is None:
        w = synth.packed_slice_8k()
    else:
        w = synth.Workload("case", "varlen", 32, 8, 128, "bf16", list(lengths), 161)
    q, k, v = synth.varlen_tensors(w)
    cu = synth.cu_seqlens(w.lengths)
    qg, kg, vg, cug = q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(cu).cuda()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    slots = 64
    trace = torch.zeros(4 * n_cu, dtype=torch.int64, device="cuda")
    items = torch.zeros(4 * slots * n_cu, dtype=torch.int64, device="cuda")
    ops.hdp_set_trace(trace)
    ops.hdp_set_item_trace(items, slots)
    try:
        out, lse = ops.hdp_attn_varlen_fwd(qg, kg, vg, cug, w.scale)
        torch.cuda.synchronize()
    finally:
        ops.hdp_set_trace(None)
        ops.hdp_set_item_trace(None)
    t = trace.view(n_cu, 4).cpu().numpy()
    it = items.view(n_cu, slots, 4).cpu().numpy()
    n_items, n_units = expected_items(w.lengths, w.H)
    done = t[:, 2]
    assert done.max() <= slots
    assert int(done.sum()) == n_items
    got_units = 0
    for b in range(n_cu):
        n = int(done[b])
        assert t[b, 0] <= t[b, 1]
        for i in range(n):
            a0, a1, a2, nu = (int(x) for x in it[b, i])
            nxt = int(it[b, i + 1, 0]) if i + 1 < n else int(t[b, 1])
            assert t[b, 0] <= a0 <= a1 <= a2 <= nxt, (b, i)
            assert nu >= 1
            got_units += nu
        assert not it[b, n:].any()                 # nothing recorded past the items it ran
    assert got_units == n_units
    print("items %d units %d over %d workgroups (max %d per workgroup)" % (n_items, n_units, n_cu, done.max()))
    # the traced launch computed the right result (every 97th row checked on the slice)
    rows = np.arange(0, q.shape[0], 97 if lengths is None else 1)
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    assert max_abs(out[idx], ro) <= TOL_BF16_OUT
    lse_close(lse[idx], rl, TOL_BF16_LSE)


def test_backward_trace_is_ordered_and_changes_nothing():
    # the backward is deterministic: a traced call gives bit-identical gradients
    w = synth.Workload("case", "varlen", 32, 8, 128, "bf16", [700, 1, 65, 1300, 31], 162)
    q, k, v, do = synth.varlen_tensors(w, with_dout=True)
    cu = synth.cu_seqlens(w.lengths)
    qg, kg, vg, dg, cug = q.cuda(), k.cuda(), v.cuda(), do.cuda(), torch.from_numpy(cu).cuda()
    o, lse = ops.hdp_attn_varlen_fwd(qg, kg, vg, cug, w.scale)
    ref = ops.hdp_attn_varlen_bwd(qg, kg, vg, o, lse, dg, cug, w.scale)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    trace = torch.zeros(4 * n_cu, dtype=torch.int64, device="cuda")
    ops.hdp_set_trace(trace)
    try:
        got = ops.hdp_attn_varlen_bwd(qg, kg, vg, o, lse, dg, cug, w.scale)
        torch.cuda.synchronize()
    finally:
        ops.hdp_set_trace(None)
    t = trace.view(n_cu, 4).cpu().numpy()
    assert (t[:, 0] > 0).all()
    assert (t[:, 0] <= t[:, 1]).all() and (t[:, 1] <= t[:, 2]).all() and (t[:, 3] == 0).all()
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_item_trace_of_a_ring_chunk_counts_every_row_tile_once():
    # chunk mode: the items are the slice's 64-row tiles times the head blocks, whatever the chunk
    H, Hkv, D, Lq, Lk = 32, 8, 128, 1000, 300
    rng = np.random.default_rng(163)
    q = synth.normal(rng, (Lq, H, D), "bf16")
    k = synth.normal(rng, (Lk, Hkv, D), "bf16")
    v = synth.normal(rng, (Lk, Hkv, D), "bf16")
    scale = 1 / math.sqrt(D)
    qg, kg, vg = q.cuda(), k.cuda(), v.cuda()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    slots = 16
    trace = torch.zeros(4 * n_cu, dtype=torch.int64, device="cuda")
    items = torch.zeros(4 * slots * n_cu, dtype=torch.int64, device="cuda")
    ops.hdp_set_trace(trace)
    ops.hdp_set_item_trace(items, slots)
    try:
        o, lse = ops.hdp_attn_chunk_partial(qg, kg, vg, 5000, 0, True, scale)   # chunk wholly in the past
        torch.cuda.synchronize()
    finally:
        ops.hdp_set_trace(None)
        ops.hdp_set_item_trace(None)
    t = trace.view(n_cu, 4).cpu().numpy()
    it = items.view(n_cu, slots, 4).cpu().numpy()
    done = t[:, 2]
    assert int(done.sum()) == math.ceil(Lq / ROWS) * (H // 4)
    units = 0
    for b in range(n_cu):
        n = int(done[b])
        for i in range(n):
            a0, a1, a2, nu = (int(x) for x in it[b, i])
            nxt = int(it[b, i + 1, 0]) if i + 1 < n else int(t[b, 1])
            assert t[b, 0] <= a0 <= a1 <= a2 <= nxt
            units += nu
    # every key of the chunk is visible to every row: each item visits all ceil(Lk / 32) units
    assert units == int(done.sum()) * math.ceil(Lk / UNIT)
    rows = np.arange(0, Lq, 7)
    ro, rl = oracle.chunk_partial(q, k, v, 5000, 0, True, scale, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    assert max_abs(o[idx], ro) <= TOL_BF16_OUT
    lse_close(lse[idx], rl, TOL_BF16_LSE)
