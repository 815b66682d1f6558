"""GPU parity of the ring-chunk backward (hdp_attn_chunk_bwd) against the fp64 oracle.

Each case hands the same inputs to both sides: bf16 q/k/v/out/dO and fp32 lse (for the small
cases, the oracle's own forward of the slice over its chunks, rounded; at full size, the seeded
synthetic out/lse of synth.ring_bwd_tensors).  The GPU adds its result to fp32 accumulators,
which start at zero unless stated.  Those accumulators are never rounded to bf16, so the check
is a plain max-abs 2e-2 on every compared element.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import boundary_rows, fp32_close
from variable_length_attention_amd import ops, synth

pytestmark = pytest.mark.gpu


def bf16(rng, shape):
    return synth.normal(rng, shape, "bf16")


def run_gpu(q, k, v, q_off, kv_off, causal, scale, out, lse, do, init=None):
    Lq, H, D = q.shape
    Lk, Hkv = k.shape[0], k.shape[1]
    dq = torch.zeros((Lq, H, D), dtype=torch.float32, device="cuda")
    dk = torch.zeros((Lk, Hkv, D), dtype=torch.float32, device="cuda")
    dv = torch.zeros((Lk, Hkv, D), dtype=torch.float32, device="cuda")
    if init is not None:
        dq += init[0].cuda()
        dk += init[1].cuda()
        dv += init[2].cuda()
    ops.hdp_attn_chunk_bwd(q.cuda(), k.cuda(), v.cuda(), q_off, kv_off, out.cuda(), lse.cuda(),
                           do.cuda(), dq, dk, dv, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def slice_forward(q, k_all, v_all, q_off, causal, scale):
    """The slice's final out (bf16) and lse (fp32) over keys 0 .. len(k_all)-1 (oracle)."""
    o, l = oracle.chunk_partial(q, k_all, v_all, q_off, 0, causal, scale)
    return torch.from_numpy(o).to(torch.bfloat16), torch.from_numpy(l).to(torch.float32)


@pytest.mark.parametrize("Lq,Lk,q_off,kv_off,causal,H,Hkv,D", [
    (200, 200, 300, 300, True, 32, 8, 128),     # diagonal chunk
    (130, 170, 400, 100, True, 32, 8, 128),     # chunk wholly in the past: every pair visible
    (150, 170, 100, 60, True, 8, 2, 128),       # partly visible, offsets not tile aligned
    (70, 130, 0, 0, False, 4, 2, 128),          # non-causal
    (45, 97, 33, 10, True, 16, 2, 64),          # D = 64
    (64, 128, 64, 64, True, 6, 2, 128),         # tile-exact sizes
])
def test_chunk_backward_small_full(Lq, Lk, q_off, kv_off, causal, H, Hkv, D):
    rng = np.random.default_rng(70 + Lq)
    scale = 1 / math.sqrt(D)
    q, do = bf16(rng, (Lq, H, D)), bf16(rng, (Lq, H, D))
    k_all, v_all = bf16(rng, (kv_off + Lk, Hkv, D)), bf16(rng, (kv_off + Lk, Hkv, D))
    out, lse = slice_forward(q, k_all, v_all, q_off, causal, scale)
    k, v = k_all[kv_off:], v_all[kv_off:]
    dq, dk, dv = run_gpu(q, k, v, q_off, kv_off, causal, scale, out, lse, do)
    rq, rk, rv = oracle.chunk_bwd(q, k, v, q_off, kv_off, causal, scale, out, lse, do)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = fp32_close(g, r)
        print("Lq=%d Lk=%d q_off=%d kv_off=%d causal=%d %s: max %.3g" % (Lq, Lk, q_off, kv_off, causal, name, e))


def test_future_chunk_adds_nothing_and_accumulators_are_updated_in_place():
    rng = np.random.default_rng(77)
    Lq, Lk, H, Hkv, D = 96, 80, 8, 2, 128
    q, do, out = bf16(rng, (Lq, H, D)), bf16(rng, (Lq, H, D)), bf16(rng, (Lq, H, D))
    k, v = bf16(rng, (Lk, Hkv, D)), bf16(rng, (Lk, Hkv, D))
    lse = torch.from_numpy(rng.standard_normal((Lq, H), dtype=np.float32))
    init = (torch.from_numpy(rng.standard_normal((Lq, H, D), dtype=np.float32)),
            torch.from_numpy(rng.standard_normal((Lk, Hkv, D), dtype=np.float32)),
            torch.from_numpy(rng.standard_normal((Lk, Hkv, D), dtype=np.float32)))
    # chunk after the slice: every pair masked, the accumulators keep their values exactly
    dq, dk, dv = run_gpu(q, k, v, 0, Lq, True, 0.1, out, lse, do, init=init)
    for g, i in zip((dq, dk, dv), init):
        assert torch.equal(g.cpu(), i)
    # the same with rows that saw no key at all anywhere (lse = -inf, out = 0): still nothing added
    lse_empty = lse.clone()
    lse_empty[::3] = -float("inf")
    out_empty = out.clone()
    out_empty[::3] = 0
    dq, dk, dv = run_gpu(q, k, v, 0, Lq, True, 0.1, out_empty, lse_empty, do, init=init)
    for g, i in zip((dq, dk, dv), init):
        assert torch.equal(g.cpu(), i)
    # a visible chunk: result = initial value + this chunk's share
    q_off = 500
    k_all, v_all = bf16(rng, (q_off + Lq, Hkv, D)), bf16(rng, (q_off + Lq, Hkv, D))
    out2, lse2 = slice_forward(q, k_all, v_all, q_off, True, 0.1)
    k2, v2 = k_all[200:200 + Lk], v_all[200:200 + Lk]
    dq, dk, dv = run_gpu(q, k2, v2, q_off, 200, True, 0.1, out2, lse2, do, init=init)
    rq, rk, rv = oracle.chunk_bwd(q, k2, v2, q_off, 200, True, 0.1, out2, lse2, do)
    for g, r, i in ((dq, rq, init[0]), (dk, rk, init[1]), (dv, rv, init[2])):
        fp32_close(g.cpu() - i, r)


def test_rows_that_see_no_key_contribute_nothing():
    # keys start 40 positions after the slice: rows 0..39 see no key of this chunk (nor any other
    # here), so the forward gives them out = 0 and lse = -inf; the row tiles that hold them also
    # hold rows that do see keys, so they go through the kernel with every pair masked
    rng = np.random.default_rng(78)
    Lq, Lk, H, Hkv, D = 96, 80, 8, 2, 128
    q, do = bf16(rng, (Lq, H, D)), bf16(rng, (Lq, H, D))
    k, v = bf16(rng, (Lk, Hkv, D)), bf16(rng, (Lk, Hkv, D))
    o, l = oracle.chunk_partial(q, k, v, 0, 40, True, 0.1)
    assert np.isneginf(l[:40]).all() and np.isfinite(l[40:]).all()
    out = torch.from_numpy(o).to(torch.bfloat16)
    lse = torch.from_numpy(l).to(torch.float32)
    dq, dk, dv = run_gpu(q, k, v, 0, 40, True, 0.1, out, lse, do)
    rq, rk, rv = oracle.chunk_bwd(q, k, v, 0, 40, True, 0.1, out, lse, do)
    for g, r in ((dq, rq), (dk, rk), (dv, rv)):
        assert torch.isfinite(g).all()
        fp32_close(g.cpu(), r)
    assert (dq[:40] == 0).all()


def test_ring_of_chunks_sums_to_the_packed_backward():
    # One causal sequence of 384 tokens as 3 slices x 3 chunks: the GPU chunk backward summed
    # over chunks (dq) and slices (dk, dv) against the oracle's packed backward.
    rng = np.random.default_rng(78)
    S, H, Hkv, D = 384, 8, 2, 128
    scale = 1 / math.sqrt(D)
    q, k, v, do = bf16(rng, (S, H, D)), bf16(rng, (S, Hkv, D)), bf16(rng, (S, Hkv, D)), bf16(rng, (S, H, D))
    cu = np.array([0, S], dtype=np.int32)
    o, l = oracle.varlen_fwd(q, k, v, cu, scale)
    out, lse = torch.from_numpy(o).to(torch.bfloat16), torch.from_numpy(l).to(torch.float32)
    cuts = [0, 128, 256, 384]
    dq = torch.zeros((S, H, D), dtype=torch.float32, device="cuda")
    dk = torch.zeros((S, Hkv, D), dtype=torch.float32, device="cuda")
    dv = torch.zeros((S, Hkv, D), dtype=torch.float32, device="cuda")
    qg, kg, vg, dog, outg, lseg = (t.cuda() for t in (q, k, v, do, out, lse))
    for a, b in zip(cuts[:-1], cuts[1:]):
        for c, e in zip(cuts[:-1], cuts[1:]):
            ops.hdp_attn_chunk_bwd(qg[a:b], kg[c:e], vg[c:e], a, c, outg[a:b], lseg[a:b], dog[a:b],
                                   dq[a:b], dk[c:e], dv[c:e], causal=True, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.varlen_bwd(q, k, v, do, cu, scale)
    for g, r in ((dq, rq), (dk, rk), (dv, rv)):
        fp32_close(g, r)


@pytest.mark.parametrize("chunk", [15, 0, 14])
def test_chunk_backward_full_size_sampled(chunk):
    # The ring share's slice (8192 rows at 122880) against one 8192-key chunk: the diagonal
    # chunk (15), the first chunk (0) and its neighbour (14); sampled rows of dq, dk, dv.
    w = synth.ring_chunks_128k()
    q, k, v = synth.ring_tensors(w)
    out, lse, do = synth.ring_bwd_tensors(w)
    scale = 1 / math.sqrt(w.D)
    c0 = chunk * w.chunk_len
    kc, vc = k[c0:c0 + w.chunk_len], v[c0:c0 + w.chunk_len]
    dq, dk, dv = run_gpu(q, kc, vc, w.q_offset, c0, True, scale, out, lse, do)
    # every 32nd row, both sides of every 64-row tile edge and the last row
    qrows = boundary_rows(w.q_len, 32)
    krows = boundary_rows(w.chunk_len, 32)
    rq, rk, rv = oracle.chunk_bwd(q, kc, vc, w.q_offset, c0, True, scale, out, lse, do,
                                  qrows=qrows, krows=krows)
    iq, ik = torch.from_numpy(qrows).cuda(), torch.from_numpy(krows).cuda()
    for name, g, r in (("dq", dq[iq], rq), ("dk", dk[ik], rk), ("dv", dv[ik], rv)):
        e = fp32_close(g, r)
        print("chunk %d %s (%d rows): max %.3g" % (chunk, name, len(r), e))
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
