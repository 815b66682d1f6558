"""GPU: calls on two streams at once, and guard bands around every output.

Two streams.  The library keeps its work-queue counters and backward workspace per stream, so
two calls in flight on two streams of one device (both at the default priority) must not
disturb each other: each result is compared with the oracle.  (A ring step of the research
digest "ByteScale: Communication-Efficient Scaling of LLM Training with a 2048K Context Length on
16384 GPUs", §3.2, computes on one slice while another is in hand; a training loop overlaps such
work with the packed slices of other sequences.)

Guard bands.  Every output is placed inside a larger buffer whose bytes before and after it
hold a sentinel pattern; after the forward, backward, chunk, chunk-backward and merge calls the
bands must be untouched, on ragged sizes where the last tiles reach past the data.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16_LSE, TOL_BF16_OUT, grad_close, lse_close, max_abs
from variable_length_attention_amd import ops, synth

pytestmark = pytest.mark.gpu


def case(lengths, H, Hkv, D, seed):
    w = synth.Workload("case", "varlen", H, Hkv, D, "bf16", list(lengths), seed)
    q, k, v, do = synth.varlen_tensors(w, with_dout=True)
    return w, q, k, v, do, synth.cu_seqlens(w.lengths)


def test_forward_and_backward_on_two_streams_at_once():
    # stream 1: a 4K-dominated pack (long items); stream 2: many short sequences, launched
    # repeatedly so that their kernels run while stream 1's are still in flight
    wa, qa, ka, va, da, cua = case([4000, 300, 129, 17], 32, 8, 128, seed=150)
    wb, qb, kb, vb, db, cub = case([100, 3, 257, 64, 512, 1, 90], 32, 8, 128, seed=151)
    ga = [t.cuda() for t in (qa, ka, va, da)] + [torch.from_numpy(cua).cuda()]
    gb = [t.cuda() for t in (qb, kb, vb, db)] + [torch.from_numpy(cub).cuda()]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    res_b = []
    with torch.cuda.stream(s1):
        oa, la = ops.hdp_attn_varlen_fwd(ga[0], ga[1], ga[2], ga[4], wa.scale)
        dqa, dka, dva = ops.hdp_attn_varlen_bwd(ga[0], ga[1], ga[2], oa, la, ga[3], ga[4], wa.scale)
    with torch.cuda.stream(s2):
        for _ in range(4):
            ob, lb = ops.hdp_attn_varlen_fwd(gb[0], gb[1], gb[2], gb[4], wb.scale)
            dqb, dkb, dvb = ops.hdp_attn_varlen_bwd(gb[0], gb[1], gb[2], ob, lb, gb[3], gb[4], wb.scale)
            res_b.append((ob, lb, dqb, dkb, dvb))
    torch.cuda.synchronize()
    ro, rl = oracle.varlen_fwd(qa, ka, va, cua, wa.scale)
    assert max_abs(oa, ro) <= TOL_BF16_OUT and max_abs(la, rl) <= TOL_BF16_LSE
    rq, rk, rv = oracle.varlen_bwd(qa, ka, va, da, cua, wa.scale)
    for g, r in ((dqa, rq), (dka, rk), (dva, rv)):
        grad_close(g, r)
    ro, rl = oracle.varlen_fwd(qb, kb, vb, cub, wb.scale)
    rq, rk, rv = oracle.varlen_bwd(qb, kb, vb, db, cub, wb.scale)
    for ob, lb, dqb, dkb, dvb in res_b:
        assert max_abs(ob, ro) <= TOL_BF16_OUT and max_abs(lb, rl) <= TOL_BF16_LSE
        for g, r in ((dqb, rq), (dkb, rk), (dvb, rv)):
            grad_close(g, r)
    # every repetition on stream 2 is bit-identical (each ran with its stream's own counters)
    for x in res_b[1:]:
        for a, b in zip(x, res_b[0]):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


BAND = 4096   # elements of sentinel before and after each output


class Guarded:
    """An output tensor of `shape` inside a flat buffer with BAND sentinel elements on each side."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape))
        self.buf = torch.empty(n + 2 * BAND, dtype=dtype, device="cuda")
        self.buf.view(torch.uint8).fill_(0xA5)
        self.ref = self.buf[:BAND].clone()
        self.t = self.buf[BAND:BAND + n].view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self, what):
        torch.cuda.synchronize()
        lo, hi = self.buf[:BAND], self.buf[-BAND:]
        assert torch.equal(lo.view(torch.uint8), self.ref.view(torch.uint8)), what + ": band before written"
        assert torch.equal(hi.view(torch.uint8), self.ref.view(torch.uint8)), what + ": band after written"


@pytest.mark.parametrize("D", [128, 64])
def test_outputs_never_write_outside_their_buffers(D):
    H, Hkv = 8, 2
    lengths = [1, 33, 0, 130, 65]
    w, q, k, v, do, cu = case(lengths, H, Hkv, D, seed=152)
    T = int(cu[-1])
    qg, kg, vg, dg = (t.cuda() for t in (q, k, v, do))
    cug = torch.from_numpy(cu).cuda()
    out = Guarded((T, H, D), torch.bfloat16)
    lse = Guarded((T, H), torch.float32)
    ops.hdp_attn_varlen_fwd(qg, kg, vg, cug, w.scale, out=out.t, lse=lse.t)
    out.check("varlen fwd out")
    lse.check("varlen fwd lse")
    dq, dk, dv = Guarded((T, H, D), torch.bfloat16), Guarded((T, Hkv, D), torch.bfloat16), Guarded((T, Hkv, D), torch.bfloat16)
    ops.hdp_attn_varlen_bwd(qg, kg, vg, out.t, lse.t, dg, cug, w.scale, dq=dq.t, dk=dk.t, dv=dv.t)
    for g, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        g.check("varlen bwd " + n)
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale)
    assert max_abs(out.t, ro) <= TOL_BF16_OUT
    # the fp32 form on the same pack
    qf, kf, vf = (t.float().cuda() for t in (q, k, v))
    out32 = Guarded((T, H, D), torch.float32)
    lse32 = Guarded((T, H), torch.float32)
    ops.hdp_attn_varlen_fwd_f32(qf, kf, vf, cug, w.scale, out=out32.t, lse=lse32.t)
    out32.check("fp32 fwd out")
    lse32.check("fp32 fwd lse")
    assert max_abs(out32.t, ro) <= 1e-5

    # ring step, its merge and its backward on ragged sizes
    Lq, Lk, q_off, kv_off = 77, 45, 60, 20
    rng = np.random.default_rng(153)
    qs, kc, vc, ds = (synth.normal(rng, shp, "bf16") for shp in ((Lq, H, D), (Lk, Hkv, D), (Lk, Hkv, D), (Lq, H, D)))
    qs_g, kc_g, vc_g, ds_g = (t.cuda() for t in (qs, kc, vc, ds))
    o_p = Guarded((Lq, H, D), torch.float32)
    l_p = Guarded((Lq, H), torch.float32)
    ops.hdp_attn_chunk_partial(qs_g, kc_g, vc_g, q_off, kv_off, True, 1 / math.sqrt(D), o_partial=o_p.t, lse=l_p.t)
    o_p.check("chunk partial o")
    l_p.check("chunk partial lse")
    co, cl = oracle.chunk_partial(qs, kc, vc, q_off, kv_off, True, 1 / math.sqrt(D))
    assert max_abs(o_p.t, co) <= TOL_BF16_OUT
    lse_close(l_p.t, cl, TOL_BF16_LSE)
    acc_o = Guarded((Lq, H, D), torch.float32, fill=o_p.t)
    acc_l = Guarded((Lq, H), torch.float32, fill=l_p.t)
    ob = Guarded((Lq, H, D), torch.bfloat16)
    ops.hdp_lse_merge(acc_o.t, acc_l.t, o_p.t, l_p.t, out_bf16=ob.t)
    for g, n in ((acc_o, "o_acc"), (acc_l, "lse_acc"), (ob, "out_bf16")):
        g.check("merge " + n)
    dq_a = Guarded((Lq, H, D), torch.float32, fill=torch.zeros((Lq, H, D), device="cuda"))
    dk_a = Guarded((Lk, Hkv, D), torch.float32, fill=torch.zeros((Lk, Hkv, D), device="cuda"))
    dv_a = Guarded((Lk, Hkv, D), torch.float32, fill=torch.zeros((Lk, Hkv, D), device="cuda"))
    ops.hdp_attn_chunk_bwd(qs_g, kc_g, vc_g, q_off, kv_off, o_p.t.to(torch.bfloat16), l_p.t, ds_g,
                           dq_a.t, dk_a.t, dv_a.t, causal=True, scale=1 / math.sqrt(D))
    for g, n in ((dq_a, "dq_acc"), (dk_a, "dk_acc"), (dv_a, "dv_acc")):
        g.check("chunk bwd " + n)


def test_wrappers_reject_mis_shaped_tensors_before_launching():
    w, q, k, v, do, cu = case([40, 9], 8, 2, 128, seed=154)
    qg, kg, vg = (t.cuda() for t in (q, k, v))
    cug = torch.from_numpy(cu).cuda()
    with pytest.raises(ValueError):
        ops.hdp_attn_varlen_fwd(qg, kg[:10], vg, cug, w.scale)
    with pytest.raises(ValueError):
        ops.hdp_attn_varlen_fwd(qg, kg, vg, cug, w.scale, out=torch.empty_like(qg)[:5])
    o, l = ops.hdp_attn_chunk_partial(qg, kg, vg, 0, 0, True, w.scale)
    with pytest.raises(ValueError):
        ops.hdp_lse_merge(o, l, o[:3], l)
    with pytest.raises(ValueError):
        ops.hdp_attn_chunk_partial(qg, kg, vg[:, :1], 0, 0, True, w.scale)
    out, lse = ops.hdp_attn_varlen_fwd(qg, kg, vg, cug, w.scale)
    with pytest.raises(ValueError):
        ops.hdp_attn_varlen_bwd(qg, kg, vg, out, lse[:4], qg, cug, w.scale)
    torch.cuda.synchronize()


def test_validation_mode_rejects_malformed_cu_seqlens(monkeypatch):
    # With HDP_VALIDATE set the library reads cu_seqlens back to the host and rejects a pack
    # whose offsets do not start at 0, decrease, or (backward) run past the caller's T rows.
    from variable_length_attention_amd import _lib
    w, q, k, v, do, cu = case([40, 9, 30], 8, 2, 128, seed=155)
    qg, kg, vg, dg = (t.cuda() for t in (q, k, v, do))
    monkeypatch.setenv("HDP_VALIDATE", "1")
    good = torch.from_numpy(cu).cuda()
    out, lse = ops.hdp_attn_varlen_fwd(qg, kg, vg, good, w.scale)
    ops.hdp_attn_varlen_bwd(qg, kg, vg, out, lse, dg, good, w.scale)
    torch.cuda.synchronize()
    for bad in ([1, 40, 49, 79], [0, 40, 30, 79]):
        with pytest.raises(_lib.HdpError) as err:
            ops.hdp_attn_varlen_fwd(qg, kg, vg, torch.tensor(bad, dtype=torch.int32, device="cuda"), w.scale)
        assert err.value.status == _lib.HDP_ERR_INVALID_ARG
    with pytest.raises(_lib.HdpError) as err:   # 80 rows claimed, 79 given
        ops.hdp_attn_varlen_bwd(qg, kg, vg, out, lse, dg, torch.tensor([0, 40, 49, 80], dtype=torch.int32,
                                                                        device="cuda"), w.scale)
    assert err.value.status == _lib.HDP_ERR_INVALID_ARG
    monkeypatch.delenv("HDP_VALIDATE")
