"""GPU parity of the backward pass against the fp64 oracle, through the C ABI.

Tolerance: gradients are bf16 results, and a bf16 number is within half its ulp of the exact
value at best; gradient magnitudes reach 8-16 here, where that half ulp (0.03) alone exceeds
2e-2.  So each element must satisfy |gpu - oracle| <= 2e-2 + half a bf16 ulp of the oracle
value, and the mean error must stay below 2e-3.

The GPU backward consumes the GPU forward's out and lse (as a training step would); the oracle
differentiates its own fp64 forward.  Every case compares every element of dq, dk and dv, the
full-size ones included (the 8K packed slice and one whole 8192-token sequence).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16_LSE, TOL_BF16_OUT, grad_close, max_abs, to_gpu
from variable_length_attention_amd import ops, synth

pytestmark = pytest.mark.gpu


def run_fwd_bwd(w, q, k, v, do, cu):
    qg, kg, vg, dog = to_gpu(q, k, v, do)
    cug = torch.from_numpy(cu).cuda()
    out, lse = ops.hdp_attn_varlen_fwd(qg, kg, vg, cug, w.scale)
    dq, dk, dv = ops.hdp_attn_varlen_bwd(qg, kg, vg, out, lse, dog, cug, w.scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def case(lengths, H, Hkv, D, seed):
    w = synth.Workload("case", "varlen", H, Hkv, D, "bf16", list(lengths), seed)
    q, k, v, do = synth.varlen_tensors(w, with_dout=True)
    return w, q, k, v, do, synth.cu_seqlens(w.lengths)


@pytest.mark.parametrize("lengths,H,Hkv,D", [
    ([1, 17, 64, 65, 127, 200, 0, 33], 32, 8, 128),
    ([100, 3, 129], 8, 8, 64),
    ([70, 31, 160], 4, 2, 128),
    ([45, 90], 16, 2, 64),
    ([300], 6, 2, 128),
])
def test_backward_small_packs_full(lengths, H, Hkv, D):
    w, q, k, v, do, cu = case(lengths, H, Hkv, D, seed=40)
    dq, dk, dv = run_fwd_bwd(w, q, k, v, do, cu)
    rq, rk, rv = oracle.varlen_bwd(q, k, v, do, cu, w.scale)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = grad_close(g, r)
        print("lengths=%s H=%d Hkv=%d D=%d %s: max %.3g, beyond half-ulp %.3g, mean %.2g"
              % (lengths, H, Hkv, D, name, *e))


def test_failed_workspace_allocation_is_reported_and_the_next_call_recovers(monkeypatch):
    # HDP_TEST_FAIL_ALLOC makes the library's workspace allocator fail when the workspace has to
    # grow; releasing it first forces the growth.  The call must return HDP_ERR_HIP without
    # launching anything, and the next call, with allocation working again, must be correct.
    from variable_length_attention_amd import _lib
    w, q, k, v, do, cu = case([70, 31, 160], 4, 2, 128, seed=41)
    torch.cuda.synchronize()
    ops.hdp_release_workspace()
    monkeypatch.setenv("HDP_TEST_FAIL_ALLOC", "1")
    with pytest.raises(_lib.HdpError) as err:
        run_fwd_bwd(w, q, k, v, do, cu)
    assert err.value.status == _lib.HDP_ERR_HIP
    monkeypatch.delenv("HDP_TEST_FAIL_ALLOC")
    dq, dk, dv = run_fwd_bwd(w, q, k, v, do, cu)
    rq, rk, rv = oracle.varlen_bwd(q, k, v, do, cu, w.scale)
    for g, r in ((dq, rq), (dk, rk), (dv, rv)):
        grad_close(g, r)


def test_backward_more_than_64_sequences_full():
    # long sequences at index 64 and later: their spans come from memory in the work queue
    rng = np.random.default_rng(42)
    lengths = [int(x) for x in rng.integers(0, 70, size=130)]
    lengths[64], lengths[90], lengths[129] = 400, 260, 150
    lengths[5] = lengths[66] = 0
    w, q, k, v, do, cu = case(lengths, 8, 2, 128, seed=43)
    dq, dk, dv = run_fwd_bwd(w, q, k, v, do, cu)
    rq, rk, rv = oracle.varlen_bwd(q, k, v, do, cu, w.scale)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = grad_close(g, r)
        print("%d sequences %s: max %.3g, beyond half-ulp %.3g, mean %.2g" % (len(lengths), name, *e))


def test_backward_is_deterministic_and_isolated_per_sequence():
    lengths = [150, 64, 257]
    w, q, k, v, do, cu = case(lengths, 32, 8, 128, seed=41)
    a = run_fwd_bwd(w, q, k, v, do, cu)
    b = run_fwd_bwd(w, q, k, v, do, cu)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    # change the middle sequence: gradients of the other two are bit-identical
    s0, s1 = int(cu[1]), int(cu[2])
    q2, k2, v2, do2 = q.clone(), k.clone(), v.clone(), do.clone()
    q2[s0:s1] *= 2
    v2[s0:s1] = -v2[s0:s1]
    do2[s0:s1] += 1
    c = run_fwd_bwd(w, q2, k2, v2, do2, cu)
    keep = torch.ones(int(cu[-1]), dtype=torch.bool)
    keep[s0:s1] = False
    keep = keep.cuda()
    for x, y in zip(a, c):
        assert torch.equal(x[keep].view(torch.int16), y[keep].view(torch.int16))


@pytest.mark.parametrize("make", [synth.fwd_bwd_8k_slice, synth.fwd_bwd_8k_single])
def test_forward_backward_full_size_every_row(make):
    # Both 8K slices of the forward + backward workload (the packed slice and one whole 8192-token
    # sequence): every row and head of out, lse, dq and every key row of dk, dv against the
    # oracle, including the first key tiles of the longest sequences, which collect the most rows.
    w = make()
    q, k, v, do = synth.varlen_tensors(w, with_dout=True)
    cu = synth.cu_seqlens(w.lengths)
    qg, kg, vg, dog = to_gpu(q, k, v, do)
    cug = torch.from_numpy(cu).cuda()
    out, lse = ops.hdp_attn_varlen_fwd(qg, kg, vg, cug, w.scale)
    dq, dk, dv = ops.hdp_attn_varlen_bwd(qg, kg, vg, out, lse, dog, cug, w.scale)
    torch.cuda.synchronize()
    ro, rl = oracle.varlen_fwd(q, k, v, cu, w.scale)
    e_out, e_lse = max_abs(out, ro), max_abs(lse, rl)
    print("%s forward: all %d rows, max|dout|=%.3g max|dlse|=%.3g" % (w.name, int(cu[-1]), e_out, e_lse))
    assert e_out <= TOL_BF16_OUT and e_lse <= TOL_BF16_LSE
    del ro, rl
    rq, rk, rv = oracle.varlen_bwd(q, k, v, do, cu, w.scale)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        e = grad_close(g, r)
        print("%s %s (every row): max %.3g, beyond half-ulp %.3g, mean %.2g" % (w.name, name, *e))
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
