"""GPU: the no-allocation backward entry point against the allocating one, through the C ABI.

hdp_attn_varlen_bwd_noalloc runs the same kernels as hdp_attn_varlen_bwd with their scratch in a
fixed device array of the library, so its dq, dk and dv must equal hdp_attn_varlen_bwd's bit for
bit.  Two calls in a row, the second on a smaller pack, check that the array's leftover contents
from the first call never leak into the second.
"""
import ctypes

import numpy as np
import pytest
import torch

from variable_length_attention_amd import _lib, ops, synth

pytestmark = pytest.mark.gpu


def noalloc_bwd(q, k, v, out, lse, do, cu, scale):
    T, H, D = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = _lib.lib().hdp_attn_varlen_bwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), do.data_ptr(),
        cu.data_ptr(), cu.numel() - 1, T, H, Hkv, D, float(scale), dq.data_ptr(), dk.data_ptr(),
        dv.data_ptr(), torch.cuda.current_stream().cuda_stream)
    _lib.check("hdp_attn_varlen_bwd_noalloc", st)
    return dq, dk, dv


def bits(t):
    return t.view(torch.int16)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_backward_equals_the_allocating_entry_point(order):
    cases = [([541, 268, 1935, 3421, 417, 826, 361, 388, 35], 32, 8, 128, 160),
             ([300, 17, 129, 0, 64], 32, 8, 128, 161)]
    for lengths, H, Hkv, D, seed in cases:
        print("noalloc case: lengths=%s H=%d Hkv=%d D=%d seed=%d" % (lengths, H, Hkv, D, seed), flush=True)
        w = synth.Workload("case", "varlen", H, Hkv, D, "bf16", lengths, seed)
        q, k, v, do = (t.cuda() for t in synth.varlen_tensors(w, with_dout=True))
        cu = torch.from_numpy(synth.cu_seqlens(lengths)).cuda()
        out, lse = ops.hdp_attn_varlen_fwd(q, k, v, cu, w.scale)
        want = ops.hdp_attn_varlen_bwd(q, k, v, out, lse, do, cu, w.scale)
        got = noalloc_bwd(q, k, v, out, lse, do, cu, w.scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, want):
            assert torch.equal(bits(a), bits(b)), name
            assert torch.isfinite(a.float()).all(), name
