"""GPU: a global batch planned by the host HDP planner, every unit run through the HIP calls.

The batch is the digest's Figure 2 example (research digest "ByteScale: Communication-Efficient
Scaling of LLM Training with a 2048K Context Length on 16384 GPUs", §3.1 and Figure 2: five
sequences of 32K, 16K, 8K, 4K and 4K tokens on ranks of C = 8K) scaled down to C = 512, so the
sequences are 2048, 1024, 512, 256 and 256 tokens.  hdp_plan_shard turns it into units of at
most C tokens; here every unit is run on the one GPU in turn:

* a packed unit (whole short sequences) runs hdp_attn_varlen_fwd / _bwd on its own slice;
* the units of a ring each run their query pieces against every piece of the ring with
  hdp_attn_chunk_partial, merged by hdp_lse_merge (digest §3.2, ring steps), and the backward
  with hdp_attn_chunk_bwd, dK/dV accumulated with the chunk they belong to.

Every sequence's out, lse, dq, dk and dv is then reassembled from the units and compared with
the oracle on that sequence alone: a wrong piece offset or length in the plan fails here.
Both the contiguous plan and the front/back paired plan (digest §4) are checked, and the
balance scheduler's rank assignment is checked to cover every unit once (digest §3.4).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16_LSE, TOL_BF16_OUT, fp32_close, grad_close, lse_close, max_abs
from variable_length_attention_amd import ops, synth

pytestmark = pytest.mark.gpu

C = 512
LENS = [2048, 1024, 512, 256, 256]
H, HKV, D = 8, 2, 128


def batch_tensors(seed=140):
    rng = np.random.default_rng(seed)
    out = []
    for s in LENS:
        out.append(tuple(synth.normal(rng, (s, h, D), "bf16") for h in (H, HKV, HKV, H)))
    return out   # per sequence: q, k, v, dO


@pytest.mark.parametrize("pair", [False, True])
def test_planned_batch_matches_the_oracle_per_sequence(pair):
    scale = 1 / math.sqrt(D)
    plan = ops.hdp_plan_shard(LENS, C, pair=pair)
    units = plan.units()
    # the plan covers every token of every sequence exactly once, in units of at most C tokens
    cover = [np.zeros(s, dtype=np.int32) for s in LENS]
    for ring, pieces in units:
        assert sum(pl for _, _, pl in pieces) <= C
        for sq, off, pl in pieces:
            cover[sq][off:off + pl] += 1
    assert all((c == 1).all() for c in cover)
    # the balance scheduler places every unit on one of 8 ranks, a ring's units on distinct ranks
    cost = ops.hdp_plan_unit_flops(plan, H, D)
    unit_rank, load = ops.hdp_plan_balance(cost, plan.ring, 8)
    assert len(unit_rank) == len(units) and all(0 <= r < 8 for r in unit_rank)
    for ring in set(plan.ring) - {-1}:
        ranks = [unit_rank[j] for j in range(len(units)) if plan.ring[j] == ring]
        assert len(set(ranks)) == len(ranks)
    assert sum(load) == sum(cost)

    data = batch_tensors()
    dev = [tuple(t.cuda() for t in x) for x in data]
    res_out = [torch.zeros((s, H, D), dtype=torch.float32, device="cuda") for s in LENS]
    res_lse = [torch.full((s, H), float("nan"), dtype=torch.float32, device="cuda") for s in LENS]
    res_dq = [torch.zeros((s, H, D), dtype=torch.float32, device="cuda") for s in LENS]
    res_dk = [torch.zeros((s, HKV, D), dtype=torch.float32, device="cuda") for s in LENS]
    res_dv = [torch.zeros((s, HKV, D), dtype=torch.float32, device="cuda") for s in LENS]
    bf16_grads = set()

    # packed units: gather the unit's sequences into one slice, forward + backward, scatter back
    for ring, pieces in units:
        if ring >= 0:
            continue
        seqs = [sq for sq, _, _ in pieces]
        assert all(off == 0 and pl == LENS[sq] for sq, off, pl in pieces)
        q, k, v, do = (torch.cat([dev[sq][i] for sq in seqs]) for i in range(4))
        cu = torch.from_numpy(synth.cu_seqlens([LENS[sq] for sq in seqs])).cuda()
        out, lse = ops.hdp_attn_varlen_fwd(q, k, v, cu, scale)
        dq, dk, dv = ops.hdp_attn_varlen_bwd(q, k, v, out, lse, do, cu, scale)
        a = 0
        for sq in seqs:
            b = a + LENS[sq]
            res_out[sq].copy_(out[a:b].float())
            res_lse[sq].copy_(lse[a:b])
            res_dq[sq].copy_(dq[a:b].float())
            res_dk[sq].copy_(dk[a:b].float())
            res_dv[sq].copy_(dv[a:b].float())
            bf16_grads.add(sq)
            a = b

    # rings: each unit's query pieces against every piece of its ring
    for ring in sorted(set(plan.ring) - {-1}):
        ring_pieces = [p for r, ps in units if r == ring for p in ps]
        q, k, v, do = dev[ring]
        merged = []
        for _, qo, ql in ring_pieces:
            acc_o = torch.zeros((ql, H, D), dtype=torch.float32, device="cuda")
            acc_l = torch.full((ql, H), -float("inf"), dtype=torch.float32, device="cuda")
            for _, ko, kl in ring_pieces:
                o, l = ops.hdp_attn_chunk_partial(q[qo:qo + ql], k[ko:ko + kl], v[ko:ko + kl], qo, ko,
                                                  True, scale)
                ops.hdp_lse_merge(acc_o, acc_l, o, l)
            res_out[ring][qo:qo + ql] = acc_o
            res_lse[ring][qo:qo + ql] = acc_l
            merged.append((qo, ql, acc_o.to(torch.bfloat16), acc_l))
        for qo, ql, out_b, lse_s in merged:
            for _, ko, kl in ring_pieces:
                ops.hdp_attn_chunk_bwd(q[qo:qo + ql], k[ko:ko + kl], v[ko:ko + kl], qo, ko, out_b, lse_s,
                                       do[qo:qo + ql], res_dq[ring][qo:qo + ql], res_dk[ring][ko:ko + kl],
                                       res_dv[ring][ko:ko + kl], causal=True, scale=scale)
    torch.cuda.synchronize()

    for sq, s in enumerate(LENS):
        q, k, v, do = data[sq]
        cu = np.array([0, s], dtype=np.int32)
        ro, rl = oracle.varlen_fwd(q, k, v, cu, scale)
        e_o = max_abs(res_out[sq], ro)
        assert e_o <= TOL_BF16_OUT, (sq, e_o)
        lse_close(res_lse[sq], rl, TOL_BF16_LSE)
        rq, rk, rv = oracle.varlen_bwd(q, k, v, do, cu, scale)
        for name, g, r in (("dq", res_dq[sq], rq), ("dk", res_dk[sq], rk), ("dv", res_dv[sq], rv)):
            if sq in bf16_grads:
                grad_close(g, r)          # bf16 results of the packed backward
            else:
                fp32_close(g, r)          # fp32 ring accumulators
        print("pair=%d sequence %d (%d tokens, %s): max|dout|=%.3g" % (pair, sq, s,
              "packed" if sq in bf16_grads else "ring", e_o))
