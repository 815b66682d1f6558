"""The seeded generators draw exactly the committed workloads (CPU).

tests/golden/lengths.json holds every named workload's sequence lengths, sizes and tensor
seed, written by tests/golden/make_lengths.py.  If the generators or numpy's random stream ever
change, this fails instead of silently changing what the parity tests and the benchmark run.
The mixes follow the length statistics of the research digest "ByteScale: Communication-
Efficient Scaling of LLM Training with a 2048K Context Length on 16384 GPUs" (§2 and Figure 1:
skewed lengths; §3.1: slices of at most C = 8K tokens packed by best fit; §2: ~32K-token
micro-batches about 10x apart in attention FLOPs).
"""
import json
import os
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_lengths  # noqa: E402
from variable_length_attention_amd import synth  # noqa: E402


def committed():
    with open(os.path.join(HERE, "golden", "lengths.json")) as f:
        return json.load(f)


def test_generators_reproduce_the_committed_workloads():
    assert make_lengths.workloads() == committed()


def test_workload_invariants():
    w = committed()
    # one rank's slice holds exactly C = 8192 tokens of whole sequences
    assert w["packed_slice_8k"]["tokens"] == 8192
    assert all(0 < s <= 8192 for s in w["packed_slice_8k"]["lengths"])
    # both micro-batches hold 32768 tokens; the long one is dominated by one 16K-32K sequence
    for name in ("microbatch_32k_long", "microbatch_32k_short"):
        assert w[name]["tokens"] == 32768
    assert 16384 <= w["microbatch_32k_long"]["lengths"][0] <= 32768
    assert max(w["microbatch_32k_short"]["lengths"]) <= 2048
    # the ring share: the last of 16 chunks of a 128K sequence
    r = w["ring_chunks_128k"]
    assert r["q_offset"] + r["q_len"] == r["n_chunks"] * r["chunk_len"] == 131072


def test_micro_batch_flop_spread_is_about_ten_times_or_more():
    # digest §2: equal-token micro-batches differ by about 10x in attention work
    w = committed()
    pairs = {n: sum(s * (s + 1) // 2 for s in w[n]["lengths"]) for n in ("microbatch_32k_long", "microbatch_32k_short")}
    ratio = pairs["microbatch_32k_long"] / pairs["microbatch_32k_short"]
    assert 9 <= ratio <= 20, ratio


@pytest.mark.parametrize("seed", [0, 5, 17])
def test_packed_slices_always_fill_capacity(seed):
    lengths = synth.packed_slice_lengths(seed)
    assert sum(lengths) == 8192 and all(s > 0 for s in lengths)
