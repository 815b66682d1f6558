"""Writes lengths.json: the sequence-length lists the seeded generators draw for every named
workload.  These are inputs, not expected results; the file pins them so that a change in the
generators (or in numpy's random stream) shows up as a failing CPU test instead of silently
changing what the parity tests and the benchmark measure.

Run from the repository root: python tests/golden/make_lengths.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from variable_length_attention_amd import synth  # noqa: E402


def workloads():
    out = {}
    for make in (synth.tiny_fp32_pack, synth.packed_slice_8k, synth.microbatch_32k_long,
                 synth.microbatch_32k_short, synth.fwd_bwd_8k_slice, synth.fwd_bwd_8k_single):
        w = make()
        out[w.name] = {"lengths": list(w.lengths), "tokens": sum(w.lengths), "H": w.H, "Hkv": w.Hkv,
                       "D": w.D, "dtype": w.dtype, "tensor_seed": w.tensor_seed}
    w = synth.ring_chunks_128k()
    out[w.name] = {"q_len": w.q_len, "q_offset": w.q_offset, "n_chunks": w.n_chunks,
                   "chunk_len": w.chunk_len, "H": w.H, "Hkv": w.Hkv, "D": w.D, "dtype": w.dtype,
                   "tensor_seed": w.tensor_seed}
    return out


if __name__ == "__main__":
    with open(os.path.join(HERE, "lengths.json"), "w") as f:
        json.dump(workloads(), f, indent=1)
        f.write("\n")
