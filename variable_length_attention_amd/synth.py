"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws sequence lengths and normally
distributed tensors.  The length mixes stand in for the datasets the pages measure on, which
are not available here; they follow the statistics the pages give:

* Digest §2 / Figure 1: lengths are heavily skewed; most samples are short (the blog summary
  of the same paper gives 80% of samples at or below 4K tokens), while a few long ones hold a
  large share of the tokens.
* Digest §3.1: a rank holds at most C tokens; sequences no longer than C are packed onto one
  rank by best fit.
* Digest §2: ~32K-token micro-batches randomly packed from the same data differ about 10x in
  attention FLOPs.

("Digest" = the research-digest page "ByteScale: Communication-Efficient Scaling of LLM
Training with a 2048K Context Length on 16384 GPUs".)

Values are float32 draws from ``numpy.random.default_rng`` rounded to bf16 (round to nearest
even) where the workload is bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

MAX_FILL_DRAWS = 4096


def log_uniform(rng: np.random.Generator, lo: int, hi: int) -> int:
    """round(exp(U(ln lo, ln hi)))."""
    return int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))


def best_fit_fill(rng: np.random.Generator, rem: int, lo: int, draw) -> List[int]:
    """Fill ``rem`` tokens: draw lengths, keep each one that still fits, skip the rest; stop
    when fewer than ``lo`` tokens remain (or after MAX_FILL_DRAWS draws); the remainder, if any,
    becomes the last sequence so the slice holds exactly ``rem`` tokens."""
    out: List[int] = []
    for _ in range(MAX_FILL_DRAWS):
        if rem < lo:
            break
        s = draw()
        if s <= rem:
            out.append(s)
            rem -= s
    if rem > 0:
        out.append(rem)
    return out


def packed_slice_lengths(seed: int = 0, capacity: int = 8192) -> List[int]:
    """One rank's slice of ``capacity`` tokens: each draw is log-uniform in [256, 4096] with
    probability 0.8, else log-uniform in [4096, 8192]; packed to exactly ``capacity``."""
    rng = np.random.default_rng(seed)

    def draw():
        if rng.random() < 0.8:
            return log_uniform(rng, 256, 4096)
        return log_uniform(rng, 4096, 8192)

    return best_fit_fill(rng, capacity, 256, draw)


def microbatch_long_lengths(seed: int = 1, tokens: int = 32768) -> List[int]:
    """A micro-batch dominated by one sequence of 16K-32K tokens, the rest short (128-2K)."""
    rng = np.random.default_rng(seed)
    first = log_uniform(rng, 16384, 32768)
    rest = best_fit_fill(rng, tokens - first, 128, lambda: log_uniform(rng, 128, 2048))
    return [first] + rest


def microbatch_short_lengths(seed: int = 2, tokens: int = 32768) -> List[int]:
    """A micro-batch of many short sequences (128-2K tokens, log-uniform)."""
    rng = np.random.default_rng(seed)
    return best_fit_fill(rng, tokens, 128, lambda: log_uniform(rng, 128, 2048))


def cu_seqlens(lengths: List[int]) -> np.ndarray:
    """Exclusive prefix sum with a leading 0, int32."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu.astype(np.int32)


def normal(rng: np.random.Generator, shape, dtype: str):
    """Standard-normal float32 draws as a CPU torch tensor of ``dtype`` ('bf16' or 'f32')."""
    import torch

    x = torch.from_numpy(rng.standard_normal(size=shape, dtype=np.float32))
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


@dataclass
class Workload:
    """A named synthetic workload: shapes, dtype and how to draw its tensors."""
    name: str
    kind: str                      # "varlen" or "ring"
    H: int
    Hkv: int
    D: int
    dtype: str
    lengths: List[int] = field(default_factory=list)
    tensor_seed: int = 0
    # ring workloads
    q_len: int = 0
    q_offset: int = 0
    n_chunks: int = 0
    chunk_len: int = 0
    backward: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def tokens(self) -> int:
        return sum(self.lengths) if self.kind == "varlen" else self.q_len


def tiny_fp32_pack() -> Workload:
    """4 sequences (17, 64, 100, 75 tokens), H = Hkv = 4, D = 64, fp32, tensors from seed 0."""
    return Workload("tiny_fp32_pack_256", "varlen", 4, 4, 64, "f32", [17, 64, 100, 75], 0)


def packed_slice_8k(seed: int = 0) -> Workload:
    """One rank's 8192-token slice of skewed-length sequences; GQA 32/8 heads, D = 128, bf16."""
    return Workload("packed_slice_8k", "varlen", 32, 8, 128, "bf16",
                    packed_slice_lengths(seed), seed + 1000)


def microbatch_32k_long(seed: int = 1) -> Workload:
    return Workload("microbatch_32k_long", "varlen", 32, 8, 128, "bf16",
                    microbatch_long_lengths(seed), seed + 1000)


def microbatch_32k_short(seed: int = 2) -> Workload:
    return Workload("microbatch_32k_short", "varlen", 32, 8, 128, "bf16",
                    microbatch_short_lengths(seed), seed + 1000)


def ring_chunks_128k(seed: int = 3) -> Workload:
    """8192 query tokens at offset 122880 of a 131072-token causal sequence against 16 K/V
    chunks of 8192 tokens (one rank's share of a 16-rank ring)."""
    return Workload("ring_chunks_128k", "ring", 32, 8, 128, "bf16", [], seed + 1000,
                    q_len=8192, q_offset=122880, n_chunks=16, chunk_len=8192)


def fwd_bwd_8k_slice(seed: int = 0) -> Workload:
    """The packed 8K slice, forward and backward."""
    w = packed_slice_8k(seed)
    w.name = "fwd_bwd_packed_slice_8k"
    w.backward = True
    w.tensor_seed = 4 + 1000
    return w


def fwd_bwd_8k_single() -> Workload:
    """One whole 8192-token sequence, forward and backward."""
    return Workload("fwd_bwd_single_8k", "varlen", 32, 8, 128, "bf16", [8192], 4 + 1000,
                    backward=True)


def varlen_tensors(w: Workload, with_dout: bool = False):
    """Draw q [T,H,D], k/v [T,Hkv,D] (and dO [T,H,D]) as CPU torch tensors, in that order."""
    T = sum(w.lengths)
    rng = np.random.default_rng(w.tensor_seed)
    q = normal(rng, (T, w.H, w.D), w.dtype)
    k = normal(rng, (T, w.Hkv, w.D), w.dtype)
    v = normal(rng, (T, w.Hkv, w.D), w.dtype)
    if not with_dout:
        return q, k, v
    do = normal(rng, (T, w.H, w.D), w.dtype)
    return q, k, v, do


def ring_tensors(w: Workload, rng_seed: Optional[int] = None):
    """q slice [q_len,H,D] and the whole key/value sequence [n_chunks*chunk_len,Hkv,D]."""
    rng = np.random.default_rng(w.tensor_seed if rng_seed is None else rng_seed)
    L = w.n_chunks * w.chunk_len
    q = normal(rng, (w.q_len, w.H, w.D), w.dtype)
    k = normal(rng, (L, w.Hkv, w.D), w.dtype)
    v = normal(rng, (L, w.Hkv, w.D), w.dtype)
    return q, k, v


def ring_bwd_tensors(w: Workload, seed: int = 5):
    """Backward inputs of a ring share that do not come from any forward: out [q_len,H,D] and dO
    [q_len,H,D] standard normal (bf16), and lse [q_len,H] = ln(number of keys the row sees over
    the whole sequence) + 0.5, the lse of standard-normal scores at unit scale, so exp(x - lse)
    stays near 1/count."""
    import torch

    rng = np.random.default_rng(seed + 1000)
    out = normal(rng, (w.q_len, w.H, w.D), w.dtype)
    dout = normal(rng, (w.q_len, w.H, w.D), w.dtype)
    count = np.arange(w.q_len, dtype=np.float64) + w.q_offset + 1
    lse = torch.from_numpy(np.repeat((np.log(count) + 0.5)[:, None], w.H, axis=1).astype(np.float32))
    return out, lse, dout
