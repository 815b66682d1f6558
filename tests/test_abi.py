"""Host-side checks of the C ABI: exports, the FLOP cost model and argument validation.

None of these launch a kernel: validation happens before any HIP call, and the FLOP functions
are host-only integer arithmetic.  The FLOP model is checked against the oracle's brute-force
enumeration of the mask.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from variable_length_attention_amd import _lib, ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hdp_attn.h")
U64_MAX = 2 ** 64 - 1


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hdp_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "hdp_attn_varlen_fwd" in names and len(names) >= 9
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = _lib.lib()
    for n in names:
        assert hasattr(lib, n)
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of date"


@pytest.mark.parametrize("s", [1, 2, 17, 64, 100, 255, 256, 512])
@pytest.mark.parametrize("causal", [True, False])
def test_seq_flops_equals_mask_enumeration(s, causal):
    for H, D in ((4, 64), (32, 128)):
        for p in (0, 1, 2):
            assert ops.hdp_seq_flops(s, H, D, causal, p) == oracle.seq_flops(s, H, D, causal, p)


def test_chunk_flops_equals_mask_enumeration_random_offsets():
    rng = np.random.default_rng(123)
    for _ in range(300):
        Lq, Lk = (int(x) for x in rng.integers(1, 80, size=2))
        q_off, kv_off = (int(x) for x in rng.integers(0, 200, size=2))
        causal = bool(rng.integers(0, 2))
        want = oracle.attn_flops(Lq, Lk, q_off, kv_off, causal, 3, 64, 0)
        assert ops.hdp_chunk_flops(Lq, Lk, q_off, kv_off, causal, 3, 64, 0) == want


def test_chunk_flops_sum_over_ring_equals_sequence_flops():
    # The steps of a ring cover every visible pair of the sequence exactly once.
    s, c, H, D = 4096, 512, 32, 128
    total = sum(ops.hdp_chunk_flops(c, c, qi * c, kj * c, True, H, D, 0)
                for qi in range(s // c) for kj in range(s // c))
    assert total == ops.hdp_seq_flops(s, H, D, True, 0)


def test_fixed_flop_values_of_the_workloads():
    # Tiny fp32 pack [17, 64, 100, 75], H = 4, D = 64.
    assert sum(ops.hdp_seq_flops(s, 4, 64) for s in (17, 64, 100, 75)) == 10_376_192
    assert ops.hdp_seq_flops(8192, 32, 128, True, 0) == 549_822_922_752
    assert ops.hdp_seq_flops(8192, 32, 128, True, 1) == 1_374_557_306_880
    # 8192 queries at offset 122880 against the 16 chunks of a 131072-token sequence.
    ring = sum(ops.hdp_chunk_flops(8192, 8192, 122880, 8192 * k, True, 32, 128, 0)
               for k in range(16))
    assert ring == 17_042_497_339_392
    assert ring == oracle.attn_flops(8192, 131072, 122880, 0, True, 32, 128, 0)


def test_flop_edge_cases():
    assert ops.hdp_seq_flops(0, 32, 128) == 0
    assert ops.hdp_seq_flops(-5, 32, 128) == 0
    assert ops.hdp_seq_flops(10, 32, 128, True, 7) == U64_MAX
    assert ops.hdp_seq_flops(2 ** 40, 2 ** 20, 128) == U64_MAX   # overflow sentinel
    assert ops.hdp_chunk_flops(10, 10, 0, 50, True, 1, 64) == 0  # chunk entirely in the future
    assert ops.hdp_chunk_flops(0, 10, 0, 0, True, 1, 64) == 0


# ------------------------------------------------------------- argument validation

NULL = None
FAKE = 0x1000  # never dereferenced: every case below fails validation or is a no-op first


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, n_seq=1, H=32, Hkv=8, D=128, scale=0.088,
             out=FAKE, lse=FAKE)
    a.update(kw)
    return _lib.lib().hdp_attn_varlen_fwd(a["q"], a["k"], a["v"], a["cu"], a["n_seq"], a["H"],
                                          a["Hkv"], a["D"], a["scale"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_seq=-1), _lib.HDP_ERR_INVALID_ARG),
    (dict(H=30, Hkv=8), _lib.HDP_ERR_INVALID_ARG),
    (dict(H=0), _lib.HDP_ERR_INVALID_ARG),
    (dict(Hkv=0), _lib.HDP_ERR_INVALID_ARG),
    (dict(D=96), _lib.HDP_ERR_UNSUPPORTED),
    (dict(D=0), _lib.HDP_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.HDP_ERR_INVALID_ARG),
    (dict(scale=float("inf")), _lib.HDP_ERR_INVALID_ARG),
    (dict(scale=-0.5), _lib.HDP_ERR_INVALID_ARG),
    (dict(q=NULL), _lib.HDP_ERR_INVALID_ARG),
    (dict(cu=NULL), _lib.HDP_ERR_INVALID_ARG),
    (dict(lse=NULL), _lib.HDP_ERR_INVALID_ARG),
    (dict(H=65544, Hkv=8), _lib.HDP_ERR_OVERFLOW),
    (dict(n_seq=0, q=NULL, out=NULL), _lib.HDP_OK),  # empty work is a no-op
])
def test_varlen_fwd_validation(kw, status):
    assert fwd(**kw) == status


def test_other_entry_points_validate_before_touching_the_gpu():
    L = _lib.lib()
    assert L.hdp_attn_varlen_fwd_f32(FAKE, FAKE, FAKE, FAKE, 1, 4, 3, 64, 0.1, FAKE, FAKE,
                                     None) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_attn_chunk_partial(FAKE, -1, FAKE, FAKE, 8, 0, 0, 1, 32, 8, 128, 0.1, FAKE,
                                    FAKE, None) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_attn_chunk_partial(FAKE, 8, FAKE, FAKE, 8, -1, 0, 1, 32, 8, 128, 0.1, FAKE,
                                    FAKE, None) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_attn_chunk_partial(FAKE, 8, NULL, FAKE, 8, 0, 0, 1, 32, 8, 128, 0.1, FAKE,
                                    FAKE, None) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_attn_chunk_partial(NULL, 0, NULL, NULL, 0, 0, 0, 1, 32, 8, 128, 0.1, NULL,
                                    NULL, None) == _lib.HDP_OK
    assert L.hdp_lse_merge(FAKE, FAKE, FAKE, FAKE, 4, 2, 32, NULL, None) == _lib.HDP_ERR_UNSUPPORTED
    assert L.hdp_lse_merge(FAKE, NULL, FAKE, FAKE, 4, 2, 64, NULL, None) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_lse_merge(NULL, NULL, NULL, NULL, 0, 2, 64, NULL, None) == _lib.HDP_OK
    assert L.hdp_attn_varlen_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, -1, 32, 8, 128,
                                 0.1, FAKE, FAKE, FAKE, None) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_attn_varlen_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 1, 10, 32, 8, 128,
                                 0.1, FAKE, FAKE, FAKE, None) == _lib.HDP_ERR_INVALID_ARG
    # chunk backward: negative sizes/offsets, a null operand, bad heads, and empty work
    cb = L.hdp_attn_chunk_bwd
    assert cb(FAKE, -1, FAKE, FAKE, 8, 0, 0, 1, 32, 8, 128, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE,
              FAKE, None) == _lib.HDP_ERR_INVALID_ARG
    assert cb(FAKE, 8, FAKE, FAKE, 8, 0, -4, 1, 32, 8, 128, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE,
              FAKE, None) == _lib.HDP_ERR_INVALID_ARG
    assert cb(FAKE, 8, FAKE, FAKE, 8, 0, 0, 1, 32, 8, 128, 0.1, FAKE, FAKE, FAKE, NULL, FAKE,
              FAKE, None) == _lib.HDP_ERR_INVALID_ARG
    assert cb(FAKE, 8, FAKE, FAKE, 8, 0, 0, 1, 32, 8, 96, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE,
              FAKE, None) == _lib.HDP_ERR_UNSUPPORTED
    assert cb(FAKE, 8, FAKE, FAKE, 8, 0, 0, 1, 30, 8, 128, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE,
              FAKE, None) == _lib.HDP_ERR_INVALID_ARG
    assert cb(FAKE, 8, FAKE, FAKE, 8, 0, 0, 1, 32, 8, 128, float("nan"), FAKE, FAKE, FAKE, FAKE,
              FAKE, FAKE, None) == _lib.HDP_ERR_INVALID_ARG
    assert cb(NULL, 0, NULL, NULL, 8, 0, 0, 1, 32, 8, 128, 0.1, NULL, NULL, NULL, NULL, NULL,
              NULL, None) == _lib.HDP_OK
    assert cb(NULL, 8, NULL, NULL, 0, 0, 0, 1, 32, 8, 128, 0.1, NULL, NULL, NULL, NULL, NULL,
              NULL, None) == _lib.HDP_OK
    for st in range(5):
        assert _lib.lib().hdp_status_string(st).startswith(b"HDP_")


def test_trace_helpers_validate_their_arguments():
    # measurement helpers only store a device pointer: no HIP call, so they run here
    L = _lib.lib()
    assert L.hdp_set_trace(NULL, -1) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_set_trace(NULL, 4) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_set_item_trace(NULL, -1, 4) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_set_item_trace(FAKE, 4, -1) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_set_item_trace(NULL, 4, 4) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_set_item_trace(FAKE, 4, 0) == _lib.HDP_ERR_INVALID_ARG
    assert L.hdp_set_item_trace(NULL, 0, 0) == _lib.HDP_OK
    assert L.hdp_set_trace(NULL, 0) == _lib.HDP_OK


def test_clock_probe_validates_before_any_hip_call():
    lib = _lib.lib()
    import ctypes
    mhz = ctypes.c_double(0.0)
    assert lib.hdp_probe_clock(0, ctypes.addressof(mhz), None) == _lib.HDP_ERR_INVALID_ARG
    assert lib.hdp_probe_clock(100, None, None) == _lib.HDP_ERR_INVALID_ARG


def test_noalloc_backward_rejects_sizes_beyond_its_scratch_before_any_hip_call():
    # 4096 + 8 * T * H must fit the fixed scratch; the check comes before any HIP call, so the
    # (never dereferenced) pointers here are placeholders
    lib = _lib.lib()
    p = 4096
    limit = (_lib.NOALLOC_SCRATCH_BYTES - 4096) // 8          # largest T * H
    H = 32
    T = limit // H + 1
    st = lib.hdp_attn_varlen_bwd_noalloc(p, p, p, p, p, p, p, 1, T, H, 8, 128, 0.1, p, p, p, None)
    assert st == _lib.HDP_ERR_SCRATCH_LIMIT
    assert b"no-allocation" in lib.hdp_status_string(st)
    # invalid arguments are reported as for the allocating entry point
    assert lib.hdp_attn_varlen_bwd_noalloc(p, p, p, p, p, p, p, 1, 10, 6, 4, 128, 0.1, p, p, p, None) == _lib.HDP_ERR_INVALID_ARG
    assert lib.hdp_attn_varlen_bwd_noalloc(p, p, p, p, p, p, p, 0, 10, 8, 2, 128, 0.1, p, p, p, None) == _lib.HDP_OK
