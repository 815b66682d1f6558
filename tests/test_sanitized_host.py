"""CPU: the host layer and the oracle, built with AddressSanitizer and UndefinedBehaviorSanitizer,
run the CPU test tier (argument checks, FLOP model, planner, oracle pins) in a subprocess.  Any
out-of-bounds access, use after free, signed overflow or other undefined behaviour in api.cpp,
plan.cpp or the oracle stops that run with a report, which fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_abi.py", "tests/test_plan.py", "tests/test_oracle_pins.py", "tests/test_synth_fixtures.py"]


@pytest.mark.skipif(os.environ.get("HDP_LIB_PATH") is not None, reason="already inside the sanitized run")
def test_cpu_tier_under_address_and_undefined_behaviour_sanitizers():
    from variable_length_attention_amd import build_sanitized

    host, orc = build_sanitized.build()
    env = build_sanitized.sanitizer_env(host, orc)
    probe = ("from variable_length_attention_amd import _lib; import oracle; "
             "print(_lib.lib()._name); print(oracle._load()._name)")
    loaded = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True)
    assert loaded.returncode == 0, loaded.stderr[-3000:]
    assert host in loaded.stdout and orc in loaded.stdout, loaded.stdout
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider"] + SUITES,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-5000:]
    assert r.returncode == 0, out[-5000:]
