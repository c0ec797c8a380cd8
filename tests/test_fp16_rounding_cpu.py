"""The prefill conversion rounds its double-precision keys to fp16 with
swan::d2h_odd (csrc/fp16_round.h: round to odd at float precision, then to
nearest even).  This host build of the same source checks it against the
compiler runtime's direct double -> fp16 conversion over every fp16
midpoint and its neighbourhood and 25 million further doubles
(tests/fp16_rounding_check.cpp)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_d2h_odd_matches_direct_conversion(tmp_path):
    exe = str(tmp_path / "fp16_rounding_check")
    src = os.path.join(ROOT, "tests", "fp16_rounding_check.cpp")
    inc = os.path.join(ROOT, "decode_attention_compressed_02_amd", "csrc")
    subprocess.run([HIPCC, "-x", "c++", "-O2", "-std=c++17", "-D__host__=", "-D__device__=", "-I", inc, src,
                    "-o", exe], check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith(" 0 mismatches"), r.stdout
