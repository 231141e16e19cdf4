"""The decode's partial-slot bookkeeping (csrc/slots.hpp: where the pieces of
a split segment store their partials, and how many the merging workgroup
waits for), compiled for the host and checked against brute-force ownership
over ragged batches, empty segments, cost units 0..12 and workgroup counts on
both sides of the unit total (tests/host/slots_check.cpp).  No GPU."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_slot_bookkeeping_matches_brute_force():
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no C++ compiler")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "slots_check")
        r = subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-Werror", "-D__host__=",
                            "-D__device__=", "-I",
                            os.path.join(ROOT, "block_paged_kv_append_amd", "csrc"),
                            os.path.join(ROOT, "tests", "host", "slots_check.cpp"), "-o", exe],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
