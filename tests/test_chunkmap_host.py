"""The chunk map of the matrix-core pass (cost units -> workgroup chunks) is
index work and must be exact: the device code replaces 64-bit division by a
double-precision estimate and one integer correction.  The same source
(csrc/gqa_chunkmap.h) is compiled for the host here and compared with exact
128-bit integer division across the range the planner admits (up to 2^16
workgroups, up to 2^18 * (2^25 + 63) cost units) and at random points.
CPU only."""
import os
import subprocess

from conftest import ROOT

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_chunk_map_is_exact(tmp_path):
    src = os.path.join(ROOT, "tests", "host", "chunkmap_check.cpp")
    inc = os.path.join(ROOT, "grouped_query_attention_decode_amd", "csrc")
    exe = str(tmp_path / "chunkmap_check")
    r = subprocess.run([HIPCC, "-O2", "-std=c++17", "-I", inc, src, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0" in r.stdout
