"""CPU replay of the dQ kernel's dS-row addressing (no GPU).

The dQ kernel loads each tile row's dS through a buffer resource over its
token group's rows; lanes without a row (past the group's last token in the
last group of a ragged length, or past a tile's rows) must be sent to the end
of that range, where the load returns zeros.  A first version loaded rows for
lanes past the sequence end.  tests/native/dq_index_check.hip calls the same
index functions as the kernel (csrc/bwd_index.h) for every workgroup, tile,
lane and slot of the parity-test shapes and of the full benchmark shapes.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "dq_index_check.hip")
CSRC = os.path.join(ROOT, "gated_block_sparse_gate_amd", "csrc")

# (B, T, Hq, Hkv, K): the small parity shapes (ragged lengths 1000, 700, 300,
# 50, 600, 260; G = 1, 2, 4, 5, 8; K = 0 and K beyond the blocks) and the
# full benchmark shapes, plus G = 3 and G = 7 (with G = 3 the last tile reaches past the
# 64 per-token rows, where the clamp matters)
SHAPES = [(1, 1024, 2, 1, 3), (1, 1000, 8, 2, 7), (1, 700, 10, 2, 5), (2, 300, 2, 2, 2),
          (1, 50, 4, 1, 3), (1, 400, 4, 2, 0), (1, 600, 4, 1, 20), (1, 260, 8, 1, 3),
          (1, 8192, 32, 8, 31), (1, 32768, 32, 8, 31), (1, 32768, 40, 8, 63), (1, 4097, 24, 3, 9),
          (1, 1000, 6, 2, 5), (1, 777, 21, 7, 4), (1, 333, 14, 2, 6),
          # one gate per query head: Hq selection heads of one query head each
          # (the dQ kernel's rows are then those of Hkv = Hq, G = 1)
          (1, 1000, 8, 8, 7), (1, 8192, 32, 32, 31)]


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("idx") / "dq_index_check")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", CSRC, SRC,
                    "-o", exe], check=True, capture_output=True)
    return exe


def test_dq_ds_addressing_stays_in_range(checker):
    args = [str(v) for s in SHAPES for v in s]
    r = subprocess.run([checker, *args], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("ok ") == len(SHAPES)
