"""CPU: the host-side bounds model of the kernels' index arithmetic, and the
C-ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/host/sta_host_model.cpp links sta_api.cpp with launchers that, instead
of launching, walk every workgroup of the grid the real launcher would use
(same parameters, work-item shapes, task decoding and window walks, taken
from sta_plan.h) and check every row read or written, the LDS staging
indices and the 32-bit load offsets. It drives the C ABI with the named
workloads, padded and ragged grids, 2D volumes, per-head windows, both token
orders, the backward, recall and fp8 entry points, and invalid calls that
must be refused before any launch."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "host", "sta_host_model.cpp"),
       os.path.join(ROOT, "sparse_attention_video_tile_amd", "csrc", "sta_api.cpp")]
INC = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "sparse_attention_video_tile_amd", "csrc")]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_model_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sta_host_model")
    build = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                            "-fno-sanitize-recover=all", "-Wall", "-Wno-unused-function", *INC, *SRC,
                            "-o", exe], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1",
                                  UBSAN_OPTIONS="print_stacktrace=1"))
    print(run.stdout)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "all in bounds" in run.stdout
    # the 30x48x80 workloads' 7200 whole-tile items leave a partly filled last
    # round, which the launcher runs as 64-row items: that path is modelled
    tails = re.search(r"\((\d+) forwards with a split last round, (\d+) one-pass recalls\)", run.stdout)
    assert tails and int(tails.group(1)) > 0, run.stdout[-500:]
    # window recall runs as one pass wherever the kernels allow: modelled too
    assert int(tails.group(2)) > 0, run.stdout[-500:]
    # padded grids with tau a multiple of 64 take each chunk's token mask from
    # precomputed tables: checked against the per-key rule on every such chunk
    masks = re.search(r"(\d+) padded chunk masks from tables", run.stdout)
    assert masks and int(masks.group(1)) > 0, run.stdout[-500:]
    # the float32 kernels' unpadded row mapping leaves a raster slice on a
    # padded grid (which is why the library refuses that case)
    assert "raster order: 324 query rows map past the 210 rows" in run.stdout
