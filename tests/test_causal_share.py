"""The balanced schedule of the ragged causal prefill (the header
page_scoring_top_amd/csrc/causal_share.hpp, which the GPU kernel runs),
built for the CPU and checked on random batches: its closed-form chunk
counts against the causal mask's definition (Modular page
"sparse_index_fp8_sm100", module description: causal masking, -inf past a
row's visible keys), and its shares covering every chunk of every query
group exactly once for several grid sizes (tests/causal_share_check.cpp)."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "page_scoring_top_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_schedule_covers_every_chunk_once(tmp_path):
    exe = str(tmp_path / "causal_share_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, "-o", exe,
                    os.path.join(HERE, "causal_share_check.cpp")], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.stdout.strip().endswith("bad 0"), r.stdout[-2000:]
