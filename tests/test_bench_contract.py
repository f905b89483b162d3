"""Host-side checks of bench.py (no GPU): the committed HBM counter summaries
still describe the kernels as they are built now, and the multi-GPU request is
refused before anything touches a device."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

COUNTERS = [
    (bench.COUNTERS_FILE, bench.SCORE_SOURCES, "score_decode.hip", 146070576),
    (bench.counters_file("decode-mtp"), bench.SCORE_SOURCES, "score_decode.hip", 35068608),
    (bench.counters_file("decode-ragged"), bench.SCORE_SOURCES, "score_decode.hip", 420807384),
    # 63 pages: fixed per-launch reads (arguments, code) are a large share
    (bench.counters_file("decode-tiny"), bench.SCORE_SOURCES, "score_decode.hip", None),
    (bench.MX_COUNTERS_FILE, bench.MX_SOURCES, "mxfp8.hip", 16384 * 2048 * 3 + 16384 * 2048 // 32),
    (bench.DQ_COUNTERS_FILE, bench.DQ_SOURCES, "dequant.hip", None),
]


@pytest.mark.parametrize("path,sources,flags_of,algo", COUNTERS,
                         ids=[os.path.basename(c[0]) for c in COUNTERS])
def test_counter_summary_matches_current_kernel(path, sources, flags_of, algo):
    """A kernel edit without new counters makes roofline.traffic null (which
    bench.py reports honestly); the skip names the stale file."""
    assert os.path.exists(path), f"{os.path.basename(path)} is missing"
    traffic = bench.read_counters(path, sources, flags_of)
    if traffic is None:
        pytest.skip(f"{os.path.basename(path)} was taken from other sources or flags (current "
                    f"hash {bench.kernel_source_hash(sources, flags_of)}): re-collect the counters")
    kv = {}
    for line in open(path):
        k, _, v = line.partition("=")
        if k.strip().startswith("hbm_"):
            kv[k.strip()] = float(v)
    assert kv["hbm_read_bytes_per_launch"] + kv["hbm_write_bytes_per_launch"] == pytest.approx(
        traffic, abs=2)
    if algo is not None:
        # Measured traffic can only exceed the algorithmic bytes by re-reads;
        # it cannot fall far below them.
        assert 0.99 * algo <= traffic <= 1.10 * algo


def test_hash_depends_on_sources_and_flags():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash(bench.SCORE_SOURCES, "score_decode.hip")
    assert h != bench.kernel_source_hash(bench.MX_SOURCES, "mxfp8.hip")
    assert h != bench.kernel_source_hash(bench.SCORE_SOURCES, "mxfp8.hip") or \
        bench._compile_flags("score_decode.hip") == bench._compile_flags("mxfp8.hip")


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stdout
