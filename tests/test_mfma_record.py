"""The committed record of the matrix-instruction accuracy probe
(profiles/mfma_accuracy.md, written from tests/test_gpu_mfma_accuracy.py on
an MI355X) re-derived on the CPU: the tiles are regenerated from the seed,
their exact dot products recomputed in integers, and the recorded outputs
give the stated error figures -- the f16 MFMA below 2^-17 of the largest
product, the fp8 MFMAs above 2^-14."""

import json
import os
import re

import numpy as np

import mfma_probe
import workloads

RECORD = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles",
                      "mfma_accuracy.md")


def load_record():
    text = open(RECORD).read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    assert m, "no JSON block in the record"
    return json.loads(m.group(1))


def test_record_rederives_on_cpu():
    r = load_record()
    a, b = workloads.mfma_probe_tiles(r["seed"], r["tiles"])
    idx = r["record_tiles"]
    n = len(idx)
    dots, maxp = mfma_probe.exact(a[idx], b[idx])
    for m in mfma_probe.METHODS:
        got = np.array([[int(h, 16) for h in tile] for tile in r["outputs_hex"][m]],
                       dtype=np.uint32).view(np.float32).reshape(n, 16, 16)
        fig = mfma_probe.worst_log2(got, dots, maxp)
        assert abs(fig - r["worst_log2_record_tiles"][m]) < 1e-9, m
    f16, fp8, f864 = (r["worst_log2_record_tiles"][m] for m in mfma_probe.METHODS)
    assert f16 <= -17.0
    assert fp8 >= -14.0 and f864 >= -14.0
