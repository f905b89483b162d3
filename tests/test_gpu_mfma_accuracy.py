"""Why the indexer kernels use the f16 MFMA and not an fp8 one (the score
tolerance is 1e-6 + 1e-5 |exact|).

The probe (tests/probe/mfma_accuracy.hip) runs 400 seeded 16 x 16 x 128 tiles
of E4M3 dot products (even tiles over the whole E4M3 range, odd tiles
cancelling to a small remainder) through three gfx950 instructions.  Against
the exact integer dot products, relative to the largest product of each dot:
the f16 MFMA on exact f16 conversions stays below 2^-17, while the fp8 MFMA
and the f8f6f4 MFMA lose more than 2^-14 -- an error that size on a dot whose
terms are as large as the dot itself already exceeds the 1e-5 tolerance.

With PAGESCORE_RECORD_DIR set, the test writes mfma_accuracy_record.json
there: the figures over all tiles and the three methods' outputs of tile 0
and of the tiles where each fp8 method does worst, the record that
profiles/mfma_accuracy.md keeps and tests/test_mfma_record.py re-derives on
the CPU."""

import ctypes
import json
import os

import numpy as np
import pytest
import torch

import mfma_probe
import workloads
from gpu_util import announce

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "probe", "libmfma_probe.so")
SEED, TILES = 17, 400


def run_probe(a, b):
    assert os.path.exists(LIB), f"{LIB} is missing: run __graft_entry__.build()"
    lib = ctypes.CDLL(LIB)
    lib.mfma_accuracy_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.mfma_accuracy_probe.restype = ctypes.c_int
    da, db = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    tiles = a.shape[0]
    out = torch.full((tiles, 3, 16, 16), float("nan"), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    rc = lib.mfma_accuracy_probe(ctypes.c_void_p(da.data_ptr()), ctypes.c_void_p(db.data_ptr()),
                                 tiles, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(s.cuda_stream))
    assert rc == 0, f"probe launch failed: {rc}"
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_matrix_instruction_accuracy():
    a, b = workloads.mfma_probe_tiles(SEED, TILES)
    announce(f"mfma accuracy probe, {TILES} tiles")
    got = run_probe(a, b)
    dots, maxp = mfma_probe.exact(a, b)
    figures = {m: mfma_probe.worst_log2(got[:, i], dots, maxp)
               for i, m in enumerate(mfma_probe.METHODS)}
    # Recorded tiles: the one where each fp8 method does worst, and tile 0.
    per_tile = [[mfma_probe.worst_log2(got[t, i][None], dots[t][None], maxp[t][None])
                 for t in range(TILES)] for i in range(3)]
    idx = sorted({0, int(np.argmax(per_tile[1])), int(np.argmax(per_tile[2]))})
    rec = {m: mfma_probe.worst_log2(got[idx, i], dots[idx], maxp[idx])
           for i, m in enumerate(mfma_probe.METHODS)}
    for m in mfma_probe.METHODS:
        print(f"[mfma-accuracy] {m}: worst |error| / max|product| = 2^{figures[m]:.2f} over "
              f"{TILES} tiles, 2^{rec[m]:.2f} over the recorded tiles {idx}", flush=True)
    out_dir = os.environ.get("PAGESCORE_RECORD_DIR")
    if out_dir:
        os.makedirs(out_dir, exist_ok=True)
        with open(os.path.join(out_dir, "mfma_accuracy_record.json"), "w") as f:
            json.dump({"seed": SEED, "tiles": TILES, "record_tiles": idx,
                       "worst_log2_all_tiles": figures, "worst_log2_record_tiles": rec,
                       "outputs_hex": {m: [[format(int(x), "08x") for x in
                                            got[t, i].astype(np.float32).view(np.uint32).ravel()]
                                           for t in idx]
                                       for i, m in enumerate(mfma_probe.METHODS)}}, f)
    f16, fp8, f864 = (figures[m] for m in mfma_probe.METHODS)
    assert f16 <= -17.0, f"f16 MFMA error 2^{f16:.2f} of the largest product"
    assert fp8 >= -14.0 and f864 >= -14.0, "an fp8 MFMA now meets the tolerance: revisit the f16 choice"
