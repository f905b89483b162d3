"""GPU parity of mxfp8_e4m3_quantize against the oracle (vLLM pull request
#65508, "How it works"): E4M3 bytes and E8M0 scale bytes bit-exact, and
nothing written outside the first cols (cols / 32) bytes of rows < rows."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import announce, host

pytestmark = pytest.mark.gpu

CANARY = 0xA5


def gpu_quantize(x: np.ndarray, x_pad: int = 0, q_pad: int = 0, s_pad: int = 0):
    import page_scoring_top_amd as ps
    rows, cols = x.shape
    xs = torch.zeros((rows, cols + x_pad), dtype=torch.int16, device="cuda")
    xs[:, :cols] = torch.from_numpy(x.view(np.int16)).to("cuda")
    xv = xs[:, :cols].view(torch.bfloat16)
    q = torch.full((rows + 1, cols + q_pad), CANARY, dtype=torch.uint8, device="cuda")
    s = torch.full((rows + 1, cols // 32 + s_pad), CANARY, dtype=torch.uint8, device="cuda")
    ps.mxfp8_e4m3_quantize(xv, q[:rows], s[:rows])
    return host(q), host(s)


def check(x, what, **pads):
    rows, cols = x.shape
    got_q, got_s = gpu_quantize(x, **pads)
    want_q, want_s = oracle.mxfp8_quantize(x)
    assert np.array_equal(got_s[:rows, :cols // 32], want_s), f"{what}: scale bytes differ"
    bad = np.argwhere(got_q[:rows, :cols] != want_q)
    assert bad.size == 0, (f"{what}: {len(bad)} E4M3 bytes differ, first at {tuple(bad[0])}: "
                           f"gpu {got_q[tuple(bad[0])]:#x} oracle {want_q[tuple(bad[0])]:#x}")
    assert (got_q[rows:] == CANARY).all() and (got_q[:, cols:] == CANARY).all()
    assert (got_s[rows:] == CANARY).all() and (got_s[:, cols // 32:] == CANARY).all()


@pytest.mark.parametrize("rows,cols", [(1, 32), (3, 96), (5, 7168), (128, 2048), (129, 2048),
                                       (300, 160)])
def test_shapes(rows, cols):
    x = workloads.mx_activations(rows * 131 + cols, rows, cols)
    announce(f"mxfp8 rows={rows} cols={cols}")
    check(x, f"{rows}x{cols}", x_pad=8, q_pad=16, s_pad=3)


def test_edge_blocks():
    """The page's edge blocks: zeros, subnormals, 446/448/450, the 1.75
    boundary and the value just above it; plus negative zeros, mixed signs
    and non-finite elements."""
    rng = np.random.default_rng(21)
    rows = []
    rows.append(np.zeros(32, np.uint16))
    rows.append(np.full(32, 0x8000, np.uint16))
    rows.append(rng.integers(1, 0x80, 32).astype(np.uint16))                    # subnormals
    rows.append(rng.integers(1, 0x80, 32).astype(np.uint16) | 0x8000)
    for top in (0x43DF, 0x43E0, 0x43E1):                                         # 446, 448, 450
        r = rng.integers(0x3000, 0x43E0, 32).astype(np.uint16)
        r[17] = top
        rows.append(r)
    for e in (1, 7, 8, 9, 100, 127, 135, 200, 254):
        for frac in (96, 97, 127, 0):
            r = rng.integers(0, (e << 7) | frac, 32).astype(np.uint16)
            r[int(rng.integers(0, 32))] = (e << 7) | frac
            r |= (rng.integers(0, 2, 32).astype(np.uint16) << 15)
            rows.append(r)
    nonfin = rng.integers(0x3000, 0x4000, 32).astype(np.uint16)
    nonfin[[0, 5, 9]] = [0x7F80, 0xFF80, 0x7FC1]
    rows.append(nonfin)
    nan_only = rng.integers(0, 0x100, 32).astype(np.uint16)
    nan_only[31] = 0xFFE1
    rows.append(nan_only)
    # Exact halfway cases for E4M3 after scaling: 1 + 1/16 and 1 + 3/16 times 2^k.
    halves = np.full(32, 0x3F80, np.uint16)                                     # 1.0
    halves[1::2] = [0x3F88, 0x3F98] * 8                                         # 1.0625, 1.1875
    halves[0] = 0x43E0                                                          # block max 448
    rows.append(halves)
    x = np.stack(rows)
    announce("mxfp8 edge blocks")
    check(x, "edge blocks")


def test_big_batch_full():
    """16,384 rows x 2,048 (a prefill-sized batch of the attention output),
    every byte against the oracle."""
    x = workloads.mx_activations(77, 16384, 2048)
    announce("mxfp8 16384 x 2048")
    check(x, "16384x2048")


def test_rows_past_one_grid_column():
    """262,147 rows: more than 65,535 groups of 4 rows, so work-groups loop
    over rows (grid y is capped); every byte against the oracle, with a
    ragged last group."""
    x = workloads.mx_activations(78, 65535 * 4 + 7, 64)
    announce("mxfp8 262147 x 64")
    check(x, "262147x64", x_pad=8, q_pad=16, s_pad=1)
