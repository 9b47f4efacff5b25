"""The span kernels' scan-order row mapping, emulated on the host in the
kernel's own arithmetic (fp32 where the kernel uses fp32), against the
oracle's scan order: every step of every chunk, all four scan orders, grid
heights below, at and above the chunk length.

Per chunk the kernel takes the first step's column and row (column-major
orders) with one integer division; a row r of the chunk is then placed with
floor((x + 1/2) * (1 / grid_h)) in fp32, x = r0 +- r. The last test checks
that floor against integer floor division for every grid height up to 2048
(and some far larger) and every x the kernel can form."""
import numpy as np
import pytest

import oracle

CHUNK = 64


def kernel_row_pos(t0, r, L, gh, gw, d):
    t = t0 + r
    if d >= 2:
        u0 = L - 1 - t0 if d == 3 else t0
        c0, r0 = u0 // gh, u0 - (u0 // gh) * gh
        x = r0 - r if d == 3 else r0 + r
        q = int(np.floor((np.float32(x) + np.float32(0.5)) * (np.float32(1.0) / np.float32(gh))))
        p = (x - q * gh) * gw + c0 + q
    else:
        p = L - 1 - t if d == 1 else t
    return p if t < L else -1


@pytest.mark.parametrize("gh,gw", [(1, 100), (100, 1), (1, 1), (30, 30), (24, 40), (64, 64),
                                   (63, 65), (130, 7), (7, 130)])
@pytest.mark.parametrize("d", [0, 1, 2, 3])
def test_row_map_matches_oracle_scan_order(gh, gw, d):
    L = gh * gw
    ref = oracle.scan_order(gh, gw, d)
    n_chunks = -(-L // CHUNK)
    got = np.array([kernel_row_pos(c * CHUNK, r, L, gh, gw, d)
                    for c in range(n_chunks) for r in range(CHUNK)])
    assert (got[:L] == ref).all()
    assert (got[L:] == -1).all()


def test_fp32_floor_division_is_exact():
    for gh in list(range(1, 2049)) + [4095, 4096, 10000, 65535, 65536, 1 << 20]:
        x = np.arange(-CHUNK - gh, gh + CHUNK + 1, dtype=np.int64)
        inv = np.float32(1.0) / np.float32(gh)
        q = np.floor((x.astype(np.float32) + np.float32(0.5)) * inv).astype(np.int64)
        assert (q == np.floor_divide(x, gh)).all(), gh
