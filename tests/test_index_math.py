"""Host-side check of an index identity the affine matrix-core GEMV relies on
(no GPU needed).

When the GEMV stages x [m][cols] (16-bit values) into LDS, chunk i (16 bytes,
i < m * cols / 8) goes to row i / (cols / 8) of the padded copy.  The kernel
takes that quotient as umulhi(i, xdiv) with xdiv = ceil(2^32 / (cols / 8)),
computed by the launcher.  This is exact when i * (cols / 8) < 2^32.  The test
checks the identity exhaustively for every width the ABI accepts
(cols % 64 == 0, up to 65536) at m = 16, the largest batch.
"""
import numpy as np


def test_multiply_high_row_of_x_chunk_is_exact():
    bad = []
    for cols in range(64, 65536 + 1, 64):
        d = cols // 8
        xdiv = -(-(1 << 32) // d)  # ceil(2^32 / d), as the launcher computes it
        assert xdiv < (1 << 32)
        i = np.arange(16 * d, dtype=np.uint64)
        got = (i * np.uint64(xdiv)) >> np.uint64(32)
        if not np.array_equal(got, i // np.uint64(d)):
            bad.append(cols)
    assert not bad, f"multiply-high row wrong for cols {bad[:8]}"
