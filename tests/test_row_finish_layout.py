"""CPU walk of how the decode kernel rotates a finished prefill row back (no GPU).

A row that one workgroup computes whole is written by the w = 512 tile itself, rotated back by the
orthonormal Sylvester Hadamard matrix (the TPLA abstract's Hadamard reparameterisation; the output
is returned in the unrotated frame).  Its 512 columns sit in the two waves of a pair, 64 lanes and
128 accumulator registers: column = 256 kh + 32 cb + 8 (j / 4) + 4 half + j % 4 for register
16 cb + j of a lane in half `half` (lanes 0-31 or 32-63; the head is the lane modulo 32).  The
kernel applies one 2-point butterfly per column bit: in registers for seven bits, by two
permlane32 swaps per register pair for the lane half, and through LDS for the wave.  Here those
steps are restated on arrays (one head; v_permlane32_swap_b32 as the ISA defines it: the upper 32
lanes of the first operand trade places with the lower 32 lanes of the second) and compared with
scipy's Hadamard matrix, so that a wrong bit, pair or sign in the layout fails on the host."""

import numpy as np
import pytest
from scipy.linalg import hadamard

N = 512


def col_of(kh, half, r):
    cb, j = divmod(r, 16)
    return 256 * kh + 32 * cb + 8 * (j >> 2) + 4 * half + (j & 3)


def load(y):
    """z[kh][lane][r] holding column col_of(kh, lane // 32, r) of y (every head the same row)."""
    z = np.zeros((2, 64, 128))
    for kh in range(2):
        for lane in range(64):
            for r in range(128):
                z[kh, lane, r] = y[col_of(kh, lane // 32, r)]
    return z


def permlane32_swap(a, b):
    """(new a, new b): lanes 32-63 of a and lanes 0-31 of b trade places."""
    na, nb = a.copy(), b.copy()
    na[32:], nb[:32] = b[:32], a[32:]
    return na, nb


def finish(z):
    z = z.copy()
    for kh in range(2):
        for k in range(7):  # register bits, lower index takes the sum
            bit = 1 << k
            for r in range(128):
                if r & bit == 0:
                    u, v = z[kh, :, r].copy(), z[kh, :, r | bit].copy()
                    z[kh, :, r], z[kh, :, r | bit] = u + v, u - v
        for r in range(0, 128, 2):  # lane-half bit
            lo, hi = permlane32_swap(z[kh, :, r], z[kh, :, r + 1])
            lo, hi = lo + hi, lo - hi
            z[kh, :, r], z[kh, :, r + 1] = permlane32_swap(lo, hi)
    out = np.full((64, N), np.nan)  # per lane; lanes of one half must agree on the head's row
    sent = {0: z[0, :, 64:].copy(), 1: z[1, :, :64].copy()}  # kh = 0 gives blocks 4..7, kh = 1 blocks 0..3
    for kh in range(2):
        keep = 0 if kh == 0 else 64
        theirs = sent[1 - kh]
        for lane in range(64):
            half = lane // 32
            for i in range(16):
                for e in range(4):
                    own, oth = z[kh, lane, keep + 4 * i + e], theirs[lane, 4 * i + e]
                    lo = own + oth if kh == 0 else oth + own
                    hi = own - oth if kh == 0 else oth - own
                    cb = (0 if kh == 0 else 4) + i // 4
                    col = 32 * cb + 8 * (i % 4) + 4 * half + e
                    for c, v in ((col, lo), (col + 256, hi)):
                        assert np.isnan(out[lane, c]), "a column written twice"
                        out[lane, c] = v
    return out / np.sqrt(N)


def test_layout_covers_every_column_once():
    seen = sorted(col_of(kh, half, r) for kh in range(2) for half in range(2) for r in range(128))
    assert seen == list(range(N))


@pytest.mark.parametrize("seed", [0, 1])
def test_finish_equals_hadamard(seed):
    y = np.random.default_rng(seed).standard_normal(N)
    out = finish(load(y))
    want = hadamard(N) @ y / np.sqrt(N)
    # every lane of a half holds the same head's row here, so the halves' lanes agree; the lower
    # half writes the columns whose bit 2 is clear, the upper half the others
    for half in range(2):
        part = out[32 * half:32 * (half + 1)]
        assert np.array_equal(np.isnan(part), np.broadcast_to(np.isnan(part[0]), part.shape))
        np.testing.assert_array_equal(part, np.broadcast_to(part[0], part.shape))
        written = ~np.isnan(part[0])
        assert np.array_equal(written, ((np.arange(N) >> 2) & 1) == half)
    got = np.where(np.isnan(out[0]), out[32], out[0])
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
