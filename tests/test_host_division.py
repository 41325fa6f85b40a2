"""The multiply-shift division used on the device to recover (slot, rank)
from a lattice row index: floor(m / d) = (m * ceil(2^38 / d)) >> 38 for any
32-bit m and 1 <= d <= 64, evaluated in 64-bit pieces exactly as
`div_by` in csrc/kernels.hpp does. Pinned against Python's integer division
on every divisor, at the edges of every quotient and on random numerators."""
import numpy as np
import pytest

MASK64 = (1 << 64) - 1


def div_magic(d: int) -> int:
    return ((1 << 38) + d - 1) // d


def div_by(m: int, magic: int) -> int:
    # the device form: two 32 x 32 -> 64-bit products, each kept to 64 bits
    lo, hi = magic & 0xFFFFFFFF, magic >> 32
    t = ((m * hi) & MASK64) + (((m * lo) & MASK64) >> 32)
    return ((t & MASK64) >> 6) & 0xFFFFFFFF


@pytest.mark.parametrize("d", range(1, 65))
def test_division_exact_for_32_bit_numerators(d):
    mg = div_magic(d)
    assert mg < (1 << 64)
    rng = np.random.default_rng(d)
    ms = set(int(x) for x in rng.integers(0, 1 << 32, 4000, dtype=np.uint64))
    ms |= {0, 1, d - 1, d, d + 1, (1 << 32) - 1, (1 << 31), (1 << 31) - 1}
    # both sides of every multiple near the top of the range and near zero
    for q in list(range(0, 2000)) + [((1 << 32) - 1) // d - k for k in range(2000)]:
        for off in (-1, 0, 1):
            m = q * d + off
            if 0 <= m < (1 << 32):
                ms.add(m)
    for m in ms:
        assert div_by(m, mg) == m // d, (m, d)


def test_row_decomposition():
    # row m = (n B + s) K + j of a lattice: rank j and slot s recovered
    for B, K in [(16, 8), (16, 16), (16, 32), (15, 7), (64, 8), (2, 64), (1, 1), (33, 9)]:
        mk, mb = div_magic(K), div_magic(B)
        for m in list(range(0, 5000)) + [(1 << 30) + 12345, (1 << 31) + 7]:
            q = div_by(m, mk)
            j = m - q * K
            s = q - div_by(q, mb) * B
            assert (j, s) == (m % K, (m // K) % B)
