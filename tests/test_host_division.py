"""The cache writer divides the rANS state by a symbol frequency with a
multiply-high and a shift, floor(x / f) = (x * magic) >> (31 + s) for states
x < 2^24, where s = floor(log2 f) and the magic is ceil(2^(31+s) / f) raised
by less than 32 so that its low 5 bits hold the shift s - 1 (the library's
table set-up). These checks pin that rule for every frequency a table can
hold (2 <= f <= 1024) at the states where an overestimate would first show:
x = q f - 1 for every q, and the top state 2^24 - 1."""
import numpy as np

STATE_TOP = 1 << 24


def packed_magic(f: int) -> tuple[int, int]:
    s = f.bit_length() - 1
    magic = -(-(1 << (31 + s)) // f)
    magic += ((s - 1) - magic) & 31
    return magic, s - 1


def test_packed_magic_fits_and_carries_its_shift():
    for f in range(2, 1025):
        magic, shift = packed_magic(f)
        assert magic < 1 << 32 and magic & 31 == shift
        assert magic * f >= 1 << (31 + shift + 1)   # never below 2^(31+s) / f


def test_packed_magic_divides_exactly_below_two_to_the_24():
    for f in range(2, 1025):
        magic, shift = packed_magic(f)
        q = np.arange(1, (STATE_TOP - 1) // f + 1, dtype=np.uint64)
        x = np.concatenate([q * np.uint64(f) - np.uint64(1), q * np.uint64(f),
                            np.array([STATE_TOP - 1], dtype=np.uint64)])
        x = x[x < STATE_TOP]
        got = ((x * np.uint64(magic)) >> np.uint64(32)) >> np.uint64(shift)
        assert np.array_equal(got, x // np.uint64(f)), f
