"""The exact binary32 emulator used by the pins (tests/f32exact.py) against
numpy's IEEE binary32 arithmetic, which rounds every operation correctly:
random operand pairs over the whole finite range, subnormals included."""
import numpy as np

import f32exact as F


def _patterns(rng, n):
    b = rng.integers(0, 2 ** 32, 4 * n, dtype=np.uint64).astype(np.uint32)
    b = b[((b >> 23) & 0xFF) != 0xFF][:n]
    # plus values near 1e-3 and the subnormal range, where the step lives
    near = (rng.standard_normal(n // 4) * 1e-3).astype(np.float32).view(np.uint32)
    sub = rng.integers(1, 1 << 23, n // 4, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([b, near, sub])


def test_ops_match_numpy():
    rng = np.random.default_rng(7)
    a = _patterns(rng, 1500)
    b = _patterns(rng, 1500)
    b = b[rng.permutation(len(b))]
    af, bf = a.view(np.float32), b.view(np.float32)
    with np.errstate(all="ignore"):
        for name, fn in (("add", np.add), ("sub", np.subtract), ("mul", np.multiply),
                         ("div", np.divide)):
            ref = fn(af, bf).view(np.uint32)
            for i in range(len(a)):
                r = int(ref[i])
                if (name == "div" and bf[i] == 0) or ((r & 0x7F800000) == 0x7F800000 and r & 0x7FFFFF):
                    continue
                got = getattr(F, name)(int(a[i]), int(b[i]))
                if r & 0x7FFFFFFF == 0:          # the emulator does not track signed zeros
                    assert got & 0x7FFFFFFF == 0
                else:
                    assert got == r, (name, hex(a[i]), hex(b[i]), hex(got), hex(r))
        s = np.abs(af)
        ref = np.sqrt(s).view(np.uint32)
        for i in range(len(s)):
            if np.isfinite(s[i]):
                assert F.sqrt(int(s.view(np.uint32)[i])) == int(ref[i])


def test_rounding_boundaries():
    from fractions import Fraction
    one = F.from_decimal("1")
    assert one == 0x3F800000
    # halfway between 1 and the next binary32 rounds to even (down), just
    # above halfway rounds up
    assert F.encode(1 + Fraction(1, 1 << 24)) == 0x3F800000
    assert F.encode(1 + Fraction(3, 1 << 24)) == 0x3F800002
    assert F.encode(1 + Fraction(1, 1 << 24) + Fraction(1, 1 << 60)) == 0x3F800001
    # overflow and the smallest subnormal
    assert F.encode(Fraction(2) ** 128) == F.INF_BITS
    assert F.encode(Fraction(1, 1 << 149)) == 1
    assert F.encode(Fraction(1, 1 << 150)) == 0          # tie with 0: even
    assert F.from_decimal("0.9") == 0x3F666666 and F.from_decimal("0.95") == 0x3F733333
