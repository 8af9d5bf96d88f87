"""java.util.Random, written from its published specification (Java SE API docs).

Test helper only: the worked examples on "Building Q8_0 and Q4_0 Like ggml"
(Examples 10, 11, 13) draw their inputs with java.util.Random(seed), so
re-creating that generator lets the tests reproduce the printed outputs.

Specification used:
  - seed scrambling: (seed ^ 0x5DEECE66D) & (2^48 - 1)
  - next(bits): seed = (seed * 0x5DEECE66D + 0xB) & (2^48 - 1);
                return (int)(seed >>> (48 - bits))   (as a signed 32-bit int)
  - nextInt(bound): power of two -> (int)((bound * (long)next(31)) >> 31);
                    otherwise rejection on next(31) with 32-bit overflow test
  - nextDouble(): ((long)next(26) << 27) + next(27)) * 2^-53
  - nextGaussian(): Marsaglia polar method with one cached value,
                    multiplier StrictMath.sqrt(-2 * StrictMath.log(s) / s)
"""
import math

_MULT = 0x5DEECE66D
_ADD = 0xB
_MASK = (1 << 48) - 1


def _to_int32(v):
    v &= 0xFFFFFFFF
    return v - (1 << 32) if v & 0x80000000 else v


class JavaRandom:
    def __init__(self, seed):
        self.seed = (seed ^ _MULT) & _MASK
        self._next_gaussian = None

    def next(self, bits):
        self.seed = (self.seed * _MULT + _ADD) & _MASK
        return _to_int32(self.seed >> (48 - bits))

    def next_int(self, bound):
        if bound <= 0:
            raise ValueError("bound must be positive")
        r = self.next(31)
        m = bound - 1
        if bound & m == 0:
            return _to_int32((bound * r) >> 31)
        u = r
        while True:
            r = u % bound
            if _to_int32(u - r + m) >= 0:
                return r
            u = self.next(31)

    def next_double(self):
        return ((self.next(26) << 27) + self.next(27)) * (1.0 / (1 << 53))

    def next_gaussian(self):
        if self._next_gaussian is not None:
            g = self._next_gaussian
            self._next_gaussian = None
            return g
        while True:
            v1 = 2 * self.next_double() - 1
            v2 = 2 * self.next_double() - 1
            s = v1 * v1 + v2 * v2
            if 0 < s < 1:
                break
        mul = math.sqrt(-2 * math.log(s) / s)
        self._next_gaussian = v2 * mul
        return v1 * mul
