"""64-bit Mersenne Twister (MT19937-64), from its published definition.

Parameters (Nishimura, "Tables of 64-bit Mersenne Twisters", ACM TOMACS 10,
2000; also fixed by the C++ standard for ``std::mt19937_64``): word size 64,
state 312 words, middle word 156, separation point 31, twist matrix
0xB5026F5AA96619E9, tempering (u, d) = (29, 0x5555555555555555),
(s, b) = (17, 0x71D67FFFEDA60000), (t, c) = (37, 0xFFF7EEE000000000), l = 43,
initialisation multiplier 6364136223846793005.

The state update is vectorised with numpy in three slices that respect the
recurrence's data dependencies; the output sequence is identical to the
element-by-element definition (checked against g++'s std::mt19937_64).
"""
import numpy as np

_N, _M = 312, 156
_A = np.uint64(0xB5026F5AA96619E9)
_UPPER = np.uint64(0xFFFFFFFF80000000)
_LOWER = np.uint64(0x000000007FFFFFFF)
_MASK64 = (1 << 64) - 1


class MT19937_64:
    def __init__(self, seed: int = 5489):
        mt = [0] * _N
        mt[0] = seed & _MASK64
        for i in range(1, _N):
            prev = mt[i - 1]
            mt[i] = (6364136223846793005 * (prev ^ (prev >> 62)) + i) & _MASK64
        self._mt = np.array(mt, dtype=np.uint64)
        self._buf = np.empty(0, np.uint64)
        self._pos = 0

    def _twist(self):
        mt = self._mt
        one = np.uint64(1)
        # i in [0, N-M): reads mt[i+1] and mt[i+M], all still old.
        i = np.arange(0, _N - _M)
        y = (mt[i] & _UPPER) | (mt[i + 1] & _LOWER)
        mt[i] = mt[i + _M] ^ (y >> one) ^ np.where((y & one) != 0, _A, np.uint64(0))
        # i in [N-M, N-1): reads mt[i+1] (old) and mt[i+M-N] (already new).
        i = np.arange(_N - _M, _N - 1)
        y = (mt[i] & _UPPER) | (mt[i + 1] & _LOWER)
        mt[i] = mt[i + _M - _N] ^ (y >> one) ^ np.where((y & one) != 0, _A, np.uint64(0))
        # i = N-1: reads mt[0] and mt[M-1], both new.
        y = (mt[_N - 1] & _UPPER) | (mt[0] & _LOWER)
        mt[_N - 1] = mt[_M - 1] ^ (y >> one) ^ (_A if (int(y) & 1) else np.uint64(0))
        # tempering of the whole block
        z = mt.copy()
        z ^= (z >> np.uint64(29)) & np.uint64(0x5555555555555555)
        z ^= (z << np.uint64(17)) & np.uint64(0x71D67FFFEDA60000)
        z ^= (z << np.uint64(37)) & np.uint64(0xFFF7EEE000000000)
        z ^= z >> np.uint64(43)
        self._buf = z
        self._pos = 0

    def next_u64(self, n: int) -> np.ndarray:
        """The next n outputs as uint64."""
        out = np.empty(n, np.uint64)
        k = 0
        while k < n:
            if self._pos >= self._buf.size:
                self._twist()
            take = min(n - k, self._buf.size - self._pos)
            out[k:k + take] = self._buf[self._pos:self._pos + take]
            self._pos += take
            k += take
        return out


def uniform01(gen: MT19937_64, n: int) -> np.ndarray:
    """n doubles uniform in [0, 1): the top 53 bits of each output times 2**-53."""
    x = gen.next_u64(n)
    return (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
