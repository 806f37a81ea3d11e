"""Philox4x64-10 and the draw layout used by the sampling ops (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The generator is written from its published definition (Salmon et al.,
"Parallel random numbers: as easy as 1, 2, 3", SC'11, Philox-4x64 with ten
rounds): each round multiplies counter words 0 and 2 by two fixed odd
constants, forms the 128-bit products, and permutes/xors the high and low
halves with the other counter words and the round key; the key is bumped by
two Weyl constants between rounds.

The pages ask that the random state belong to the request and that every
call advance it (FlashInfer Sorting-Free Sampling explainer, "Seed、offset 与
deterministic 的边界" and "动态 batch 中的 RNG 所有权").  The pages name no
generator; Philox is what the benchmark spec names.  Draw layout (a reading
of the pages, stated once here and in the C header):

    key     = (seed, 0)
    counter = (offset, sid, r // 4, 0)     r = 0, 1, 2, ... draw number
    word    = Philox4x64-10(counter, key)[r % 4]
    u_r     = (word >> 11) / 2**53          53-bit uniform in [0, 1)

``sid`` is the output index when one scalar seed serves the whole call and 0
when every output brings its own seed, so that an output's stream depends only
on its own (seed, offset) and not on its position in the batch.
"""

MASK64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B


def philox4x64_10(counter, key):
    """Return the four 64-bit output words of Philox4x64-10(counter, key)."""
    c0, c1, c2, c3 = (int(v) & MASK64 for v in counter)
    k0, k1 = (int(v) & MASK64 for v in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        prod0 = PHILOX_M0 * c0
        prod1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((prod1 >> 64) ^ c1 ^ k0, prod1 & MASK64,
                          (prod0 >> 64) ^ c3 ^ k1, prod0 & MASK64)
    return c0, c1, c2, c3


def draw_bits53(seed, offset, sid, r):
    """Integer a in [0, 2**53) such that the r-th uniform of a stream is a / 2**53."""
    words = philox4x64_10((offset, sid, r // 4, 0), (seed, 0))
    return words[r % 4] >> 11


def draw_uniform(seed, offset, sid, r):
    """The r-th uniform in [0, 1) of the stream (seed, offset, sid), as a float."""
    return draw_bits53(seed, offset, sid, r) / float(1 << 53)


class Stream:
    """Sequential view of one output's draws: ``next()`` returns a 53-bit integer."""

    def __init__(self, seed, offset, sid):
        self.seed, self.offset, self.sid = int(seed), int(offset), int(sid)
        self.used = 0

    def next(self):
        a = draw_bits53(self.seed, self.offset, self.sid, self.used)
        self.used += 1
        return a
