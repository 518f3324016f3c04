"""Philox4x32-10 and the uniform conversions of the sampler contract (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source of the generator: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, section on the Philox
family (N=4 words of W=32 bits, R=10 rounds), with the constants and word
order of the authors' Random123 distribution, whose known-answer vectors pin
this module (``tests/golden/philox4x32_10_kat.txt``).

The pages on DFlash 2 name no generator at all; they only say the sampler
preserves the target distribution (P1 "DFlash 2: Block diffusion, wearing a
drafter's coat", section "Lossless, with conditions I did not used to state").
A counter-based generator keyed by (stream seed) and indexed by (cycle,
position, slot) is a reading of the pages: it makes every draw independent of
every decision ("non-anticipating"), and makes resuming at any cycle exact.

Definition used here.  State: four 32-bit counter words x0..x3 and two 32-bit
key words k0, k1.  One round computes the two 64-bit products M0*x0 and M1*x2,
and the new words are
    x0' = hi(M1*x2) ^ x1 ^ k0,   x1' = lo(M1*x2),
    x2' = hi(M0*x0) ^ x3 ^ k1,   x3' = lo(M0*x0).
Between rounds the key is advanced by the Weyl constants (k0 += W0, k1 += W1,
mod 2^32).  Ten rounds, the first with the key as given.
"""

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(key, ctr):
    """One Philox4x32-10 block: ``key`` = (k0, k1), ``ctr`` = (x0, x1, x2, x3).

    Pure-Python integers; returns a tuple of four ints in [0, 2^32).
    """
    k0, k1 = int(key[0]) & _MASK, int(key[1]) & _MASK
    x0, x1, x2, x3 = (int(c) & _MASK for c in ctr)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + W0) & _MASK
            k1 = (k1 + W1) & _MASK
        p0 = M0 * x0
        p1 = M1 * x2
        x0, x1, x2, x3 = ((p1 >> 32) ^ x1 ^ k0, p1 & _MASK,
                          (p0 >> 32) ^ x3 ^ k1, p0 & _MASK)
    return (x0, x1, x2, x3)


def philox4x32_10_np(k0, k1, x0, x1, x2, x3):
    """Vectorised form of :func:`philox4x32_10` over broadcastable arrays.

    All arguments are integer arrays (any width); arithmetic is carried in
    uint64 with explicit masking.  Returns four uint64 arrays of 32-bit words.
    """
    m = np.uint64(_MASK)
    k0 = np.asarray(k0, dtype=np.uint64) & m
    k1 = np.asarray(k1, dtype=np.uint64) & m
    x0 = np.asarray(x0, dtype=np.uint64) & m
    x1 = np.asarray(x1, dtype=np.uint64) & m
    x2 = np.asarray(x2, dtype=np.uint64) & m
    x3 = np.asarray(x3, dtype=np.uint64) & m
    x0, x1, x2, x3, k0, k1 = np.broadcast_arrays(x0, x1, x2, x3, k0, k1)
    x0, x1, x2, x3, k0, k1 = (a.copy() for a in (x0, x1, x2, x3, k0, k1))
    sh = np.uint64(32)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(W0)) & m
            k1 = (k1 + np.uint64(W1)) & m
        p0 = np.uint64(M0) * x0          # < 2^64, exact in uint64
        p1 = np.uint64(M1) * x2
        x0, x1, x2, x3 = (((p1 >> sh) ^ x1 ^ k0) & m, p1 & m,
                          ((p0 >> sh) ^ x3 ^ k1) & m, p0 & m)
    return x0, x1, x2, x3


def stream_block(seed, cycle, position, slot):
    """The four words drawn for (stream seed, cycle, position, slot).

    Key = (low, high) 32-bit halves of the 64-bit stream seed; counter =
    (cycle low, cycle high, position, slot).  Positions are 1-based block
    positions (1..L+1); slot 0 carries the trace and accept draws of that
    position, slot 1 the two draws of the residual/bonus sample.
    """
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    cycle = int(cycle) & 0xFFFFFFFFFFFFFFFF
    return philox4x32_10((seed & _MASK, seed >> 32),
                         (cycle & _MASK, cycle >> 32, position, slot))


def u01_f32(word):
    """Uniform in (0, 1) from one 32-bit word, exactly representable in fp32.

    Keeps the top 23 bits k and returns (2k + 1) / 2^24: an odd multiple of
    2^-24 below 1, so it has at most 24 significant bits and converts to
    float32 without rounding.  Returned as a Python float (float64).
    """
    k = (int(word) & _MASK) >> 9
    return (2 * k + 1) / float(1 << 24)


def u01_f64(word_hi, word_lo):
    """Uniform in (0, 1) from two 32-bit words, exactly representable in fp64.

    Forms the 64-bit value hi:lo, keeps its top 52 bits k and returns
    (2k + 1) / 2^53, which has at most 53 significant bits.
    """
    v = ((int(word_hi) & _MASK) << 32) | (int(word_lo) & _MASK)
    k = v >> 12
    return (2 * k + 1) / float(1 << 53)
