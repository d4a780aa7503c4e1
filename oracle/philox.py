"""Philox4x32-10 and the decode-step uniforms (oracle; test infrastructure only).

Philox4x32-R is the counter-based generator of Salmon, Moraes, Dror and Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).  One round maps a
128-bit counter (c0, c1, c2, c3) under a 64-bit key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with M0 = 0xD2511F53, M1 = 0xCD9E8D57; between rounds the key is bumped by the
Weyl constants (0x9E3779B9, 0xBB67AE85).  Ten rounds are applied.  Pinned by
the generator's published known-answer vectors (tests/golden/philox4x32_10_kat.txt).

The method needs a uniform u ~ U(0,1) for every acceptance test and every
categorical draw (wiki note, section *Method*: a uniform draw compared with p(x)/q(x)).
The pages do not say how it is drawn; the reading taken here is a counter-based
stream so that two implementations draw identical numbers:

    key     = (seed mod 2^32, seed >> 32)
    counter = (slot, t, position, purpose)      purpose 0 = accept test, 1 = draw
    u       = ((word0 >> 8) + 0.5) * 2^-24      in the open interval (0, 1)

``t`` is the per-slot pass counter (0 for prefill), ``position`` the absolute
sequence position of the token being tested or drawn.
"""
import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint64(0x9E3779B9)
W1 = np.uint64(0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)
ROUNDS = 10


def philox4x32(counter, key, rounds=ROUNDS):
    """Philox4x32-R on arrays of counters.

    counter: uint32-compatible array [..., 4]; key: uint32-compatible array [..., 2]
    (broadcast against counter).  Returns uint32 array [..., 4].
    """
    c = np.asarray(counter, dtype=np.uint64) & MASK32
    k = np.asarray(key, dtype=np.uint64) & MASK32
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0 = np.broadcast_to(k[..., 0], c0.shape).copy()
    k1 = np.broadcast_to(k[..., 1], c0.shape).copy()
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = M0 * c0            # < 2^64: exact in uint64
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def key_of_seed(seed):
    seed = int(seed)
    return np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)


def uniform(seed, slot, t, position, purpose):
    """u(slot, t, position, purpose) in (0, 1) as float64 (an odd multiple of 2^-25, exact in float64).

    All four counter fields broadcast; returns an array of that broadcast shape
    (a Python float when every argument is a scalar).
    """
    slot, t, position, purpose = np.broadcast_arrays(
        np.asarray(slot, dtype=np.int64), np.asarray(t, dtype=np.int64),
        np.asarray(position, dtype=np.int64), np.asarray(purpose, dtype=np.int64))
    ctr = np.stack([slot, t, position, purpose], axis=-1).astype(np.uint64) & MASK32
    w = philox4x32(ctr, key_of_seed(seed))
    u = ((w[..., 0] >> np.uint32(8)).astype(np.float64) + 0.5) * (2.0 ** -24)
    if u.shape == ():
        return float(u)
    return u


PURPOSE_ACCEPT = 0
PURPOSE_DRAW = 1
