"""Counter-based random draws for the sampler -- TEST INFRASTRUCTURE (see the package
docstring).

The "ember internals" page, section "sampler", step 5, draws r uniform in [0, 1) from a
seeded generator without naming it. Draws made on the device need a generator that any
(position, batch row) can evaluate on its own, so the reading is a counter-based one:
Philox4x32-10 (J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel random numbers: as easy
as 1, 2, 3", SC'11), written here from its published definition, independently of the
device code:

* state: a counter of four 32-bit words and a key of two;
* one round: the products M0 * c0 and M1 * c2 (64-bit, split into high and low words)
  give the new counter (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0))
  with M0 = 0xD2511F53, M1 = 0xCD9E8D57;
* ten rounds, the key raised by the Weyl constants (0x9E3779B9, 0xBB67AE85) between
  consecutive rounds.

The draw of batch row b for the token predicted from the logits at position q is the
first output word of Philox4x32-10 at counter (q, b, 0, 0) and key (seed mod 2^32,
seed div 2^32), as u = (word >> 8) * 2^-24: 24 random bits, exactly representable in
f32, in [0, 1).

Pinned by the generator's published known-answer vectors (tests/test_oracle_rng.py).
"""
import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds. counter: four uint32 words (arrays broadcast), key: two.
    Returns the four output words as uint64 arrays holding 32-bit values."""
    c = [np.asarray(w, np.uint64) & MASK for w in counter]
    k0 = np.asarray(key[0], np.uint64) & MASK
    k1 = np.asarray(key[1], np.uint64) & MASK
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = np.uint64(M0) * c[0]               # < 2^64: no overflow in uint64
        p1 = np.uint64(M1) * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return c


def uniform(seed, pos, row):
    """The draw u in [0, 1) (float32) of batch row `row` at position `pos` (arrays
    broadcast) for `seed` (a 64-bit integer)."""
    seed = int(seed)
    pos = np.asarray(pos, np.uint64)
    row = np.asarray(row, np.uint64)
    zero = np.zeros_like(pos + row)
    w = philox4x32_10((pos + zero, row + zero, zero, zero), (seed & MASK, (seed >> 32) & MASK))[0]
    return ((w >> np.uint64(8)).astype(np.float64) * 2.0 ** -24).astype(np.float32)
