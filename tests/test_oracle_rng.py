"""Pins of the oracle's counter-based generator (Philox4x32-10, Salmon et al., SC'11):
the generator's published known-answer vectors, and the distribution of the derived
uniform draws."""
import numpy as np

from oracle.rng import philox4x32_10, uniform

# (counter, key) -> output words, the known-answer vectors published with the generator
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


def test_known_answers():
    for ctr, key, want in KAT:
        got = tuple(int(w) for w in philox4x32_10(ctr, key))
        assert got == want, [hex(g) for g in got]


def test_vectorised_equals_scalar():
    pos = np.arange(40) * 7919
    rows = np.arange(40) % 5
    out = philox4x32_10((pos, rows, 0, 0), (12345, 678))
    for i in range(40):
        one = philox4x32_10((int(pos[i]), int(rows[i]), 0, 0), (12345, 678))
        assert all(int(out[j][i]) == int(one[j]) for j in range(4))


def test_uniform_draws():
    pos, row = np.meshgrid(np.arange(4096), np.arange(16), indexing="ij")
    u = uniform(2024, pos, row).ravel()
    assert u.dtype == np.float32
    assert (u >= 0).all() and (u < 1).all()
    # 24 random bits: every draw a multiple of 2^-24
    assert np.array_equal(u.astype(np.float64) * 2**24, np.floor(u.astype(np.float64) * 2**24))
    # mean and a 64-bin chi-square within generous bounds for 65536 draws
    assert abs(u.mean() - 0.5) < 0.01
    counts = np.bincount((u * 64).astype(int), minlength=64)
    chi2 = ((counts - u.size / 64) ** 2 / (u.size / 64)).sum()
    assert chi2 < 120                           # 63 degrees of freedom
    # another seed, position or row gives other draws
    assert not np.array_equal(uniform(2025, pos, row).ravel(), u)
    assert uniform(7, 3, 1) != uniform(7, 1, 3)
