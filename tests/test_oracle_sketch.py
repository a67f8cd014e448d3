"""Pins for the oracle's S generator and bf16 rounding.

S must have i.i.d. N(0,1) entries and be a deterministic function of the seed
("The Geometry of Forgetting", QJL section).  The bf16 rounding is checked on
hand-worked bit patterns.  Bit equality with the C library's own generator is
in test_abi_host.py.
"""

import math

import numpy as np
import pytest
from scipy import stats

import oracle
from oracle import qjl as oq


def test_bf16_rounding_hand_values():
    cases = {
        1.0: 0x3F80,
        -2.5: 0xC020,
        0.0: 0x0000,
        1.0 + 2.0 ** -8: 0x3F80,            # halfway, 0x3F80 is even -> stays
        1.0 + 3 * 2.0 ** -8: 0x3F82,        # halfway between 0x3F81 and 0x3F82 -> even
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,   # just above halfway -> up
        1.0 + 2.0 ** -8 - 2.0 ** -20: 0x3F80,   # just below halfway -> down
        # fp64 -> fp32 first: the 2^-30 tail is lost in fp32 (below half an fp32
        # ulp of 1), leaving an exact bf16 tie that goes to even.
        1.0 + 2.0 ** -8 + 2.0 ** -30: 0x3F80,
        65280.0: 0x477F,                    # 255 * 2^8, exact
    }
    for x, want in cases.items():
        got = int(oracle.float64_to_bf16_bits(np.array([x]))[0])
        assert got == want, (x, hex(got), hex(want))
    back = oracle.bf16_bits_to_float64(np.array([0x3F80, 0xC020, 0x477F], dtype=np.uint16))
    assert back.tolist() == [1.0, -2.5, 65280.0]


def test_uniform_map_is_open_at_zero():
    assert oq._uniform_open0_closed1(0) == 2.0 ** -53
    assert oq._uniform_open0_closed1((1 << 64) - 1) == 1.0


def test_sketch_deterministic_and_seed_dependent():
    a = oracle.sketch_bf16_bits(42, 16, 64)
    b = oracle.sketch_bf16_bits(42, 16, 64)
    c = oracle.sketch_bf16_bits(43, 16, 64)
    assert np.array_equal(a, b)
    assert (a != c).mean() > 0.9
    # the layout is [d][m]: a different (d, m) with the same element count
    # reads the same stream in the same element order
    flat = oracle.sketch_bf16_bits(42, 32, 32).reshape(-1)
    assert np.array_equal(a.reshape(-1), flat)


@pytest.mark.parametrize("seed", [42, 7, 2 ** 63 + 5])
def test_sketch_entries_are_standard_normal(seed):
    d, m = 128, 256
    z = oq._sketch_f64(seed, d, m).reshape(-1)
    n = z.size
    assert abs(z.mean()) < 4.0 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 4.0 * math.sqrt(2.0 / n)
    assert stats.kstest(z, "norm").pvalue > 1e-3
    # the two members of a Box-Muller pair are uncorrelated
    r = np.corrcoef(z[0::2], z[1::2])[0, 1]
    assert abs(r) < 4.0 / math.sqrt(n / 2)
    # neighbouring sketch columns are uncorrelated too
    S = z.reshape(d, m)
    r2 = np.corrcoef(S[:, :-1].reshape(-1), S[:, 1:].reshape(-1))[0, 1]
    assert abs(r2) < 4.0 / math.sqrt(n)


def test_sketch_bf16_is_rounding_of_normals():
    d, m = 64, 128
    z = oq._sketch_f64(42, d, m)
    s = oracle.sketch(42, d, m)
    rel = np.abs(s - z) / np.abs(z)
    assert rel.max() <= 2.0 ** -8 * (1 + 1e-6)
    assert np.all(np.sign(s) == np.sign(z))
