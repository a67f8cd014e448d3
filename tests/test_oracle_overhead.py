"""Pins for the storage arithmetic against the pages' worked numbers.

Fixture: tests/golden/overhead.json ("The Geometry of Forgetting", section
"The overhead nobody tells you about"; "QJL: 1-Bit Quantized JL Transform ...",
Abstract).
"""

import json
import os

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "overhead.json")


def load():
    with open(GOLDEN) as f:
        return json.load(f)


def test_page_worked_examples():
    g = load()
    for c in g["cases"]:
        eff = oracle.effective_bits_per_number(c["bits"], c["block"], g["zero_point_bits"],
                                               g["scale_bits"])
        assert eff == c["effective_bits"]
        if "overhead_fraction" in c:
            assert oracle.overhead_fraction(c["bits"], c["block"]) == c["overhead_fraction"]


def test_one_to_two_extra_bits():
    g = load()
    lo, hi = g["extra_bits_range"]
    extra = [oracle.effective_bits_per_number(0, b) for b in g["extra_bits_range_blocks"]]
    assert extra == [lo, hi]


def test_qjl_has_no_per_block_constants():
    g = load()
    assert oracle.qjl_per_block_constants() == g["qjl_per_block_constants"]
    # bytes stored are the sign bits plus one fp32 norm per key, for any block size
    assert oracle.qjl_stored_bytes(32768, 256) == 32768 * 36
    assert oracle.qjl_stored_bytes(65536, 512) == 65536 * 68
    assert oracle.qjl_bits_per_coordinate(128, 256) == 2.25
    assert oracle.qjl_bits_per_coordinate(128, 512) == 4.25
