"""Storage arithmetic: per-block quantization overhead vs QJL (test infrastructure).

"The Geometry of Forgetting: How Three Papers Cracked KV Cache Quantization",
section "The overhead nobody tells you about": a block quantizer stores a
full-precision zero point and scale for every block, so a b-bit code with
block size B costs b + (bits of zero point + bits of scale) / B bits per
number.  The page works the 4-bit, block-64 case (5 bits) and the 2-bit,
block-64 case (the constants are half the budget).  "QJL: 1-Bit Quantized JL
Transform for KV Cache Quantization with Zero Overhead", Abstract: the
constants add 1 or 2 bits per number depending on the block, and QJL stores
none.

Parity pinned by the page's worked numbers (``tests/golden/overhead.json``).
"""

from __future__ import annotations


def effective_bits_per_number(bits: float, block: int, zero_point_bits: int = 32,
                              scale_bits: int = 32) -> float:
    """Bits per stored number for a block quantizer with per-block constants."""
    if block <= 0:
        raise ValueError("block must be positive")
    return bits + (zero_point_bits + scale_bits) / block


def overhead_fraction(bits: float, block: int, zero_point_bits: int = 32,
                      scale_bits: int = 32) -> float:
    """Per-block constants as a fraction of the nominal code budget."""
    return (effective_bits_per_number(bits, block, zero_point_bits, scale_bits) - bits) / bits


def qjl_per_block_constants() -> int:
    """QJL stores no zero point and no scale: zero constants per block."""
    return 0


def qjl_stored_bytes(num_keys: int, m: int, norm_bytes: int = 4) -> int:
    """Bytes stored for num_keys QJL keys: m sign bits plus one fp32 norm each."""
    if m % 8:
        raise ValueError("m must be a multiple of 8")
    return num_keys * (m // 8 + norm_bytes)


def qjl_bits_per_coordinate(d: int, m: int, norm_bits: int = 32) -> float:
    """Stored bits per key coordinate: (m sign bits + the norm) / d."""
    return (m + norm_bits) / d
