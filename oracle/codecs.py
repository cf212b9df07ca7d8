"""Storage decoders used by the oracle (fp64 results).  TEST INFRASTRUCTURE ONLY.

* bf16: the upper 16 bits of an IEEE binary32 word; widening is exact.
* FP8 E4M3 as OCP "E4M3FN": 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
  bits, no infinities, codes 0x7F / 0xFF are NaN, largest finite 448.  The
  Step-3 report (section 4.1) runs attention in FP8, and the Step-5 page
  rounds its indexer operands to E4M3; neither page spells out the encoding,
  so the OCP definition is taken as written in its specification:
    exponent field e > 0:  (-1)^s * 2^(e-7) * (1 + m/8)
    exponent field e = 0:  (-1)^s * 2^(-6) * (m/8)
  Every one of the 256 codes is exact in fp64.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Widen bf16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_codes_to_f64(codes):
    """Decode OCP E4M3FN byte codes (uint8) to float64 from the field formula."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    exp = (c >> 3) & 0xF
    man = c & 0x7
    normal = (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    subnormal = (man / 8.0) * 2.0 ** -6
    mag = np.where(exp == 0, subnormal, normal)
    val = np.where(sign == 1, -mag, mag)
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return val.astype(np.float64)


def decode_storage(raw, fmt):
    """Decode a raw storage array: fmt in {"f32", "bf16", "e4m3"}, or "f64" for
    values that are already exact (the query path's fp64 output handed to the
    attention unrounded when the two steps are checked as one chain)."""
    if fmt == "f64":
        return np.asarray(raw, dtype=np.float64)
    if fmt == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if fmt == "bf16":
        return bf16_bits_to_f64(raw)
    if fmt == "e4m3":
        return e4m3fn_codes_to_f64(raw)
    raise ValueError(f"unknown storage format {fmt!r}")
