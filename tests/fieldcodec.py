"""Bit-field decoder for IEEE-style binary formats, written from the format
definitions (sign, biased exponent, fraction).  Used to pin the oracle's
decoders and to build exact references independent of them."""


def decode_fields(bits: int, exp_bits: int, frac_bits: int) -> float:
    """Value of a (1 + exp_bits + frac_bits)-bit IEEE-style pattern."""
    sign = -1.0 if (bits >> (exp_bits + frac_bits)) & 1 else 1.0
    e = (bits >> frac_bits) & ((1 << exp_bits) - 1)
    f = bits & ((1 << frac_bits) - 1)
    bias = (1 << (exp_bits - 1)) - 1
    if e == (1 << exp_bits) - 1:
        return sign * float("inf") if f == 0 else float("nan")
    if e == 0:
        return sign * f * 2.0 ** (1 - bias - frac_bits)
    return sign * (1 + f / float(1 << frac_bits)) * 2.0 ** (e - bias)


def fp16(bits: int) -> float:
    return decode_fields(int(bits), 5, 10)


def bf16(bits: int) -> float:
    return decode_fields(int(bits), 8, 7)
