"""Number-format decoders of the oracle, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Each decoder turns stored bit patterns into exact float64 values:

* IEEE 754 binary16 (fp16): 1 sign bit, 5 exponent bits (bias 15),
  10 fraction bits; exponent 0 is subnormal, exponent 31 is inf/NaN.
* bfloat16: the upper half of an IEEE binary32: 1 sign bit, 8 exponent
  bits (bias 127), 7 fraction bits; exponent 0 is subnormal, 255 inf/NaN.
* OCP FP8 E4M3 "fn" (finite): 1 sign bit, 4 exponent bits (bias 7),
  3 fraction bits; exponent 0 is subnormal; only the all-ones pattern
  S.1111.111 is NaN; there is no infinity, so the largest value is 448.

The K/V dtypes of the workloads (fp16, bf16, fp8 e4m3 with a per-KV-head
scale) are the ones the Quest page (§2, eq. (9)-(11), FP16 KV) and the
PageWeaver notes (FP8 E4M3 KV with BF16 queries) name.  fp32 inputs need
no decoder.

One encoder: real values to E4M3 "fn" codes by round-to-nearest, ties to
the even code (the code whose lowest fraction bit is 0), after clamping to
the finite range [-448, 448]; it picks among the decoded finite values, so it
shares nothing with the decoder but the table of codes.
"""
import numpy as np


def _decode_ieee(bits, exp_bits, frac_bits, has_inf=True):
    """Generic sign/exponent/fraction decoder to float64, one element at a time
    in vectorised form.  ``bits`` is an unsigned integer array."""
    bits = np.asarray(bits).astype(np.int64)
    bias = (1 << (exp_bits - 1)) - 1
    sign = np.where((bits >> (exp_bits + frac_bits)) & 1, -1.0, 1.0)
    e = (bits >> frac_bits) & ((1 << exp_bits) - 1)
    f = (bits & ((1 << frac_bits) - 1)).astype(np.float64)
    scale = float(1 << frac_bits)
    normal = sign * np.ldexp(1.0 + f / scale, (e - bias).astype(np.int64))
    subnormal = sign * np.ldexp(f / scale, 1 - bias)
    out = np.where(e == 0, subnormal, normal)
    e_max = (1 << exp_bits) - 1
    if has_inf:
        special = np.where(f == 0, sign * np.inf, np.nan)
        out = np.where(e == e_max, special, out)
    return out


def decode_fp16(bits):
    """IEEE binary16 bit patterns (uint16) -> float64."""
    return _decode_ieee(np.asarray(bits, dtype=np.uint16), 5, 10)


def decode_bf16(bits):
    """bfloat16 bit patterns (uint16) -> float64."""
    return _decode_ieee(np.asarray(bits, dtype=np.uint16), 8, 7)


def decode_e4m3fn(codes):
    """OCP FP8 E4M3 (finite-only variant) codes (uint8) -> float64."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = _decode_ieee(codes, 4, 3, has_inf=False)
    nan = (codes.astype(np.int64) & 0x7F) == 0x7F
    return np.where(nan, np.nan, out)


_TABLES = {}


def _table(dtype):
    """Every code of a 16- or 8-bit format decoded once by the decoders above;
    decoding a large array is then a table lookup (same values)."""
    if dtype not in _TABLES:
        if dtype == "f16":
            _TABLES[dtype] = decode_fp16(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16))
        elif dtype == "bf16":
            _TABLES[dtype] = decode_bf16(np.arange(1 << 16, dtype=np.uint32).astype(np.uint16))
        else:
            _TABLES[dtype] = decode_e4m3fn(np.arange(256, dtype=np.uint8))
    return _TABLES[dtype]


def decode(raw, dtype):
    """Decode a stored array of the named dtype ('f32', 'f16', 'bf16', 'e4m3')
    to float64.  'f16' arrays may be given as numpy float16 or uint16 bits."""
    raw = np.asarray(raw)
    if dtype == "f32":
        return raw.astype(np.float32).astype(np.float64)
    if dtype == "f16":
        if raw.dtype == np.float16:
            raw = raw.view(np.uint16)
        return _table("f16")[raw]
    if dtype == "bf16":
        return _table("bf16")[raw.view(np.uint16)]
    if dtype == "e4m3":
        return _table("e4m3")[raw.view(np.uint8)]
    raise ValueError(f"unknown dtype {dtype!r}")


def _e4m3_code_table():
    """(sorted distinct finite values, the code of each) of E4M3 fn; zero is
    the +0 code."""
    codes = np.arange(256, dtype=np.uint8)
    vals = decode_e4m3fn(codes)
    keep = np.isfinite(vals) & ~((codes == 0x80))       # one zero: +0
    order = np.argsort(vals[keep], kind="stable")
    return vals[keep][order], codes[keep][order]


def encode_e4m3fn_rne(x):
    """Real values (float64 array) -> E4M3 fn codes (uint8): clamp to
    [-448, 448], then the nearest finite value, a tie going to the even code.
    NaN input is not allowed (the writers never produce it)."""
    vals, codes = _e4m3_code_table()
    x = np.clip(np.asarray(x, np.float64), -448.0, 448.0)
    assert not np.isnan(x).any(), "NaN has no rounding"
    hi = np.clip(np.searchsorted(vals, x, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    exact = vals[hi] == x
    d_lo = x - vals[lo]
    d_hi = vals[hi] - x
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    pick = np.where(exact | take_hi, hi, lo)
    return codes[pick].astype(np.uint8)
