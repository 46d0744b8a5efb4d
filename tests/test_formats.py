"""The oracle's number-format decoders against torch's conversions, over
every code of each format (an independent library implementation)."""
import numpy as np
import torch

from oracle import formats


def _same(a, b):
    a, b = np.asarray(a), np.asarray(b)
    nan = np.isnan(b)
    assert np.array_equal(np.isnan(a), nan)
    assert np.array_equal(a[~nan], b[~nan])
    # signed zeros match too
    assert np.array_equal(np.signbit(a[~nan]), np.signbit(b[~nan]))


def test_fp16_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.float16).double().numpy()
    _same(formats.decode_fp16(codes), ref)


def test_bf16_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    _same(formats.decode_bf16(codes), ref)


def test_e4m3fn_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    _same(formats.decode_e4m3fn(codes), ref)
    assert formats.decode_e4m3fn(np.array([0x7E], np.uint8))[0] == 448.0


def test_e4m3fn_encoder_round_trips_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = formats.decode_e4m3fn(codes)
    fin = np.isfinite(vals)
    back = formats.decode_e4m3fn(formats.encode_e4m3fn_rne(vals[fin]))
    assert np.array_equal(back, vals[fin])


def test_e4m3fn_encoder_ties_to_even_and_clamps():
    """Midpoints between neighbouring codes go to the even code (fraction
    bit 0), by hand: between 1.0 (0x38) and 1.125 (0x39) 1.0625 -> 1.0; between
    1.125 and 1.25 (0x3A) 1.1875 -> 1.25; in the subnormals between 2^-9 (0x01)
    and 2^-8 (0x02) 1.5 * 2^-9 -> 2^-8; beyond the range the encoder clamps to
    +-448 (0x7E / 0xFE), never NaN."""
    x = np.array([1.0625, 1.1875, 1.5 * 2.0 ** -9, 0.5 * 2.0 ** -9, 500.0, -1e9, 448.0, 464.0])
    got = formats.encode_e4m3fn_rne(x)
    assert got.tolist() == [0x38, 0x3A, 0x02, 0x00, 0x7E, 0xFE, 0x7E, 0x7E]
    # just off a midpoint the nearest value wins
    got = formats.encode_e4m3fn_rne(np.array([np.nextafter(1.0625, 2.0), np.nextafter(1.1875, 0.0)]))
    assert got.tolist() == [0x39, 0x39]


def test_e4m3fn_encoder_matches_torch_inside_the_range():
    """torch's float -> float8_e4m3fn cast (round to nearest even; NaN past
    the range, where the encoder clamps instead) on seeded float32 values of
    every magnitude within +-448."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000) * 100, rng.uniform(-448, 448, 100000),
                        rng.standard_normal(100000) * 1e-3]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = formats.encode_e4m3fn_rne(x.astype(np.float64))
    assert np.array_equal(formats.decode_e4m3fn(got), formats.decode_e4m3fn(ref))
