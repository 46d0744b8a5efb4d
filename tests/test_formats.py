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
