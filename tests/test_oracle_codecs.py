"""Pins of the oracle's storage decoders against torch's CPU casts (an independent library implementation of the
IEEE binary32, bfloat16 and OCP FP8 E4M3 formats)."""
import numpy as np
import torch

from oracle import sa_oracle as O


def test_e4m3_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.decode_e4m3(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_array_equal(got[m], ref[m])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0


def test_bf16_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.decode_bf16(codes)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_array_equal(got[m], ref[m])


def test_f32_sample():
    x = np.random.default_rng(0).normal(size=1000).astype(np.float32)
    np.testing.assert_array_equal(O.decode_f32(x.view(np.uint32)), x.astype(np.float64))
