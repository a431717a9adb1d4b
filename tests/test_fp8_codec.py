"""Pins of the oracle's OCP e4m3fn codec: the format definition's closed
forms, and torch's float8_e4m3fn conversion (a library routine) over every
bf16 bit pattern and a large random float32 sample.  CPU only."""
import numpy as np
import torch

from oracle import rpa_oracle as O


def torch_encode(x32: np.ndarray, scale: float) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x32, dtype=np.float32))
    return torch.clamp(t / scale, -448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(codes[nan]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_closed_forms():
    # largest finite 1.75 * 2^8 = 448 -> 0x7E; clamped values stay 448
    assert O.quantize_e4m3(np.array([448.0, 449.0, 1e4, -1e4]), 1.0).tolist() == \
        [0x7E, 0x7E, 0x7E, 0xFE]
    # 17 is halfway between 16 (0x58) and 18 (0x59): even code 0x58; 19 -> 20 (0x5A)
    assert O.quantize_e4m3(np.array([17.0, 19.0]), 1.0).tolist() == [0x58, 0x5A]
    # smallest subnormal 2^-9 = code 1; half of it ties to 0; 1.5 * 2^-9 ties to code 2
    assert O.quantize_e4m3(np.array([2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10]), 1.0).tolist() == \
        [1, 0, 2]
    # signed zero and NaN
    assert O.quantize_e4m3(np.array([0.0, -0.0, np.nan]), 1.0).tolist() == [0x00, 0x80, 0x7F]
    # min normal 2^-6 = 0x08; 1.0 = 0x38
    assert O.quantize_e4m3(np.array([2.0 ** -6, 1.0]), 1.0).tolist() == [0x08, 0x38]


def test_encode_every_bf16_pattern_matches_torch():
    pats = np.arange(65536, dtype=np.uint32)
    x = (pats << 16).view(np.float32)
    finite = np.isfinite(x)
    ours = O.quantize_e4m3(x[finite], 1.0)
    ref = torch_encode(x[finite], 1.0)
    np.testing.assert_array_equal(ours, ref)


def test_encode_random_fp32_with_scales_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(2_000_000) * np.exp(rng.uniform(-12, 8, 2_000_000))).astype(np.float32)
    for scale in (1.0, 0.05, 3.7, 1e-3):
        np.testing.assert_array_equal(O.quantize_e4m3(x, scale), torch_encode(x, scale))
