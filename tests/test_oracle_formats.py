"""Pins of the oracle's number formats against library routines and closed forms.

E4M3 and the bf16/fp16 widenings and roundings are checked exhaustively (or on dense
samples with every tie case) against torch/numpy conversions.  E2M1 has no library
conversion in this torch build, so a generic minifloat decoder is first validated on
E4M3 and E5M2 against torch and then used on the E2M1 field layout (1 sign, 2 exponent
bits with bias 1, 1 mantissa bit), together with the format's closed-form facts.
"""
import math

import numpy as np
import pytest
import torch


def minifloat(code: int, ebits: int, mbits: int, bias: int) -> float:
    """Generic sign/exponent/mantissa decoder (no inf/NaN handling)."""
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        v = (m / (1 << mbits)) * 2.0 ** (1 - bias)
    else:
        v = (1 + m / (1 << mbits)) * 2.0 ** (e - bias)
    return -v if s else v


def test_minifloat_decoder_matches_torch_fp8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    e4 = codes.view(torch.float8_e4m3fn).float().tolist()
    e5 = codes.view(torch.float8_e5m2).float().tolist()
    for c in range(256):
        if not math.isnan(e4[c]):
            assert minifloat(c, 4, 3, 7) == e4[c]
        if not (math.isnan(e5[c]) or math.isinf(e5[c])):
            assert minifloat(c, 5, 2, 15) == e5[c]


def test_e4m3_all_bytes_match_torch(orc):
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    got = np.array([orc.e4m3(b) for b in range(256)], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert nan.sum() == 2 and np.nanmax(got) == 448.0
    assert orc.e4m3(0x01) == 2.0 ** -9          # smallest subnormal


def test_e2m1_table(orc):
    vals = [orc.e2m1(c) for c in range(16)]
    for c in range(16):
        assert vals[c] == minifloat(c, 2, 1, 1)
    mags = sorted(set(abs(v) for v in vals))
    assert mags == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # 8 magnitudes, max 6
    for c in range(8):
        assert vals[c + 8] == -vals[c]                       # bit 3 is the sign


def test_bf16_widen_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan].view(np.uint32), got[~nan].view(np.uint32))


def test_fp16_widen_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.fp16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan].view(np.uint32), got[~nan].view(np.uint32))


def _narrowing_cases(seed=0):
    rng = np.random.default_rng(seed)
    x = [rng.standard_normal(200000).astype(np.float32),
         (rng.standard_normal(100000) * 1e-6).astype(np.float32),
         (rng.standard_normal(100000) * 3e4).astype(np.float32),
         (rng.standard_normal(50000) * 1e38).astype(np.float32),
         np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.99, 65520, 1e-8, 2 ** -24,
                   2 ** -25, 3 * 2 ** -26, 2 ** -149, 3.4e38], np.float32)]
    # exact ties between neighbouring bf16 / fp16 values, and their neighbours
    b = rng.integers(0, 0x7f00, 50000, dtype=np.uint32)
    ties16 = ((b << 16) | 0x8000).view(np.float32)
    h = rng.integers(0, 0x7bff, 50000, dtype=np.uint32).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    tiesh = ((lo + hi) / 2).astype(np.float32)
    x += [ties16, -ties16, tiesh, -tiesh, np.nextafter(tiesh, np.float32(0)),
          np.nextafter(tiesh, np.float32(np.inf))]
    return np.concatenate(x).astype(np.float32)


def test_f32_to_bf16_rne(orc):
    x = _narrowing_cases()
    got = orc.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    nan = orc.f32_to_bf16(np.array([np.nan], np.float32))
    assert np.isnan(orc.bf16_to_f32(nan)[0])


def test_f32_to_fp16_rne(orc):
    x = _narrowing_cases(1)
    got = orc.f32_to_fp16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    assert np.isnan(orc.fp16_to_f32(orc.f32_to_fp16(np.array([np.nan], np.float32)))[0])


def test_padded_k(orc):
    for k, kp in [(1, 256), (256, 256), (257, 512), (5376, 5376), (14336, 14336), (20000, 20224)]:
        assert orc.padded_k(k) == kp


if __name__ == "__main__":
    pytest.main([__file__, "-q"])
