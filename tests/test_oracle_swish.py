"""Pins of the oracle's reproducible exponential, logistic and SwiGLU element.

The exponential is pinned to the mathematics: within 1 ulp of the correctly rounded
exp (float64 math.exp is accurate far below binary32 resolution) everywhere it is
finite, exact at 0, and saturating to +inf / 0 at the documented thresholds.  The
constants it uses are the nearest binary32 values of exact rationals, checked here with
exact rational arithmetic.  SwiGLU is pinned against torch's SiLU in float64 (gate =
first half, value = second half, modelpad.app MLP paragraph).
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import torch


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| in binary32 ulps of b (both finite float32 arrays)."""
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7fffffff), ia)
    ib = np.where(ib < 0, -(ib & 0x7fffffff), ib)
    return np.abs(ia - ib)


def nearest_f32(fr: Fraction) -> float:
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    return float(min(cands, key=lambda v: (abs(Fraction(float(v)) - fr),
                                            int(np.float32(v).view(np.uint32)) & 1)))


def test_exp_constants_are_nearest_binary32():
    """The hex literals in oracle.c are RN(1/n!), RN(log2 e), and the Cody-Waite split of ln 2."""
    getcontext().prec = 60
    ln2 = Fraction(str(Decimal(2).ln()))
    log2e = Fraction(str(1 / Decimal(2).ln()))
    src = open(__file__.replace("tests/test_oracle_swish.py", "oracle/oracle.c")).read()

    def lit(name):
        line = [l for l in src.splitlines() if f"float {name} =" in l][0]
        return float.fromhex(line.split("=")[1].strip().rstrip(";").rstrip("f"))

    assert lit("OR_LOG2E") == nearest_f32(log2e)
    for n in range(2, 8):
        assert lit(f"OR_C{n}") == nearest_f32(Fraction(1, math.factorial(n)))
    l1 = Fraction(lit("OR_L1"))
    assert abs(l1 - ln2) < Fraction(1, 2 ** 15)            # L1 is ln2 truncated
    assert (l1 * 2 ** 15).denominator == 1                  # 15 fractional bits
    assert lit("OR_L2") == nearest_f32(ln2 - l1)


def test_exp_accuracy_dense(orc):
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-104.0, 89.0, 2_000_000),
                        rng.uniform(-2, 2, 500_000),
                        np.linspace(-87.5, -86.5, 20001), np.linspace(88.0, 88.75, 20001)]).astype(np.float32)
    got = orc.exp(x)
    with np.errstate(over="ignore", under="ignore"):
        ref = np.exp(x.astype(np.float64))
    ref32 = ref.astype(np.float32)
    fin = np.isfinite(ref32) & (ref32 > np.float32(1.17549435e-38))
    assert ulp_diff(got[fin], ref32[fin]).max() <= 1
    sub = np.isfinite(ref32) & ~fin          # subnormal results: absolute error in units of 2^-149
    err = np.abs(got[sub].astype(np.float64) - ref[sub]) / 2.0 ** -149
    assert err.max() <= 1.0
    assert np.isinf(got[np.isinf(ref32)]).all()


def test_exp_special_values(orc):
    x = np.array([0.0, -0.0, 1.0, np.inf, -np.inf, np.nan, 89.5, -110.0, 88.0, -104.0], np.float32)
    y = orc.exp(x)
    assert y[0] == 1.0 and y[1] == 1.0
    assert abs(float(y[2]) - math.e) < 3e-7
    assert np.isinf(y[3]) and y[4] == 0.0 and np.isnan(y[5])
    assert np.isinf(y[6]) and y[7] == 0.0
    # exp(-104) = 6.8e-46 lies below half the smallest subnormal (7.0e-46): rounds to 0
    assert np.isfinite(y[8]) and y[9] == 0.0
    assert orc.exp(np.array([-103.0], np.float32))[0] == np.float32(math.exp(-103.0))  # 2^-149


def test_exp_monotone_on_bf16_grid(orc):
    h = np.arange(0, 0x7f80, dtype=np.uint32)
    x = np.concatenate([-(h[::-1] << 16).view(np.float32), (h << 16).view(np.float32)])
    y = orc.exp(x)
    assert (y[1:] >= y[:-1]).all()


def test_sigmoid_all_bf16_and_fp16(orc):
    h = np.arange(65536, dtype=np.uint32)
    xs = [(h << 16).view(np.float32), h.astype(np.uint16).view(np.float16).astype(np.float32)]
    for x in xs:
        x = x[np.isfinite(x)]
        got = orc.sigmoid(x)
        with np.errstate(over="ignore"):
            ref = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
        ref32 = ref.astype(np.float32)
        norm = ref32 > np.float32(1.17549435e-38)
        assert ulp_diff(got[norm], ref32[norm]).max() <= 2
        # subnormal sigma: accurate while exp(-a) is finite; beyond (a < -88.72) the
        # denominator overflows and sigma is exactly 0 by construction
        sub = ~norm & (x >= -88.72)
        assert (np.abs(got[sub].astype(np.float64) - ref[sub]) <= 2.0 ** -148).all()
        assert (got[x < -89.0] == 0).all()
    assert orc.sigmoid(np.array([0.0], np.float32))[0] == 0.5


def test_swiglu_gate_value_order_against_torch_silu(orc):
    rng = np.random.default_rng(1)
    gate = rng.standard_normal(100000).astype(np.float32) * 3
    value = rng.standard_normal(100000).astype(np.float32)
    got = orc.swiglu(gate, value).astype(np.float64)
    ref = (torch.nn.functional.silu(torch.from_numpy(gate).double()) * torch.from_numpy(value).double()).numpy()
    assert np.allclose(got, ref, rtol=3e-7, atol=1e-30)
    swapped = (torch.nn.functional.silu(torch.from_numpy(value).double()) * torch.from_numpy(gate).double()).numpy()
    assert not np.allclose(got, swapped, rtol=1e-2)
    assert (orc.swiglu(np.zeros(4, np.float32), np.ones(4, np.float32)) == 0).all()
