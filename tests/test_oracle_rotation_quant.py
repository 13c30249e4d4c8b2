"""Pins of the oracle's ConvRot256 rotation and row quantizer.

Rotation: for integer inputs |x| <= 2^15 every butterfly of the binary32 transform is
exact, so 16 * rotate(x) must equal the int64 product with scipy's Sylvester-ordered
Hadamard matrix (a library routine); this fixes the matrix, its ordering, the butterfly
signs and the 1/16 normalisation.  Orthogonality, involution and Parseval follow.

Quantizer (ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet: rows quantized to
S8 with an FP32 scale, one rounded FP32 reciprocal per row): error bound, full range use,
zero rows, power-of-two invariance, round-half-even on hand-chosen rows whose scale is
exactly 1, and the reciprocal (not division) reading on rows where the two differ.
"""
import numpy as np
import scipy.linalg


H256 = scipy.linalg.hadamard(256).astype(np.int64)


def test_fwht_integer_brute_force(orc):
    rng = np.random.default_rng(0)
    for trial in range(50):
        x = rng.integers(-(2 ** 15), 2 ** 15 + 1, 256).astype(np.int64)
        y = orc.fwht256(x.astype(np.float32)).astype(np.float64) * 16
        assert np.array_equal(y.astype(np.int64), H256 @ x)
        assert np.array_equal(y, np.round(y))


def test_rotation_matrix_is_sylvester_over_16_and_orthogonal(orc):
    R = np.stack([orc.fwht256(np.eye(256, dtype=np.float32)[i]) for i in range(256)]).astype(np.float64)
    assert np.array_equal(R, H256 / 16.0)          # rows are e_i R; R symmetric
    assert np.array_equal(R, R.T)
    assert np.abs(R @ R.T - np.eye(256)).max() < 1e-15


def test_rotation_involution_and_parseval(orc):
    rng = np.random.default_rng(1)
    xi = rng.integers(-1000, 1000, 256).astype(np.float32)
    assert np.array_equal(orc.fwht256(orc.fwht256(xi)), xi)   # R R = I exactly on integers
    x = rng.standard_normal(256).astype(np.float32)
    y = orc.fwht256(x)
    assert abs(np.linalg.norm(y.astype(np.float64)) / np.linalg.norm(x.astype(np.float64)) - 1) < 1e-6


def test_convrot_is_block_diagonal(orc):
    rng = np.random.default_rng(2)
    x = rng.integers(-500, 500, (5, 768)).astype(np.float32)
    y = orc.convrot256(x).astype(np.float64) * 16
    ref = x.astype(np.int64) @ np.kron(np.eye(3, dtype=np.int64), H256)
    assert np.array_equal(y.astype(np.int64), ref)


def test_rotation_preserves_products(orc):
    """(x R)(w R)^T = x w^T: the inverse rotation folds into the weights."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((8, 1024)).astype(np.float32)
    w = rng.standard_normal((16, 1024)).astype(np.float32)
    xr = orc.convrot256(x).astype(np.float64)
    wr = orc.convrot256(w).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.abs(xr @ wr.T - ref).max() / np.abs(ref).max() < 1e-5


def test_quant_error_bound_and_range(orc):
    rng = np.random.default_rng(4)
    y = (rng.standard_normal((64, 512)) * rng.uniform(1e-3, 1e3, (64, 1))).astype(np.float32)
    y[5] = 0.0
    q, s = orc.row_quant(y)
    assert q.dtype == np.int8 and q.min() >= -127
    assert s[5] == 0 and (q[5] == 0).all()
    nz = np.arange(64) != 5
    assert (np.abs(q[nz]).max(axis=1) == 127).all()
    err = np.abs(y[nz].astype(np.float64) - q[nz].astype(np.float64) * s[nz, None].astype(np.float64))
    assert (err <= s[nz, None].astype(np.float64) * 0.5 * (1 + 2 ** -20)).all()
    amax = np.abs(y[nz]).max(axis=1)
    assert np.array_equal(s[nz], (amax / np.float32(127)).astype(np.float32))


def test_quant_power_of_two_invariance(orc):
    rng = np.random.default_rng(5)
    y = rng.standard_normal((16, 256)).astype(np.float32)
    q0, s0 = orc.row_quant(y)
    for j in (-20, -3, 5, 30):
        q1, s1 = orc.row_quant(y * np.float32(2.0 ** j))
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1, s0 * np.float32(2.0 ** j))


def test_quant_round_half_even_closed_form(orc):
    # max |y| = 127 -> s = 1 and r = 1 exactly, so q = rint(y) with ties to even
    y = np.zeros((1, 256), np.float32)
    vals = [127.0, 0.5, 1.5, 2.5, -2.5, -0.5, 3.49, -126.5, 125.5]
    y[0, :len(vals)] = vals
    q, s = orc.row_quant(y)
    assert s[0] == 1.0
    assert q[0, :len(vals)].tolist() == [127, 0, 2, 2, -2, 0, 3, -126, 126]


def test_quant_uses_row_reciprocal_not_division(orc):
    """Find rows where rint(y * RN(127/a)) and rint(y / RN(a/127)) differ; the oracle
    must give the reciprocal form (the reading of the FP32 scale reciprocal)."""
    rng = np.random.default_rng(6)
    y = rng.standard_normal((20000, 256)).astype(np.float32)
    a = np.abs(y).max(axis=1, keepdims=True)
    via_r = np.rint(y * (np.float32(127) / a))
    via_s = np.rint(y / (a / np.float32(127)))
    rows = np.where((via_r != via_s).any(axis=1))[0]
    assert rows.size > 0
    q, _ = orc.row_quant(y[rows])
    assert np.array_equal(q.astype(np.float32), np.clip(via_r[rows], -127, 127))
    assert not np.array_equal(q.astype(np.float32), np.clip(via_s[rows], -127, 127))


def test_quant_rows_whose_reciprocal_overflows(orc):
    """Rows with max |y| below 127/FLT_MAX (~3.7e-37), where 127/a is not a finite FP32
    value.  Pinned without the oracle's formula: (1) the codes equal those of the same row
    at normal magnitude (the rows are exact power-of-two copies: multiples of 2^-11 stay
    exact down to 2^-147), (2) the fp64 error bound |127*y/a - q| <= 1/2 holds (a sign-only
    quantization, what an infinite r gives, fails it), (3) zero elements give code 0."""
    rng = np.random.default_rng(7)
    y = (rng.integers(-2047, 2048, (24, 512)) * 2.0 ** -11).astype(np.float32)
    y[:, ::7] = 0.0
    y[3, :] = 0.0
    y[3, 100] = 1.5                                  # one nonzero element
    for shift in (-124, -130, -136):           # normal, partly and mostly subnormal rows
        yt = (y.astype(np.float64) * 2.0 ** shift).astype(np.float32)
        assert np.array_equal(yt.astype(np.float64) * 2.0 ** -shift, y.astype(np.float64))   # exact copies
        a = np.abs(yt).max(axis=1)
        with np.errstate(over="ignore", divide="ignore"):
            assert np.isinf(np.float32(127) / a).all()          # the reciprocal overflows
        q, s = orc.row_quant(yt)
        q0, _ = orc.row_quant(y)
        assert np.array_equal(q, q0)
        t = 127.0 * yt.astype(np.float64) / a[:, None].astype(np.float64)
        assert (np.abs(t - q) <= 0.5 * (1 + 2 ** -20)).all()
        assert (q[yt == 0] == 0).all()
        assert (np.abs(q).max(axis=1) == 127).all()
        assert np.array_equal(s, (a / np.float32(127)).astype(np.float32))
