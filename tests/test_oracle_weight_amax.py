"""Pins of the oracle's rotated weight row maxima (the a of the row quantizer, computed
without the codes; ComfyUI Turing Utils README, "Load ConvRot DiT ..." bullet: the row
scale of a weight covers its whole padded row).

Pinned by an exact brute force that shares nothing with the oracle's transform (decoded
values from the closed-form E2M1 and E4M3 values, the rotation from scipy's Hadamard matrix
in float64 — every value here is a small dyadic number, so float32 and float64 agree
exactly), by the quantizer's own identities (s = a/127 and max |q| = 127 from the separate
preparation call), and by zero rows and garbage in the serialized padding.
"""
import numpy as np
import scipy.linalg

import oracle

H256 = scipy.linalg.hadamard(256).astype(np.float64)
E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6])
# E4M3 bytes with their values: 0x30 = 2^-1, 0x38 = 1, 0x40 = 2, 0x3c = 1.5, 0x00 = 0
SF_BYTES = np.array([0x30, 0x38, 0x40, 0x3C, 0x00], np.uint8)
SF_VALUES = np.array([0.5, 1.0, 2.0, 1.5, 0.0])


def _packed(rng, N, K):
    nib = rng.integers(0, 16, (N, K))
    codes = np.zeros((N, (K + 1) // 2), np.uint8)
    codes[:, :] = nib[:, 0::2].astype(np.uint8)
    codes[:, :K // 2] |= (nib[:, 1::2].astype(np.uint8) << 4)
    si = rng.integers(0, len(SF_BYTES), (N, (K + 15) // 16))
    return nib, codes, SF_BYTES[si], SF_VALUES[si]


def test_weight_amax_brute_force():
    rng = np.random.default_rng(21)
    for N, K in ((7, 512), (5, 300), (3, 1000), (2, 16)):
        nib, codes, sf, sfv = _packed(rng, N, K)
        g = 0.25
        kp = oracle.padded_k(K)
        w = np.zeros((N, kp))
        w[:, :K] = E2M1[nib] * np.repeat(sfv, 16, axis=1)[:, :K] * g
        y = np.concatenate([w[:, b:b + 256] @ H256 for b in range(0, kp, 256)], axis=1) / 16.0
        ref = np.abs(y).max(axis=1).astype(np.float32)
        a = oracle.weight_amax_nvfp4(codes, sf, g, K)
        assert np.array_equal(a, ref), (N, K)


def test_weight_amax_matches_the_quantizer():
    rng = np.random.default_rng(22)
    N, K = 40, 1300
    nib, codes, sf, _ = _packed(rng, N, K)
    codes[3] = 0                                   # a zero row
    g = np.float32(0.0137)
    a = oracle.weight_amax_nvfp4(codes, sf, float(g), K)
    q, s = oracle.prep_weight_nvfp4(codes, sf, float(g), K)
    assert a[3] == 0.0 and s[3] == 0.0 and not q[3].any()
    nz = a > 0
    assert np.array_equal(s[nz], (a[nz] / np.float32(127)).astype(np.float32))
    assert np.all(np.abs(q[nz]).max(axis=1) == 127)
    # q is the rounding of y * RN(127/a): recompute from the decoded, rotated rows
    y = oracle.convrot256(oracle.nvfp4_decode(codes, sf, float(g), K))
    r = (np.float32(127) / a[nz]).astype(np.float32)
    qq = np.clip(np.rint((y[nz] * r[:, None]).astype(np.float32)), -127, 127)
    assert np.array_equal(q[nz], qq.astype(np.int8))


def test_weight_amax_ignores_serialized_padding():
    rng = np.random.default_rng(23)
    N, K = 6, 301                                  # odd K: the last byte holds one element
    _, codes, sf, _ = _packed(rng, N, K)
    codes[:, -1] &= 0x0F                           # clean padding nibble
    wide = np.concatenate([codes, rng.integers(0, 256, (N, 9), dtype=np.uint8)], axis=1)
    wide[:, codes.shape[1] - 1] |= 0xA0            # garbage in the padding nibble
    sfw = np.concatenate([sf, rng.integers(0, 256, (N, 3), dtype=np.uint8)], axis=1)
    a0 = oracle.weight_amax_nvfp4(codes, sf, 0.5, K)
    a1 = oracle.weight_amax_nvfp4(wide, sfw, 0.5, K)
    assert np.array_equal(a0, a1)
