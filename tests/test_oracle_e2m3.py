"""Pins of the oracle's second storage form of 4-bit code rows: each code -7..7 stored as
the E2M3 (6-bit float) number of the same value, in 96-byte units of 128 codes (quarters
of 32 codes as 192-bit fields, code e in bits 6e..6e+5; the fields' first 16 bytes in the
order Q0, Q2, Q1, Q3, then their last 8 bytes in the same order), rows stored in quads
(unit u of row 4q + i at q * ld + u * 384 + i * 96).  The pages describe no
W4A4 format (ComfyUI Turing Utils README names W4A4 dispatch only); this form exists so that
6-bit floating-point matrix cores multiply the codes exactly."""
import numpy as np
import pytest

import oracle
from test_oracle_formats import minifloat


@pytest.fixture(scope="module")
def orc():
    oracle.build.build()
    return oracle


def test_e2m3_decoder_matches_the_generic_minifloat(orc):
    """All 64 codes against the minifloat decoder validated on torch's FP8 formats (2
    exponent bits, bias 1, 3 mantissa bits, no inf/NaN)."""
    for c in range(64):
        assert orc.e2m3(c) == minifloat(c, 2, 3, 1), c
    assert orc.e2m3(0b011110) == 7.0 and orc.e2m3(0b011111) == 7.5 and orc.e2m3(0b000001) == 0.125


def test_hand_worked_unit(orc):
    """Codes 1 at k = 0 and 1, 3 at 32, -7 at 64, 5 at 85, -1 at 127 of a 128-code row.
    E2M3: 1 = 0b001000, 3 = 1.5 * 2 = 0b010100, 5 = 1.25 * 4 = 0b011010, 7 = 1.75 * 4 =
    0b011110, sign bit 0b100000.  Heads (bits 0..127) of Q0 Q2 Q1 Q3 at bytes 0, 16, 32, 48,
    tails (bits 128..191) at 64, 72, 80, 88.  k = 0 -> byte 0 = 0x08; k = 1 -> bits 6..11:
    byte 0 bits 6, 7 = 0, byte 1 = 0x08 >> 2 = 0x02; k = 32 (Q1 head) -> byte 32 = 0x14;
    k = 64 (Q2 head) -> byte 16 = 0x3E; k = 85 (Q2, e = 21, bits 126..131: the last two bits
    of the head, the first four of the tail) -> 0b011010: bits 0, 1 = 0b10 into byte 16 + 15
    bits 6, 7 (0x80), bits 2..5 = 0b0110 into byte 72 bits 0..3 (0x06); k = 127 (Q3, e = 31,
    bits 186..191, the tail's byte 7 bits 2..7) -> byte 88 + 7 = 95 = 0x28 << 2 = 0xA0.
    A single row is row 0 of its quad: the quad's 384 bytes hold it at 0..95, zeros after."""
    q = np.zeros((1, 128), np.int8)
    q[0, [0, 1, 32, 64, 85, 127]] = [1, 1, 3, -7, 5, -1]
    p = orc.pack_e2m3(q)
    assert p.shape == (1, 384)
    want = np.zeros(384, np.uint8)
    want[[0, 1, 32, 16, 31, 72, 95]] = [0x08, 0x02, 0x14, 0x3E, 0x80, 0x06, 0xA0]
    assert np.array_equal(p[0], want), np.nonzero(p[0])


def test_quad_placement(orc):
    """Row 4q + i, unit u starts at quad q's row of the array, byte u * 384 + i * 96: a code
    1 at column 128 (unit 1, Q0, code 0) of row 6 (quad 1, i = 2) lands in byte 0x08 at
    array row 1, byte 384 + 192; the same code at column 0 of row 3 at array row 0, byte 288."""
    q = np.zeros((7, 256), np.int8)
    q[6, 128] = 1
    q[3, 0] = 1
    p = orc.pack_e2m3(q)
    assert p.shape == (2, 768)
    assert p[1, 384 + 192] == 0x08 and p[0, 288] == 0x08
    assert np.count_nonzero(p) == 2


def test_round_trip_and_agreement_with_the_nibble_form(orc):
    rng = np.random.default_rng(3)
    q = rng.integers(-7, 8, (9, 768), dtype=np.int8)
    p = orc.pack_e2m3(q)
    assert p.shape == (3, 2304)
    assert np.array_equal(orc.unpack_e2m3(p, 768, 9), q)
    assert np.array_equal(orc.unpack_s4(orc.pack_s4(q), 768), q)
    # every value occurs, in every quarter position of a unit
    for v in range(-7, 8):
        qq = np.full((1, 128), v, np.int8)
        assert np.array_equal(orc.unpack_e2m3(orc.pack_e2m3(qq), 128, 1), qq)


def test_gemm_e2m3_int64_brute_force(orc):
    rng = np.random.default_rng(4)
    for (M, N, K_pad) in [(1, 1, 256), (7, 13, 512)]:
        qa = rng.integers(-7, 8, (M, K_pad), dtype=np.int8)
        qb = rng.integers(-7, 8, (N, K_pad), dtype=np.int8)
        ref = qa.astype(np.int64) @ qb.astype(np.int64).T
        got = orc.gemm_e2m3(orc.pack_e2m3(qa), orc.pack_e2m3(qb), K_pad, M, N)
        assert np.array_equal(got.astype(np.int64), ref)
