"""Pins of the oracle's E4M3 / E8M0 (MXFP8) codec: values fixed by the OCP
8-bit float and Microscaling formats, brute-force nearest-code search, and
constructed blocks whose scale and codes follow from the scale rule."""
import math

import numpy as np
import pytest

import oracle

FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_e4m3_decode_format_facts():
    # OCP E4M3: largest finite 448 (S.1111.110), S.1111.111 NaN, smallest subnormal
    # 2^-9, smallest normal 2^-6, 1.0 = exponent field 7.
    assert oracle.e4m3_decode(0x7E) == 448.0
    assert math.isnan(oracle.e4m3_decode(0x7F)) and math.isnan(oracle.e4m3_decode(0xFF))
    assert oracle.e4m3_decode(0x01) == 2.0 ** -9
    assert oracle.e4m3_decode(0x08) == 2.0 ** -6
    assert oracle.e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert oracle.e4m3_decode(0x38) == 1.0
    assert oracle.e4m3_decode(0x00) == 0.0 and math.copysign(1, oracle.e4m3_decode(0x80)) < 0
    pos = [oracle.e4m3_decode(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))          # strictly increasing
    assert all(oracle.e4m3_decode(c | 0x80) == -oracle.e4m3_decode(c) for c in range(0x7F))
    # 126 positive finite values, three mantissa bits => ratio of neighbours <= 1 + 1/8
    assert all(b / a <= 1.125 + 1e-15 for a, b in zip(pos[8:], pos[9:]))


def _brute_encode(v):
    """Nearest finite code by exhaustive search; ties -> even code; saturate."""
    best = None
    for c in FINITE:
        dv = oracle.e4m3_decode(c)
        if math.copysign(1, dv) != math.copysign(1, v):
            continue
        err = abs(dv - v)
        if best is None or err < best[0] or (err == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (err, c)
    return best[1]


def test_e4m3_encode_matches_brute_force():
    rng = np.random.default_rng(0)
    vals = list(rng.normal(size=400) * 30) + list(rng.normal(size=200) * 0.01)
    pos = [oracle.e4m3_decode(c) for c in range(0x7F)]
    mids = [(a + b) / 2 for a, b in zip(pos, pos[1:])]            # exact ties
    vals += mids + [-m for m in mids] + [1e-9, -1e-9, 447.9, 449.0, 464.0, 1e6, -1e6]
    for v in vals:
        assert oracle.e4m3_encode(v) == _brute_encode(v), v


def test_e4m3_round_trip_all_codes():
    for c in FINITE:
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c


@pytest.mark.parametrize("n", [-20, -3, 0, 5, 40])
def test_mx_scale_rule_constructed_blocks(n):
    rng = np.random.default_rng(n + 100)
    base = rng.uniform(-1, 1, size=32) * 2.0 ** n
    # amax = 2^n exactly -> shared = n - 8, element amax -> 256 (code 0x78)
    b1 = base.copy(); b1[5] = 2.0 ** n
    # amax = 448 * 2^n -> shared = n, element 448 (0x7E)
    b2 = base.copy(); b2[7] = -448.0 * 2.0 ** n
    # amax just below 2^(n+9) -> shared = n, element saturates to 448
    b3 = base.copy(); b3[0] = 511.0 * 2.0 ** n
    codes, scales = oracle.mx_quantize(np.stack([b1, b2, b3]))
    assert scales[0, 0] == n - 8 + 127 and codes[0, 5] == 0x78
    assert scales[1, 0] == n + 127 and codes[1, 7] == 0xFE
    assert scales[2, 0] == n + 127 and codes[2, 0] == 0x7E


def test_mx_zero_block_and_relative_error():
    codes, scales = oracle.mx_quantize(np.zeros((1, 64)))
    assert np.all(codes == 0) and np.all(scales == 0)
    rng = np.random.default_rng(7)
    v = rng.normal(size=(50, 128))
    codes, scales = oracle.mx_quantize(v)
    deq = oracle.mx_dequantize(codes, scales)
    blocks = np.abs(v).reshape(50, 4, 32).max(axis=2)
    shared = np.floor(np.log2(blocks)) - 8
    sc = np.repeat(2.0 ** shared, 32, axis=1)
    a = np.abs(v) / sc
    normal = (a >= 2.0 ** -6) & (a <= 448)
    # normal elements: |err| <= half a unit in the 4th significant bit (2^-4 relative)
    assert np.all(np.abs(deq - v)[normal] <= np.abs(v)[normal] * 2.0 ** -4 + 1e-300)
    # subnormal elements: |err| <= half the subnormal quantum
    assert np.all(np.abs(deq - v)[~normal & (a < 1)] <= 2.0 ** -10 * sc[~normal & (a < 1)])
    np.testing.assert_array_equal(scales, (shared + 127).astype(np.uint8))
