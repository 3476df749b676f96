"""Pins of the oracle's Q8_0 activation quantization.

Definition: minfer README (nano-inference page), milestone M3.5 (int8
activations) with the 34-byte Q8_0 block implied by milestone M14's 248 MB
lm_head: d = max|x|/127 (fp32), q = round-half-away(x/d), stored binary16(d).
"""
import numpy as np
import pytest

from conftest import load_golden, parse_number

CASES = load_golden("q8_0_blocks.txt")


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_q8_0_golden_blocks(oracle, case):
    x = np.array([parse_number(t) for t in case["x"]], np.float32)
    assert x.size == 32
    if case["name"] == "unit_scale_ties":
        assert x[7].view(np.uint32) == 0x3effffff  # 0.5 - 2^-25
    blk = oracle.quantize_q8_0(x[None, :])[0, 0]
    d = int(blk[0]) | (int(blk[1]) << 8)
    q = blk[2:].view(np.int8)
    assert d == int(case["d"][0], 16)
    assert list(q) == [int(t) for t in case["q"]]


def _blocks(seed, n):
    rng = np.random.default_rng(seed)
    scale = np.float32(10.0) ** rng.uniform(-6, 5, size=(n, 1)).astype(np.float32)
    x = (rng.standard_normal((n, 32)).astype(np.float32) * scale).astype(np.float32)
    # sprinkle exact zeros, duplicate maxima and sign flips
    x[rng.random((n, 32)) < 0.05] = 0
    x[::7, 3] = -x[::7].__abs__().max(axis=1)
    x[::11, 5] = x[::11].__abs__().max(axis=1)
    return x


def test_q8_0_properties_random(oracle):
    x = _blocks(3, 20000)
    out = oracle.quantize_q8_0(x.reshape(1, -1)).reshape(-1, 34)
    d16 = out[:, 0:2].copy().view(np.uint16)[:, 0]
    q = out[:, 2:].view(np.int8).astype(np.int32)
    amax = np.abs(x).max(axis=1)
    d32 = (amax / np.float32(127)).astype(np.float32)           # NumPy IEEE fp32 division
    assert np.array_equal(d16, d32.astype(np.float16).view(np.uint16))
    assert np.abs(q).max() <= 127
    nz = amax > 0
    # the block maximum maps to +-127 with its sign
    arg = np.abs(x).argmax(axis=1)
    rows = np.arange(x.shape[0])
    assert np.all(q[rows[nz], arg[nz]] == np.where(x[rows[nz], arg[nz]] > 0, 127, -127))
    # |x/d - q| <= 1/2, with x/d the fp32 quotient, ties resolved away from zero
    v = (x[nz] / d32[nz, None]).astype(np.float32).astype(np.float64)
    err = v - q[nz]
    assert np.abs(err).max() <= 0.5
    ties = np.abs(err) == 0.5
    assert np.all(np.sign(err[ties]) == -np.sign(v[ties]))
    assert np.all(q[~nz] == 0) and np.all(d16[~nz] == 0)


def test_q8_0_rows_are_independent_blocks(oracle):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    whole = oracle.quantize_q8_0(x)
    assert whole.shape == (3, 8, 34)
    for r in range(3):
        for b in range(8):
            one = oracle.quantize_q8_0(x[r:r + 1, 32 * b:32 * b + 32])
            assert np.array_equal(one[0, 0], whole[r, b])


def test_q8_0_near_ties(oracle):
    # values within a few ulps of (k + 1/2) * d for scales d that are not powers
    # of two: q must be the half-away rounding of the fp32 quotient x / d (NumPy's
    # IEEE division), which a reciprocal multiply or a different divisor misses
    rng = np.random.default_rng(13)
    nblk = 20000
    amax = (np.float32(2.0) ** rng.uniform(-20, 20, nblk).astype(np.float32)).astype(np.float32)
    d = (amax / np.float32(127)).astype(np.float32)
    k = rng.integers(-126, 126, size=(nblk, 31)).astype(np.float32)
    base = ((k + np.float32(0.5)) * d[:, None]).astype(np.float32)
    nudge = rng.integers(-3, 4, size=(nblk, 31))
    x = base.copy()
    for step in range(3):
        up, dn = nudge > step, nudge < -step
        x = np.where(up, np.nextafter(x, np.float32(np.inf)), x)
        x = np.where(dn, np.nextafter(x, np.float32(-np.inf)), x)
    x = np.clip(x, -amax[:, None], amax[:, None]).astype(np.float32)
    blocks = np.concatenate([amax[:, None], x], axis=1).astype(np.float32)
    out = oracle.quantize_q8_0(blocks.reshape(1, -1)).reshape(-1, 34)
    q = out[:, 2:].view(np.int8).astype(np.float64)
    v = (blocks / d[:, None]).astype(np.float32).astype(np.float64)
    expect = np.sign(v) * np.floor(np.abs(v) + 0.5)      # exact in fp64
    assert np.array_equal(q, expect)
