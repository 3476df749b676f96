"""Pins of the oracle's binary16 conversions against NumPy's IEEE-754 implementation.

The Q4_0 and Q8_0 scales are binary16 (GGUF block formats used by the minfer
README's loader, nano-inference page); the oracle converts them with its own
code, checked here exhaustively (decode) and on >= 10^7 samples plus every tie
(encode, round to nearest even, subnormals kept, overflow to infinity).
"""
import numpy as np


def test_fp16_decode_exhaustive(oracle):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.fp16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _np_encode(f):
    with np.errstate(over="ignore"):
        return np.asarray(f, np.float32).astype(np.float16).view(np.uint16)


def test_fp16_encode_random_bits(oracle):
    rng = np.random.default_rng(7)
    # exponents from far below the subnormal range to beyond overflow
    e = rng.integers(127 - 30, 127 + 18, size=10_000_000, dtype=np.uint32)
    m = rng.integers(0, 1 << 23, size=e.size, dtype=np.uint32)
    s = rng.integers(0, 2, size=e.size, dtype=np.uint32)
    f = ((s << 31) | (e << 23) | m).view(np.float32)
    assert np.array_equal(oracle.f32_to_fp16(f), _np_encode(f))


def test_fp16_encode_every_tie_and_neighbour(oracle):
    # midpoints between consecutive finite binary16 values (exact in fp32), and
    # the fp32 values one ulp either side of each midpoint
    h = np.arange(0, 0x7bff, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)  # exactly representable
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    top = np.array([65504.0, 65519.996, 65520.0, 65536.0, 1e30, np.inf, -np.inf], np.float32)
    f = np.concatenate([mid, up, dn, -mid, -up, -dn, top])
    assert np.array_equal(oracle.f32_to_fp16(f), _np_encode(f))


def test_fp16_encode_specials(oracle):
    f = np.array([0.0, -0.0, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14,
                  65504.0, 65520.0], np.float32)
    got = oracle.f32_to_fp16(f)
    assert list(got) == [0x0000, 0x8000, 0x0001, 0x0000, 0x0001, 0x0400, 0x7bff, 0x7c00]
    assert (oracle.f32_to_fp16(np.array([np.nan], np.float32))[0] & 0x7c00) == 0x7c00
