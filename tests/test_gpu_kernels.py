"""GPU parity of the single-matrix entry points against the CPU oracle.

Q8_0 quantization, the repack and the per-block integer sums must match the
oracle bit for bit; GEMV outputs within 1e-5 * sum_b |d_w d_x s| (the
tolerance of the fp32 accumulation; the exact value is the oracle's fp64 sum).
Every call goes through the C ABI of libq4stream.
"""
import numpy as np
import pytest
import torch

from conftest import load_golden, parse_number
from gpu_helpers import (assert_within, dev, packed_weights, padding_is_zero, q8_canonical,
                         require_gpu, to_dev, unpack_packed)
from q4_weight_streaming_amd import _lib as q
from q4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


# shapes: (rows, cols) -- config matrices, K splits 1/2/4, ragged rows and chunks
SHAPES = [(1536, 1536), (256, 1536), (8960, 1536), (1536, 8960), (512, 3584), (3584, 18944),
          (1, 32), (63, 288), (65, 64), (257, 1536), (100, 2304), (130, 4128), (70, 96)]


def _inputs(rows, cols, n, tag=0):
    rng = synth.generator(900 + tag, rows, cols, n)
    return synth.q4_0_weights(rows, cols, rng), synth.activation(n, cols, rng)


# ------------------------------------------------------------------ quantize

def test_quantize_golden_blocks(oracle):
    cases = load_golden("q8_0_blocks.txt")
    x = np.array([[parse_number(t) for c in cases for t in c["x"]]], np.float32)
    got = q8_canonical(q.quantize_q8_0(to_dev(x)), 1, x.shape[1])
    ref = oracle.quantize_q8_0(x)
    assert np.array_equal(got, ref)
    for i, c in enumerate(cases):                              # and the hand values
        assert int(got[0, i, 0]) | int(got[0, i, 1]) << 8 == int(c["d"][0], 16)
        assert list(got[0, i, 2:].view(np.int8)) == [int(t) for t in c["q"]]


# up to 8 rows the quantizer stores with the non-temporal hint, past 8 without: both are covered
@pytest.mark.parametrize("n,cols", [(1, 1536), (3, 8960), (8, 3584), (8, 18944), (2, 32), (5, 96),
                                    (9, 1536), (24, 288), (17, 8960)])
def test_quantize_bit_exact(oracle, n, cols):
    x = synth.activation(n, cols, synth.generator(7, n, cols, 1))
    got = q8_canonical(q.quantize_q8_0(to_dev(x)), n, cols)
    assert np.array_equal(got, oracle.quantize_q8_0(x))


def test_quantize_near_ties_and_scales(oracle):
    rng = np.random.default_rng(21)
    nblk = 4096
    amax = (np.float32(2.0) ** rng.uniform(-26, 22, nblk).astype(np.float32)).astype(np.float32)
    d = (amax / np.float32(127)).astype(np.float32)
    k = rng.integers(-126, 126, size=(nblk, 31)).astype(np.float32)
    x = ((k + np.float32(0.5)) * d[:, None]).astype(np.float32)
    x = np.where(rng.random(x.shape) < 0.3, np.nextafter(x, np.float32(np.inf)), x)
    x = np.where(rng.random(x.shape) < 0.3, np.nextafter(x, np.float32(-np.inf)), x)
    x = np.clip(x, -amax[:, None], amax[:, None])
    blocks = np.concatenate([amax[:, None] * np.sign(rng.random((nblk, 1)) - 0.5).astype(np.float32), x], 1)
    blocks[::17] = 0                                           # all-zero blocks
    xs = blocks.astype(np.float32).reshape(4, -1)
    got = q8_canonical(q.quantize_q8_0(to_dev(xs)), 4, xs.shape[1])
    assert np.array_equal(got, oracle.quantize_q8_0(xs))


def test_quantize_extreme_scales(oracle):
    """Block maxima at and around the ends of the kernel's division-free range
    (a in [2^-96, 2^96] for the scale, d in [2^-125, 2^125] for the reciprocal),
    subnormal maxima and values (down to d = 2^-149), and the largest allowed
    magnitude; each block
    holds its maximum, near-ties (k + 1/2) d nudged by an ulp, and random values."""
    rng = np.random.default_rng(23)
    f32 = np.float32
    edges = [2.0 ** -97, 2.0 ** -96, 2.0 ** -95, 127 * 2.0 ** -126, 127 * 2.0 ** -125, 127 * 2.0 ** -124,
             1e-36, 1e-38, 1e-40, 2.0 ** -142, 2.0 ** -140, 2.0 ** 22, 7.9e6]
    amax = []
    for e in edges:
        e = f32(e)
        amax += [np.nextafter(e, f32(0)), e, np.nextafter(e, f32(np.inf))]
    amax = np.array([a for a in amax if a > 0], np.float32)
    reps = 8
    amax = np.repeat(amax, reps)
    nblk = amax.size
    d = (amax / f32(127)).astype(np.float32)
    k = rng.integers(-126, 126, size=(nblk, 15)).astype(np.float32)
    ties = ((k + f32(0.5)) * d[:, None]).astype(np.float32)
    ties = np.where(rng.random(ties.shape) < 0.4, np.nextafter(ties, f32(np.inf)), ties)
    ties = np.where(rng.random(ties.shape) < 0.4, np.nextafter(ties, f32(-np.inf)), ties)
    rand = ((rng.random((nblk, 16)) * 2 - 1) * amax[:, None]).astype(np.float32)
    x = np.clip(np.concatenate([ties, rand], 1), -amax[:, None], amax[:, None])
    sign = np.where(rng.random((nblk, 1)) < 0.5, f32(-1), f32(1))
    blocks = np.concatenate([amax[:, None] * sign, x], 1).astype(np.float32)
    perm = rng.permuted(np.tile(np.arange(32), (nblk, 1)), axis=1)  # maximum anywhere in the block
    blocks = np.take_along_axis(blocks, perm, 1)
    xs = blocks.reshape(reps, -1)
    got = q8_canonical(q.quantize_q8_0(to_dev(xs)), reps, xs.shape[1])
    assert np.array_equal(got, oracle.quantize_q8_0(xs))


def test_quantize_empty_is_noop():
    x = torch.empty((0, 64), dtype=torch.float32, device=dev())
    assert q.quantize_q8_0(x).numel() == 0


# ------------------------------------------------------------------ repack

@pytest.mark.parametrize("rows,cols", [(1, 32), (63, 288), (65, 64), (257, 1536), (1536, 1536), (70, 96)])
def test_repack_round_trip(rows, cols):
    w, _ = _inputs(rows, cols, 1)
    packed = packed_weights(w, rows, cols).cpu().numpy()
    assert packed.size == q.packed_bytes(rows, cols)
    assert np.array_equal(unpack_packed(packed, rows, cols), w)
    assert padding_is_zero(packed, rows, cols)


# ------------------------------------------------------------------ block sums

@pytest.mark.parametrize("rows,cols,n", [(1, 32, 1), (63, 288, 3), (257, 1536, 8), (130, 4128, 2),
                                         (65, 64, 5)])
def test_block_sums_bit_exact(oracle, rows, cols, n):
    w, x = _inputs(rows, cols, n)
    xq = q.quantize_q8_0(to_dev(x))
    got = q.block_sums(packed_weights(w, rows, cols), xq, rows, cols, n).cpu().numpy()
    ref = oracle.block_sums(w, oracle.quantize_q8_0(x), rows, cols, n)
    assert np.array_equal(got, ref)


def test_block_sums_wide_bit_exact(oracle):
    rows, cols, n = 130, 4128, 24
    w, x = _inputs(rows, cols, n, tag=3)
    xq = q.quantize_q8_0(to_dev(x))
    got = q.block_sums(packed_weights(w, rows, cols), xq, rows, cols, n).cpu().numpy()
    assert np.array_equal(got, oracle.block_sums(w, oracle.quantize_q8_0(x), rows, cols, n))


def test_block_sums_extremes(oracle):
    # all nibbles 0 against q = -127 gives +32512 per block, the largest |s|
    rows, cols = 64, 256
    w, _ = _inputs(rows, cols, 1)
    w[..., 2:] = 0x00
    x = np.full((1, cols), -1.0, np.float32)
    got = q.block_sums(packed_weights(w, rows, cols), q.quantize_q8_0(to_dev(x)), rows, cols, 1).cpu().numpy()
    assert (got == 32512).all()


# ------------------------------------------------------------------ GEMV

@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("n", [1, 2, 8])
def test_gemv_parity(oracle, rows, cols, n):
    w, x = _inputs(rows, cols, n)
    wp = packed_weights(w, rows, cols)
    xq = q.quantize_q8_0(to_dev(x))
    y = q.gemv_q4_0(wp, xq, rows, cols, n).cpu().numpy()
    y_ref, S = oracle.gemv(w, oracle.quantize_q8_0(x), rows, cols, n)
    assert_within(y, y_ref, S, what=f"{rows}x{cols} n={n}")


@pytest.mark.parametrize("rows,cols", [(257, 1536), (100, 2304), (130, 4128), (1536, 8960)])
def test_gemv_n_invariance_and_determinism(rows, cols):
    # row t of an n-row call equals the 1-row call on that activation, bit for bit
    w, x = _inputs(rows, cols, 8, tag=1)
    wp = packed_weights(w, rows, cols)
    xq8 = q.quantize_q8_0(to_dev(x))
    y8 = q.gemv_q4_0(wp, xq8, rows, cols, 8)
    y8b = q.gemv_q4_0(wp, xq8, rows, cols, 8)
    assert torch.equal(y8, y8b)
    for n in (1, 3, 5, 8):
        yn = q.gemv_q4_0(wp, q.quantize_q8_0(to_dev(x[:n])), rows, cols, n)
        assert torch.equal(yn, y8[:n])
    for t in range(8):
        y1 = q.gemv_q4_0(wp, q.quantize_q8_0(to_dev(x[t:t + 1])), rows, cols, 1)
        assert torch.equal(y1[0], y8[t])


WIDE_SHAPES = [(1536, 1536), (256, 1536), (1536, 8960), (63, 288), (65, 64), (257, 1536), (130, 4128),
               (70, 96)]


@pytest.mark.parametrize("rows,cols", WIDE_SHAPES)
@pytest.mark.parametrize("n", [9, 16, 17, 24])
def test_gemv_wide_parity(oracle, rows, cols, n):
    # 9..24 activation rows in one weight pass (token tiles of 8)
    w, x = _inputs(rows, cols, n, tag=4)
    wp = packed_weights(w, rows, cols)
    y = q.gemv_q4_0(wp, q.quantize_q8_0(to_dev(x)), rows, cols, n).cpu().numpy()
    y_ref, S = oracle.gemv(w, oracle.quantize_q8_0(x), rows, cols, n)
    assert_within(y, y_ref, S, what=f"{rows}x{cols} n={n}")


@pytest.mark.parametrize("rows,cols", [(257, 1536), (130, 4128), (1536, 8960), (70, 96)])
def test_gemv_wide_rows_equal_one_row(rows, cols):
    # every row of a 9..24-row call equals the 1-row call on that activation, bit for bit
    w, x = _inputs(rows, cols, 24, tag=5)
    wp = packed_weights(w, rows, cols)
    y24 = q.gemv_q4_0(wp, q.quantize_q8_0(to_dev(x)), rows, cols, 24)
    assert torch.equal(y24, q.gemv_q4_0(wp, q.quantize_q8_0(to_dev(x)), rows, cols, 24))
    for n in (9, 12, 16, 17, 23):
        yn = q.gemv_q4_0(wp, q.quantize_q8_0(to_dev(x[:n])), rows, cols, n)
        assert torch.equal(yn, y24[:n])
    for t in range(24):
        y1 = q.gemv_q4_0(wp, q.quantize_q8_0(to_dev(x[t:t + 1])), rows, cols, 1)
        assert torch.equal(y1[0], y24[t]), t


def test_gemv_closed_forms():
    rows, cols = 200, 2560
    w, x = _inputs(rows, cols, 2)
    xq = q.quantize_q8_0(to_dev(x))
    zero = w.copy()
    zero[..., 2:] = 0x88                                        # every nibble 8: weight 0
    assert (q.gemv_q4_0(packed_weights(zero, rows, cols), xq, rows, cols, 2) == 0).all()
    # doubling every d_w (exact in binary16 away from overflow) doubles y exactly
    dw = w[..., 0:2].copy().view("<f2")
    w2 = w.copy()
    w2[..., 0:2] = (dw.astype(np.float32) * 2).astype("<f2").view(np.uint8)
    y1 = q.gemv_q4_0(packed_weights(w, rows, cols), xq, rows, cols, 2)
    y2 = q.gemv_q4_0(packed_weights(w2, rows, cols), xq, rows, cols, 2)
    assert torch.equal(y2, 2 * y1)


def test_gemv_empty_and_zero_width():
    wp = torch.empty(0, dtype=torch.uint8, device=dev())
    xq = torch.empty(0, dtype=torch.uint8, device=dev())
    y = torch.full((3, 40), 7.0, device=dev())
    q.gemv_q4_0(wp, xq, 40, 0, 3, out=y)                       # K = 0: the empty sum
    assert (y == 0).all()
    y = torch.full((20, 40), 7.0, device=dev())
    q.gemv_q4_0(wp, xq, 40, 0, 20, out=y)                      # and on the wide path
    assert (y == 0).all()
    q.gemv_q4_0(wp, xq, 0, 64, 1, out=torch.empty((1, 0), device=dev()))   # no rows: no-op


def test_measurement_reads_stay_in_their_buffers():
    # the read benchmarks (no outputs besides the sink): whole units only, a tail shorter than a
    # unit untouched; each returns cleanly and leaves the sink as it was
    sink = torch.zeros(4, dtype=torch.int32, device=dev())
    buf = torch.ones(3 * 9216 + 5000, dtype=torch.uint8, device=dev())
    q.bench_read_units(buf, 9216, sink)
    q.bench_read_units(buf, 55296, sink)                       # no whole unit: nothing to read
    q.bench_read(buf[: (buf.numel() // 16) * 16], 4, 8, sink)
    torch.cuda.synchronize()
    assert (sink == 0).all()
