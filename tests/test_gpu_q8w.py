"""GPU parity of the Q8_0-weight entry points (the 8-bit output head) against
the CPU oracle.

Repack, per-block integer sums and the Q8_0 -> Q4_0 requantization must match
bit for bit; GEMV outputs within 1e-5 * sum_b |d_w d_x s| of the oracle's fp64
sum.  Every call goes through the C ABI of libq4stream.
"""
import numpy as np
import pytest
import torch

from conftest import load_golden
from gpu_helpers import (assert_within, dev, packed_weights, q8_canonical, require_gpu, to_dev,
                         unpack_packed_q8)
from q4_weight_streaming_amd import _lib as q
from q4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


SHAPES = [(1536, 1536), (256, 1536), (8960, 1536), (1536, 8960), (512, 3584), (1, 32), (63, 288),
          (65, 64), (257, 1536), (100, 2304), (130, 4128), (70, 96)]


def _inputs(rows, cols, n, tag=0):
    rng = synth.generator(950 + tag, rows, cols, n)
    return synth.q8_0_weights(rows, cols, rng), synth.activation(n, cols, rng)


def _packed(w8, rows, cols):
    return q.repack_q8_0(to_dev(w8.reshape(-1)), rows, cols)


def _run(w8, x, rows, cols, n, oracle):
    """GPU: quantize + Q8_0-weight GEMV; oracle: its quantizer + its GEMV on the same fp32 x."""
    xq_dev = q.quantize_q8_0(to_dev(x))
    xq_ref = oracle.quantize_q8_0(x)
    assert np.array_equal(q8_canonical(xq_dev, n, cols), xq_ref)
    y = q.gemv_q8_0(_packed(w8, rows, cols), xq_dev, rows, cols, n).cpu().numpy()
    y_ref, S = oracle.q8w_gemv(w8, xq_ref, rows, cols, n)
    return y, y_ref, S, xq_dev


# ------------------------------------------------------------------ repack

@pytest.mark.parametrize("rows,cols", [(1, 32), (63, 288), (65, 64), (257, 1536), (1536, 1536), (70, 96)])
def test_repack_q8_round_trip(rows, cols):
    w8, _ = _inputs(rows, cols, 1)
    got, pad_zero = unpack_packed_q8(_packed(w8, rows, cols).cpu().numpy(), rows, cols)
    assert np.array_equal(got, w8)
    assert pad_zero


# --------------------------------------------------------------- block sums

@pytest.mark.parametrize("rows,cols,n", [(63, 288, 1), (130, 4128, 3), (70, 96, 8), (257, 1536, 2)])
def test_block_sums_q8_bit_exact(oracle, rows, cols, n):
    w8, x = _inputs(rows, cols, n, 1)
    xq = q.quantize_q8_0(to_dev(x))
    s = q.block_sums_q8_0(_packed(w8, rows, cols), xq, rows, cols, n).cpu().numpy()
    xq8 = oracle.quantize_q8_0(x)
    assert np.array_equal(q8_canonical(xq, n, cols), xq8)      # the GPU's bytes are the oracle's
    assert np.array_equal(s, oracle.q8w_block_sums(w8, xq8, rows, cols, n))


# -------------------------------------------------------------------- GEMV

@pytest.mark.parametrize("n", [1, 2, 8])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_gemv_q8_matches_oracle(oracle, rows, cols, n):
    w8, x = _inputs(rows, cols, n)
    y, y_ref, S, _ = _run(w8, x, rows, cols, n, oracle)
    assert_within(y, y_ref, S, what=f"q8w {rows}x{cols} n={n}")


@pytest.mark.parametrize("rows,cols", [(1536, 8960), (257, 1536), (70, 96), (130, 4128)])
def test_gemv_q8_rows_independent_of_n_and_deterministic(rows, cols):
    w8, x = _inputs(rows, cols, 8, 2)
    wp = _packed(w8, rows, cols)
    x_t = to_dev(x)
    singles = [q.gemv_q8_0(wp, q.quantize_q8_0(x_t[t:t + 1].contiguous()), rows, cols, 1).cpu().numpy()[0]
               for t in range(8)]
    for n in range(2, 9):
        xq = q.quantize_q8_0(x_t[:n].contiguous())
        a = q.gemv_q8_0(wp, xq, rows, cols, n).cpu().numpy()
        b = q.gemv_q8_0(wp, xq, rows, cols, n).cpu().numpy()
        assert np.array_equal(a, b)
        for t in range(n):
            assert np.array_equal(a[t], singles[t]), (n, t)


@pytest.mark.parametrize("rows,cols", [(1536, 1536), (257, 1536), (64, 32), (130, 96), (70, 2048), (3, 1824),
                                       (1, 288), (130, 4128), (100, 2304)])
def test_gemv_q8_from_f32_equals_two_launches(oracle, rows, cols):
    """q4s_gemv_q8_0_f32: one launch quantizing inside (cols <= 2048: every chunk count 1..8,
    padding blocks, ragged row groups), or a quantize launch and the GEMV (wider): x_q8 equals
    the oracle's quantizer byte for byte and y the two-launch form bit for bit."""
    w8, x = _inputs(rows, cols, 1, tag=3)
    wp = _packed(w8, rows, cols)
    xq_fill = torch.full((q.q8_bytes(1, cols),), 0xA5, dtype=torch.uint8, device=dev())  # every byte written
    y, xq = q.gemv_q8_0_f32(wp, to_dev(x), rows, cols, x_q8=xq_fill)
    xq_two = q.quantize_q8_0(to_dev(x))
    y_two = q.gemv_q8_0(wp, xq_two, rows, cols, 1)
    torch.cuda.synchronize()
    assert np.array_equal(q8_canonical(xq, 1, cols), oracle.quantize_q8_0(x))
    assert torch.equal(xq, xq_two)                                   # padded d_x entries included
    assert torch.equal(y, y_two)


def test_gemv_q8_unit_weights_exact():
    # every weight 1 with d_w = 1, integer activations whose blocks hold +-127:
    # d_x = 1, q = x, so y = sum(x) exactly for every row
    rows, cols, n = 130, 4128, 3
    w8 = np.zeros((rows, cols // 32, 34), np.uint8)
    w8[..., 0:2] = [0x00, 0x3c]
    w8[..., 2:] = 1
    rng = np.random.default_rng(3)
    x = rng.integers(-127, 128, size=(n, cols)).astype(np.float32)
    x[:, ::32] = 127.0
    y = q.gemv_q8_0(_packed(w8, rows, cols), q.quantize_q8_0(to_dev(x)), rows, cols, n).cpu().numpy()
    assert np.array_equal(y, np.repeat(x.sum(1, dtype=np.float64)[:, None], rows, 1).astype(np.float32))


def test_gemv_q8_empty_shapes():
    wp = _packed(np.zeros((64, 0, 34), np.uint8), 64, 0)
    xq = torch.zeros(q.q8_bytes(2, 0) or 16, dtype=torch.uint8, device=dev())
    y = torch.full((2, 64), 7.0, device=dev())
    q.gemv_q8_0(wp if wp.numel() else torch.zeros(16, dtype=torch.uint8, device=dev()), xq, 64, 0, 2, out=y)
    assert (y.cpu().numpy() == 0).all()                  # cols == 0: the empty sum
    y0 = torch.empty((1, 0), device=dev())
    q.gemv_q8_0(torch.zeros(16, dtype=torch.uint8, device=dev()), xq, 0, 64, 1, out=y0)


@pytest.mark.parametrize("n", [1, 8])
def test_gemv_q8_lm_head_full(oracle, n):
    # the 8-bit output head of the 1.5B stack: 151936 x 1536 (248 MB)
    rows, cols = 151936, 1536
    rng = synth.generator(3, 196, 0, 0)
    w8 = synth.q8_0_weights(rows, cols, rng)
    x = synth.activation(n, cols, synth.generator(3, 196, 0, 1), outliers=0)
    y, y_ref, S, _ = _run(w8, x, rows, cols, n, oracle)
    assert_within(y, y_ref, S, what=f"q8 lm_head n={n}")


def test_gemv_q8_from_f32_lm_head_full(oracle):
    # the one-launch form at the benchmark's 151936 x 1536 head: against the oracle, and the
    # two-launch form bit for bit
    rows, cols = 151936, 1536
    w8 = synth.q8_0_weights(rows, cols, synth.generator(3, 196, 0, 0))
    x = synth.activation(1, cols, synth.generator(3, 196, 0, 1), outliers=0)
    wp = _packed(w8, rows, cols)
    y, xq = q.gemv_q8_0_f32(wp, to_dev(x), rows, cols)
    y_two = q.gemv_q8_0(wp, q.quantize_q8_0(to_dev(x)), rows, cols, 1)
    assert torch.equal(y, y_two)
    xq_ref = oracle.quantize_q8_0(x)
    assert np.array_equal(q8_canonical(xq, 1, cols), xq_ref)
    y_ref, S = oracle.q8w_gemv(w8, xq_ref, rows, cols, 1)
    assert_within(y.cpu().numpy(), y_ref, S, what="q8 lm_head from f32")


# --------------------------------------------------------------- requant

RQ = load_golden("requant_q4_0.txt")


def test_requant_golden_blocks():
    q8 = np.stack([np.array([int(t, 16) for t in c["q8"]], np.uint8) for c in RQ])
    want = np.stack([np.array([int(t, 16) for t in c["q4"]], np.uint8) for c in RQ])
    got = q.requant_q8_0_to_q4_0(to_dev(q8.reshape(-1)), 1, 32 * len(RQ)).cpu().numpy().reshape(len(RQ), 18)
    assert np.array_equal(got, want)


def _requant_inputs(rows, cols, seed):
    rng = np.random.default_rng(seed)
    w8 = synth.q8_0_weights(rows, cols, rng).reshape(-1, 34)
    nblk = w8.shape[0]
    # special blocks: negative and subnormal scales, zero values, -128, magnitude ties
    w8[::7, 1] |= 0x80
    w8[3::11, 0:2] = [0x01, 0x00]
    w8[5::13, 2:] = 0
    w8[6::17, 2 + 9] = 0x80
    t = np.arange(nblk)[::19]
    w8[t, 2:] = 3
    w8[t, 2 + 4] = 100
    w8[t, 2 + 20] = 0x9c                                   # -100: the same magnitude, later
    return w8.reshape(rows, cols // 32, 34)


@pytest.mark.parametrize("rows,cols", [(64, 256), (257, 1536), (151936, 1536)])
def test_requant_bit_exact(oracle, rows, cols):
    w8 = _requant_inputs(rows, cols, rows + cols)
    got = q.requant_q8_0_to_q4_0(to_dev(w8.reshape(-1)), rows, cols).cpu().numpy()
    assert np.array_equal(got.reshape(rows, cols // 32, 18), oracle.requant_q8_0_to_q4_0(w8))


def test_requant_then_q4_gemv(oracle):
    # the load path of an 8-bit head: requantize, repack, stream as Q4_0
    rows, cols, n = 1536, 1536, 2
    w8 = _requant_inputs(rows, cols, 77)
    w4 = q.requant_q8_0_to_q4_0(to_dev(w8.reshape(-1)), rows, cols)
    wp = q.repack_q4_0(w4, rows, cols)
    x = synth.activation(n, cols, np.random.default_rng(78))
    y = q.gemv_q4_0(wp, q.quantize_q8_0(to_dev(x)), rows, cols, n).cpu().numpy()
    y_ref, S = oracle.gemv(oracle.requant_q8_0_to_q4_0(w8), oracle.quantize_q8_0(x), rows, cols, n)
    assert_within(y, y_ref, S, what="requant -> q4 gemv")
