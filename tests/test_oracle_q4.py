"""Pins of the oracle's Q4_0 decoding, per-block integer sums and GEMV.

Definitions: minfer README (nano-inference page) -- Q4_0 GGUF weights (gguf.h
bullet of "How it works"), (nibble - 8) * d with an exact integer sum per
block (milestone M9), int8 activations (M3.5), 18/34-byte blocks (M14).
"""
import numpy as np
import pytest

from conftest import load_golden, parse_number
from q4_weight_streaming_amd import synth

Q4_CASES = load_golden("q4_0_blocks.txt")
SUM_CASES = load_golden("block_sums.txt")


@pytest.mark.parametrize("case", Q4_CASES, ids=[c["name"] for c in Q4_CASES])
def test_q4_0_golden_decode(oracle, case):
    blk = np.array([int(t, 16) for t in case["bytes"]], np.uint8)
    d, nib = oracle.decode_q4_0(blk)
    assert float(d) == parse_number(case["d"][0])
    assert list(nib) == [int(t) for t in case["nibbles"]]


def _expand(tokens, n, conv):
    vals = [conv(t) for t in tokens]
    return vals * n if len(vals) == 1 else vals


@pytest.mark.parametrize("case", SUM_CASES, ids=[c["name"] for c in SUM_CASES])
def test_block_sum_golden(oracle, case):
    qs = _expand(case["qs"], 16, lambda t: int(t, 16))
    q = _expand(case["q"], 32, int)
    w = np.array([0x00, 0x3c] + qs, np.uint8)          # d_w = 1
    x = np.zeros(34, np.uint8)
    x[0:2] = [0x00, 0x3c]                               # d_x = 1
    x[2:] = np.array(q, np.int8).view(np.uint8)
    assert oracle.block_dot(w, x) == int(case["s"][0])


def _nibbles_numpy(w):
    """Independent nibble extraction: low nibbles are elements 0..15, high 16..31."""
    qs = w[..., 2:18]
    return np.concatenate([qs & 0x0F, qs >> 4], axis=-1).astype(np.int64)


def test_block_sums_fold_identity_and_brute_force(oracle):
    # sum (n - 8) q == sum n q - 8 sum q  (milestone M9's folded offset), checked
    # against pure-Python loops on a small random set
    rng = np.random.default_rng(11)
    rows, cols, n = 5, 96, 3
    w = synth.q4_0_weights(rows, cols, rng)
    x = rng.standard_normal((n, cols)).astype(np.float32) * 3
    xq = oracle.quantize_q8_0(x)
    s = oracle.block_sums(w, xq, rows, cols, n)
    nib = _nibbles_numpy(w)                              # [rows][nb][32]
    q = xq[..., 2:].view(np.int8).astype(np.int64)       # [n][nb][32]
    fold = np.einsum("rbj,tbj->trb", nib, q) - 8 * q.sum(-1)[:, None, :]
    assert np.array_equal(s, fold)
    for t in range(n):
        for r in range(rows):
            for b in range(cols // 32):
                acc = 0
                for j in range(32):
                    byte = int(w[r, b, 2 + (j % 16)])
                    nibble = (byte & 15) if j < 16 else (byte >> 4)
                    acc += (nibble - 8) * int(q[t, b, j])
                assert s[t, r, b] == acc


def test_gemv_golden_small(oracle):
    g = load_golden("gemv_small.txt")[0]
    rows, cols = int(g["rows"][0]), int(g["cols"][0])
    w = np.array([[int(t, 16) for t in g["w_row0"]], [int(t, 16) for t in g["w_row1"]]],
                 np.uint8).reshape(rows, cols // 32, 18)
    x = np.array([parse_number(t) for t in g["x"]], np.float32)[None, :]
    xq = oracle.quantize_q8_0(x)
    y, S = oracle.gemv(w, xq, rows, cols, 1)
    assert list(y[0]) == [float(v) for v in g["y"]]
    assert list(S[0]) == [float(v) for v in g["S"]]


@pytest.mark.parametrize("rows,cols,n", [(1, 32, 1), (3, 64, 2), (70, 96, 1), (17, 288, 8),
                                         (129, 1536, 4), (40, 8960, 1)])
def test_gemv_matches_fp64_bruteforce(oracle, bruteforce, rows, cols, n):
    rng = synth.generator(99, rows, cols, n)
    w = synth.q4_0_weights(rows, cols, rng)
    x = synth.activation(n, cols, rng)
    xq = oracle.quantize_q8_0(x)
    y, S, y64 = oracle.gemv(w, xq, rows, cols, n, want_y64=True)
    ref = bruteforce.gemv64(w, xq, rows, cols, n)
    assert np.all(np.abs(y64 - ref) <= 1e-12 * S + 1e-300)
    # y is the fp32 rounding of the fp64 value
    assert np.all(np.abs(y.astype(np.float64) - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-12 * S)
    assert np.all(S >= np.abs(ref) * (1 - 1e-12))


def test_gemv_rows_selects_rows(oracle):
    rng = synth.generator(98, 0, 0, 0)
    rows, cols, n = 50, 128, 3
    w = synth.q4_0_weights(rows, cols, rng)
    xq = oracle.quantize_q8_0(synth.activation(n, cols, rng))
    y, S = oracle.gemv(w, xq, rows, cols, n)
    idx = np.array([49, 0, 7, 7, 31], np.int64)
    ys, Ss = oracle.gemv_rows(w, xq, cols, n, idx)
    assert np.array_equal(ys, y[:, idx]) and np.array_equal(Ss, S[:, idx])


def test_gemv_all_eight_nibbles_is_exact_zero(oracle):
    rng = np.random.default_rng(1)
    rows, cols = 9, 256
    w = synth.q4_0_weights(rows, cols, rng)
    w[..., 2:] = 0x88
    xq = oracle.quantize_q8_0(rng.standard_normal((2, cols)).astype(np.float32))
    y, S = oracle.gemv(w, xq, rows, cols, 2)
    assert np.all(y == 0) and np.all(S == 0)


def test_gemv_one_hot_activation_closed_form(oracle):
    # x = +-v at column k only: d_x = binary16(v/127), q_k = +-127, so
    # y_r = d_w[r, k//32] * d_x * (+-127) * (nibble_{r,k} - 8)
    rng = np.random.default_rng(2)
    rows, cols = 33, 320
    w = synth.q4_0_weights(rows, cols, rng)
    nib = _nibbles_numpy(w).reshape(rows, cols)
    dw = w[:, :, 0:2].copy().view("<f2")[:, :, 0].astype(np.float64)
    for k, v in [(0, 3.0), (17, -0.7), (31, 1e-3), (200, -55.5), (319, 2.0 ** -10)]:
        x = np.zeros((1, cols), np.float32)
        x[0, k] = v
        xq = oracle.quantize_q8_0(x)
        y, _ = oracle.gemv(w, xq, rows, cols, 1)
        dx = float(np.float16(np.float32(abs(v)) / np.float32(127)))
        expect = dw[:, k // 32] * dx * np.sign(v) * 127 * (nib[:, k] - 8)
        assert np.array_equal(y[0].astype(np.float64), expect.astype(np.float32).astype(np.float64))


def test_format_sizes_match_the_pages():
    g = load_golden("format_sizes.txt")[0]
    vocab, hidden = 151936, 1536
    assert vocab * hidden // 32 * 34 == int(g["lm_head_q8_0_bytes"][0])
    assert vocab * hidden // 32 * 18 == int(g["lm_head_q4_0_bytes"][0])
    total = sum(s.q4_bytes for s in synth.qwen25_1p5b())
    assert total == int(g["qwen25_1p5b_token_bytes"][0])
    assert round(total / 1e9, 3) == float(g["qwen25_1p5b_token_gb_stated"][0])
    assert len(synth.qwen25_1p5b()) == 197
