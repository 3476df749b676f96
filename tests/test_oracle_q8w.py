"""Pins of the oracle's Q8_0-weight GEMV and of the Q8_0 -> Q4_0 requantization.

Definitions: minfer README (nano-inference page) -- the int8 lm_head of
milestone M6 and the gemv_q8_dp4a bullet of "How it works" (Q8_0 weights,
int8 MACs against the same Q8_0 activation), the 34-byte Q8_0 block of
milestone M14, and the load-time requantization of 8-bit heads to Q4_0
(M14, M18; rounding rule read as the GGUF reference one).
"""
import numpy as np
import pytest

from conftest import load_golden, parse_number
from q4_weight_streaming_amd import synth

GEMV = load_golden("q8w_gemv_small.txt")[0]
RQ_CASES = load_golden("requant_q4_0.txt")


def _hex(tokens):
    return np.array([int(t, 16) for t in tokens], np.uint8)


def test_q8w_gemv_golden(oracle):
    rows, cols, n = int(GEMV["rows"][0]), int(GEMV["cols"][0]), int(GEMV["n"][0])
    w = np.stack([_hex(GEMV[f"w_row{r}"]) for r in range(rows)])
    x = np.stack([_hex(GEMV[f"x_row{t}"]) for t in range(n)])
    y, S = oracle.q8w_gemv(w, x, rows, cols, n)
    for t in range(n):
        assert list(y[t]) == [parse_number(v) for v in GEMV[f"y_row{t}"]]
        assert list(S[t]) == [parse_number(v) for v in GEMV[f"S_row{t}"]]


def test_q8w_block_sums_brute_force(oracle):
    rng = np.random.default_rng(21)
    rows, cols, n = 6, 160, 3
    w = synth.q8_0_weights(rows, cols, rng)
    x = synth.q8_0_weights(n, cols, rng)
    s = oracle.q8w_block_sums(w, x, rows, cols, n)
    wq = w[..., 2:].view(np.int8).astype(np.int64)       # [rows][nb][32]
    xq = x[..., 2:].view(np.int8).astype(np.int64)       # [n][nb][32]
    for t in range(n):
        for r in range(rows):
            for b in range(cols // 32):
                assert s[t, r, b] == sum(int(wq[r, b, j]) * int(xq[t, b, j]) for j in range(32))


@pytest.mark.parametrize("rows,cols,n", [(17, 288, 8), (70, 96, 1), (3, 2048, 2)])
def test_q8w_gemv_matches_fp64_bruteforce(oracle, bruteforce, rows, cols, n):
    rng = np.random.default_rng(rows * 1000 + cols + n)
    w = synth.q8_0_weights(rows, cols, rng)
    xq = oracle.quantize_q8_0(synth.activation(n, cols, rng))
    y, S, y64 = oracle.q8w_gemv(w, xq, rows, cols, n, want_y64=True)
    ref = bruteforce.q8w_gemv64(w, xq, rows, cols, n)
    # the oracle's fp64 sum of exact terms and the dequantized matmul agree to
    # fp64 rounding; y is that value rounded once to fp32
    assert np.all(np.abs(y64 - ref) <= 1e-12 * S + 1e-300)
    assert np.array_equal(y, y64.astype(np.float32))


def test_q8w_gemv_unit_weights_closed_form(oracle):
    # every weight 1 with d_w = 1: y = sum_b d_x[b] * sum_j q_j
    rows, cols, n = 3, 128, 2
    w = np.zeros((rows, cols // 32, 34), np.uint8)
    w[..., 0:2] = [0x00, 0x3c]
    w[..., 2:] = 1
    rng = np.random.default_rng(5)
    xq = oracle.quantize_q8_0(synth.activation(n, cols, rng))
    y, _ = oracle.q8w_gemv(w, xq, rows, cols, n)
    d = xq[..., 0:2].copy().view("<f2")[..., 0].astype(np.float64)
    q = xq[..., 2:].view(np.int8).astype(np.int64).sum(-1)
    expect = (d * q).sum(-1).astype(np.float32)
    for r in range(rows):
        assert np.array_equal(y[:, r], expect)


def test_q8w_block_dot_is_symmetric(oracle):
    rng = np.random.default_rng(8)
    a = synth.q8_0_weights(1, 32, rng)[0, 0]
    b = synth.q8_0_weights(1, 32, rng)[0, 0]
    assert oracle.q8w_block_dot(a, b) == oracle.q8w_block_dot(b, a)


@pytest.mark.parametrize("case", RQ_CASES, ids=[c["name"] for c in RQ_CASES])
def test_requant_golden(oracle, case):
    out = oracle.requant_q8_0_to_q4_0(_hex(case["q8"]))
    assert list(out) == list(_hex(case["q4"]))


def _embed_q4_in_q8(w4):
    """Q4_0 blocks [..., 18] -> the Q8_0 blocks [..., 34] holding the same values: d, n - 8."""
    nib = np.concatenate([w4[..., 2:] & 0x0F, w4[..., 2:] >> 4], axis=-1).astype(np.int8) - 8
    out = np.empty(w4.shape[:-1] + (34,), np.uint8)
    out[..., 0:2] = w4[..., 0:2]
    out[..., 2:] = nib.view(np.uint8)
    return out


def test_requant_round_trips_q4_0_blocks(oracle):
    # A Q4_0 block with a nibble 0 has its largest magnitude -8 d at that
    # nibble, so the rule recovers d exactly and every nibble: requantizing its
    # Q8_0 image gives the same 18 bytes back (positive and negative scales).
    rng = np.random.default_rng(31)
    w4 = synth.q4_0_weights(64, 32 * 16, rng).reshape(-1, 18)
    pos = rng.integers(0, 32, size=w4.shape[0])
    for i, p in enumerate(pos):                      # force one nibble 0
        if p < 16:
            w4[i, 2 + p] &= 0xF0
        else:
            w4[i, 2 + p - 16] &= 0x0F
    w4[::3, 1] |= 0x80                               # every third scale negative
    back = oracle.requant_q8_0_to_q4_0(_embed_q4_in_q8(w4))
    assert np.array_equal(back, w4)


def test_requant_rounds_to_nearest_level(oracle):
    # away from the rule's rounding details, each nibble is the nearest level
    # (n - 8) * d of the exact d = vmax / -8, clamped to 0..15
    rng = np.random.default_rng(41)
    w8 = synth.q8_0_weights(200, 32 * 8, rng).reshape(-1, 34)
    out = oracle.requant_q8_0_to_q4_0(w8)
    d8 = w8[:, 0:2].copy().view("<f2")[:, 0].astype(np.float64)
    x = w8[:, 2:].view(np.int8).astype(np.float64) * d8[:, None]
    imax = np.argmax(np.abs(x), axis=1)
    vmax = x[np.arange(len(x)), imax]
    ok = vmax != 0
    d = vmax[ok] / -8.0
    r = x[ok] / d[:, None] + 8.0
    near_half = np.abs(r - np.floor(r) - 0.5) < 1e-4
    expect = np.clip(np.floor(r + 0.5), 0, 15)
    nib = np.concatenate([out[ok, 2:] & 0x0F, out[ok, 2:] >> 4], axis=1)
    assert np.all((nib == expect) | near_half)
    assert np.all(nib[np.arange(len(nib)), imax[ok]] == 0)
    ds = out[ok, 0:2].copy().view("<f2")[:, 0].astype(np.float64)
    assert np.array_equal(ds, d.astype(np.float32).astype(np.float16).astype(np.float64))
