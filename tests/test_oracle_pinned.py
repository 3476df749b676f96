"""Pins of the oracle's fixed-order fp32 GEMV, its RMS norm and the chained step.

The fixed order is the reading of milestone M16 of the "minfer" README
(nano-inference page: every float operation explicitly rounded, so a token's
result does not depend on the step size).  Pins: hand-derived rows whose value
depends on the order (tests/golden/pinned_order.txt), exactness where every
order is exact, and the fp32 error bound against the fp64 GEMV.  The chained
step ("How it works", src/mega.cu bullet; M15, M19) is pinned by an independent
fp64 evaluation without quantization and by the special case in which it
reduces to one GEMV.
"""
import math
import os

import numpy as np
import pytest

from q4_weight_streaming_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pinned_order.txt")
U = 2.0 ** -24


def _load_cases():
    cases, cur = [], None
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *rest = line.split()
        if key == "case":
            cur = {"name": rest[0], "terms": []}
            cases.append(cur)
        elif key == "nb":
            cur["nb"] = int(rest[0])
        elif key == "term":
            cur["terms"].append((int(rest[0]), int(rest[1])))
        elif key == "expect":
            cur["expect"] = float(rest[0])
    return cases


CASES = _load_cases()
_SCALES = {2 ** 24: (4096.0, 4096.0), 2 ** 25: (8192.0, 4096.0), 2: (2.0, 1.0), 1: (1.0, 1.0)}


def term_row(nb, terms):
    """One Q4_0 row and one Q8_0 activation whose block b contributes exactly the given terms."""
    w = np.zeros((1, nb, 18), np.uint8)
    x = np.zeros((1, nb, 34), np.uint8)
    one = np.array([1.0], "<f2").view(np.uint8)
    w[0, :, 0:2] = one
    w[0, :, 2:] = 0x88                      # every nibble 8: weight value 0
    x[0, :, 0:2] = one                      # q = 0
    for b, t in terms:
        dw, dx = _SCALES[t]
        w[0, b, 0:2] = np.array([dw], "<f2").view(np.uint8)
        w[0, b, 2] = 0x89                   # element 0 has nibble 9: weight 1 * d_w
        x[0, b, 0:2] = np.array([dx], "<f2").view(np.uint8)
        x[0, b, 2] = 1                      # q_0 = 1: s = 1
    return w, x


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_pinned_order_golden(oracle, case):
    w, x = term_row(case["nb"], case["terms"])
    y = oracle.gemv_f32(w, x, 1, case["nb"] * 32, 1)
    assert y[0, 0] == np.float32(case["expect"]), (case["name"], float(y[0, 0]))


@pytest.mark.parametrize("rows,cols,n", [(70, 256, 3), (33, 2304, 2), (9, 4608, 1), (5, 17408, 1)])
def test_pinned_exact_with_unit_scales(oracle, rows, cols, n):
    """Scales 1: every partial sum is an integer far below 2^24, so every order is exact."""
    rng = synth.generator(91, rows, cols, 0)
    w = synth.q4_0_weights(rows, cols, rng)
    w[:, :, 0:2] = np.array([1.0], "<f2").view(np.uint8)
    xq = np.zeros((n, cols // 32, 34), np.uint8)
    xq[:, :, 0:2] = np.array([1.0], "<f2").view(np.uint8)
    xq[:, :, 2:] = rng.integers(-127, 128, size=(n, cols // 32, 32)).astype(np.int8).view(np.uint8)
    y32 = oracle.gemv_f32(w, xq, rows, cols, n)
    _, _, y64 = oracle.gemv(w, xq, rows, cols, n, want_y64=True)
    assert np.abs(y64).max() < 2 ** 23
    np.testing.assert_array_equal(y32, y64.astype(np.float32))


@pytest.mark.parametrize("rows,cols,n", [(130, 1536, 2), (64, 8960, 1), (17, 18944, 1), (40, 800, 3)])
def test_pinned_within_fp32_bound_of_fp64(oracle, rows, cols, n):
    """Each rounding errs by at most 2^-24 of a partial sum, itself at most S: one per
    block, two per segment, one per range -> |y32 - y64| <= (nb + 2 nc + 4) 2^-24 S."""
    w = synth.q4_0_weights(rows, cols, synth.generator(92, rows, cols, 0))
    x = synth.activation(n, cols, synth.generator(92, rows, cols, 1))
    xq = oracle.quantize_q8_0(x)
    y32 = oracle.gemv_f32(w, xq, rows, cols, n)
    _, S, y64 = oracle.gemv(w, xq, rows, cols, n, want_y64=True)
    nb = cols // 32
    nc = (nb + 7) // 8
    assert np.all(np.abs(y32.astype(np.float64) - y64) <= (nb + 2 * nc + 4) * U * S)
    idx = np.array([0, rows // 2, rows - 1])
    np.testing.assert_array_equal(oracle.gemv_f32_rows(w, xq, cols, n, idx), y32[:, idx])


# ---------------------------------------------------------------- RMS norm

def test_rmsnorm_order_golden(oracle):
    """256 values: lane l of the 64 partial sums owns elements 4l..4l+3.  x_0 = 4096
    (square 2^24) and x_1 = 1 (lane 0: 2^24 + 1 ties back to 2^24), x_4 = x_8 = x_12 = 1
    (lanes 1, 2, 3), x_128 = 1 (lane 32).
    The tree (32, 16, 8, 4, 2, 1): p_0 = 2^24 + 1 -> 2^24 (tie to even); at d = 2,
    p_0 = 2^24 + p_2 -> 2^24 and p_1 = p_1 + p_3 = 2; at d = 1, p_0 = 2^24 + 2.  (The
    reverse tree gives 2^24 + 4, a sequential sum 2^24; lanes owning elements l, l + 64,
    l + 128, l + 192 put x_1 on lane 1 and end at 2^24 + 3 -> 2^24 + 4.)  Then ss / 256 = 2^16 + 2^-7
    exactly, + 1e-6 rounds back, and sqrt(2^16 + 2^-7) = 256 + 2^-16 - tiny rounds to
    256: the outputs are x / 256 exactly (2^24 + 4 would give 256 + 2^-15)."""
    x = np.zeros(256, np.float32)
    x[0] = 4096.0
    x[[1, 4, 8, 12, 128]] = 1.0
    out, ss = oracle.rmsnorm(x)
    assert ss == 2.0 ** 24 + 2
    np.testing.assert_array_equal(out, x / np.float32(256.0))


@pytest.mark.parametrize("c,n", [(2.0 ** -10, 64), (2.0 ** -10, 1536), (3.0, 128), (1e-4, 3584)])
def test_rmsnorm_constant_vector_closed_form(oracle, c, n):
    """x_i = c for all i: the result is c / sqrt(c^2 + 1e-6) in every element (to 3 ulp)."""
    out, _ = oracle.rmsnorm(np.full(n, c, np.float32))
    c32 = float(np.float32(c))
    ref = c32 / np.sqrt(c32 * c32 + 1e-6)
    assert np.all(np.abs(out.astype(np.float64) - ref) <= 3 * U * abs(ref) * 2)


def test_rmsnorm_within_bound_of_fp64(oracle):
    x = synth.activation(1, 8960, synth.generator(93, 0, 0, 1))[0]
    out, ss = oracle.rmsnorm(x)
    x64 = x.astype(np.float64)
    ss64 = float(np.sum(x64 * x64))
    assert abs(ss - ss64) <= (8960 / 64 + 8) * U * ss64
    ref = x64 / np.sqrt(ss64 / 8960 + 1e-6)
    assert np.all(np.abs(out - ref) <= 1e-5 * np.abs(ref) + 1e-30)


@pytest.mark.parametrize("c,n", [(1e-3, 64), (1e-3, 1536), (3.0, 128), (1e-4, 3584)])
def test_rmsnorm_f64_constant_vector_closed_form(oracle, c, n):
    """The order-free fp64 norm on x_i = c: c / sqrt(c^2 + 1e-6).  At c = 1e-3 the epsilon is
    as large as the mean square (result 1/sqrt(2)), so a wrong epsilon, a sum in place of the
    mean or a missing square root moves it far beyond the 4-ulp margin."""
    out = oracle.rmsnorm_f64(np.full(n, c, np.float32))
    c32 = float(np.float32(c))
    ref = c32 / math.sqrt(c32 * c32 + 1e-6)
    assert out.dtype == np.float64 and np.all(np.abs(out - ref) <= 4 * 2.0 ** -53 * abs(ref))
    if c == 1e-3:
        assert abs(out[0] - 2 ** -0.5) < 1e-3


def test_rmsnorm_f64_exact_arithmetic():
    """Against the definition in exact rational arithmetic (the mean square as a fraction,
    the square root to 40 digits): every element within 1e-15 relative."""
    from decimal import Decimal, getcontext
    from fractions import Fraction
    from oracle import oracle
    getcontext().prec = 40
    x = synth.activation(1, 96, synth.generator(94, 0, 0, 1))[0]
    ms = sum(Fraction(float(v)) ** 2 for v in x) / len(x) + Fraction(1, 10 ** 6)
    root = (Decimal(ms.numerator) / Decimal(ms.denominator)).sqrt()
    out = oracle.rmsnorm_f64(x)
    for v, o in zip(x, out):
        exact = Decimal(float(v)) / root
        assert abs(Decimal(float(o)) - exact) <= Decimal("1e-15") * abs(exact) + Decimal("1e-300")


def test_rmsnorm_fixed_order_within_fp32_bound_of_f64(oracle):
    """The fixed-order fp32 norm against the order-free fp64 one: each output within
    ((n/64 + 6)/2 + 4) ulp-units (2^-24) of relative error -- the bound the GPU norm-phase
    check uses (half the sum of squares' chain and butterfly error, then the mean, epsilon,
    square root and division)."""
    for n, seed in [(1536, 95), (3584, 96), (8960, 97)]:
        x = synth.activation(1, n, synth.generator(seed, 0, 0, 1))[0]
        out, _ = oracle.rmsnorm(x)
        ref = oracle.rmsnorm_f64(x)
        delta = ((n / 64 + 6) / 2 + 4) * U
        assert np.all(np.abs(out - ref) <= delta * np.abs(ref) + 1e-30)


# ---------------------------------------------------------------- chained step

E, D, F, V, L = 256, 64, 384, 320, 2


def _chain_inputs(seed):
    shapes = [(E, E), (D, E), (D, E), (E, E), (F, E), (F, E), (E, F)] * L + [(V, E)]
    ws = [synth.q4_0_weights(r, c, synth.generator(seed, m, 0, 0)) for m, (r, c) in enumerate(shapes)]
    # a small input without outlier channels, so that the attention-side branch o is
    # comparable to h and every branch of the step shows in the outputs
    h0 = 0.05 * synth.activation(1, E, synth.generator(seed, 999, 0, 1), outliers=0)[0]
    return ws, h0


def test_chain_matches_unquantized_fp64(oracle, bruteforce):
    """Without quantization (fp64 activations) the chain differs only by the Q8_0 rounding of
    its activations (at most 1/254 of a block's largest value per element, compounding over
    the phases: 0.4-2.3% of a vector's largest element here); every vector agrees within
    5% of its largest element, while a miswired step moves some vector by 30% or more."""
    ws, h0 = _chain_inputs(94)
    acts, logits = oracle.chain_step(ws, E, D, F, V, h0)
    ref, ref_logits = bruteforce.chain64(ws, E, D, F, V, h0)
    lay, _ = oracle.chain_layout(E, D, F)
    for l in range(L):
        for name, (off, n) in lay.items():
            got, want = acts[l, off:off + n], ref[l][name]
            assert np.abs(got - want).max() <= 0.05 * np.abs(want).max(), (l, name)
    assert np.abs(logits - ref_logits).max() <= 0.05 * np.abs(ref_logits).max()


def test_chain_without_residual_branches_is_one_gemv(oracle):
    """Zero output and down projections: every layer returns its input, so the logits are
    the head applied to Q8_0(norm(h0)) -- one GEMV -- and h1 = h2 = h0 in every layer."""
    ws, h0 = _chain_inputs(95)
    for l in range(L):
        for i in (3, 6):
            ws[7 * l + i] = ws[7 * l + i].copy()
            ws[7 * l + i][..., 0:2] = 0         # d_w = +0
    acts, logits = oracle.chain_step(ws, E, D, F, V, h0)
    lay, _ = oracle.chain_layout(E, D, F)
    for l in range(L):
        for name in ("h1", "h2"):
            off, n = lay[name]
            np.testing.assert_array_equal(acts[l, off:off + n], h0)
    nrm, _ = oracle.rmsnorm(h0)
    np.testing.assert_array_equal(logits, oracle.gemv_f32(ws[-1], oracle.quantize_q8_0(nrm[None]), V, E, 1)[0])
