"""Independent fp64 brute-force check of the C oracle.  Test infrastructure only.

Dequantizes both operands to fp64 with NumPy's own binary16 decoding and forms
the product with a plain matrix multiply:

    W[r, 32b + j] = (nibble_{r,b,j} - 8) * d_w[r, b]      (Q4_0, GGUF element order)
    X[n, 32b + j] = q_{n,b,j} * d_x[n, b]                   (Q8_0)
    y64 = X @ W.T                                           (fp64)

This reaches the GEMV result by a different route from ``q4_oracle.c``
(dequantize-then-matmul instead of per-block integer sums), so agreement pins
the oracle's block decoding, offset handling and scaling.  It shares no code
with the oracle or with the GPU path.
"""
from __future__ import annotations

import numpy as np


def dequant_q4_0(w: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Q4_0 blocks [rows][cols/32][18] -> fp64 [rows][cols]."""
    w = np.asarray(w, dtype=np.uint8).reshape(rows, cols // 32, 18)
    d = w[:, :, 0:2].copy().view("<f2")[:, :, 0].astype(np.float64)  # NumPy binary16 decode
    qs = w[:, :, 2:].astype(np.int64)
    lo = qs & 0x0F          # elements 0..15
    hi = qs >> 4            # elements 16..31
    nib = np.concatenate([lo, hi], axis=2)  # [rows][nb][32]
    return ((nib - 8).astype(np.float64) * d[:, :, None]).reshape(rows, cols)


def dequant_q8_0(xq8: np.ndarray, n: int, cols: int) -> np.ndarray:
    """Q8_0 blocks [n][cols/32][34] -> fp64 [n][cols]."""
    x = np.asarray(xq8, dtype=np.uint8).reshape(n, cols // 32, 34)
    d = x[:, :, 0:2].copy().view("<f2")[:, :, 0].astype(np.float64)
    q = x[:, :, 2:].copy().view(np.int8).astype(np.float64)
    return (q * d[:, :, None]).reshape(n, cols)


def dequant_q8_0_weights(w: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Q8_0 weight blocks [rows][cols/32][34] -> fp64 [rows][cols]."""
    return dequant_q8_0(w, rows, cols)


def q8w_gemv64(w: np.ndarray, xq8: np.ndarray, rows: int, cols: int, n: int) -> np.ndarray:
    """fp64 y [n][rows] of a Q8_0-weight GEMV by dequantize-then-matmul."""
    return dequant_q8_0(xq8, n, cols) @ dequant_q8_0_weights(w, rows, cols).T


def gemv64(w: np.ndarray, xq8: np.ndarray, rows: int, cols: int, n: int) -> np.ndarray:
    """fp64 y [n][rows] by dequantize-then-matmul."""
    W = dequant_q4_0(w, rows, cols)
    X = dequant_q8_0(xq8, n, cols)
    return X @ W.T


def chain64(weights, E: int, D: int, F: int, V: int, h0: np.ndarray):
    """The chained step with exact (unquantized) activations, in fp64: each matrix is
    dequantized and applied to the activation itself, norms in fp64.  Differs from the
    quantized chain only by the Q8_0 rounding of the activations.
    Returns (dict of per-layer vectors, logits)."""
    layers = len(weights) // 7
    def nrm(x):
        return x / np.sqrt(np.mean(x * x) + 1e-6)
    h = np.asarray(h0, dtype=np.float64)
    out = []
    for l in range(layers):
        Wq, Wk, Wv, Wo, Wg, Wu, Wd = (
            dequant_q4_0(weights[7 * l + i], r, c)
            for i, (r, c) in enumerate([(E, E), (D, E), (D, E), (E, E), (F, E), (F, E), (E, F)]))
        a = nrm(h)
        q, k, v = Wq @ a, Wk @ a, Wv @ a
        o = Wo @ q
        h1 = h + o
        c = nrm(h1)
        g, u = Wg @ c, Wu @ c
        dn = Wd @ (g * u)
        h2 = h1 + dn
        out.append(dict(q=q, k=k, v=v, o=o, h1=h1, g=g, u=u, dn=dn, h2=h2))
        h = h2
    logits = dequant_q4_0(weights[-1], V, E) @ nrm(h)
    return out, logits
