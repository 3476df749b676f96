"""ctypes front end of the plain C oracle (``q4_oracle.c``).  Test infrastructure only.

The oracle is a slow, obviously correct CPU implementation of what the GPU path
computes (the "minfer" README on the nano-inference page: the Q4_0 weight
format of the GGUF loader bullet, the int8 activations of milestone M3.5, the
per-block integer sums with the (nibble - 8) offset of milestone M9, and the
block sizes of milestone M14).  Only ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg may import this module; the product
path never does.  It shares no code with the HIP library.

Canonical layouts used here:
  Q4_0 weights : uint8 [rows][cols/32][18]  (fp16 d little-endian, 16 nibble bytes)
  Q8_0 blocks  : uint8 [n][cols/32][34]     (fp16 d little-endian, 32 int8 q)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

QK = 32
Q4_BLOCK_BYTES = 18
Q8_BLOCK_BYTES = 34


def build(force: bool = True) -> str:
    """Compile q4_oracle.c with plain gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    L = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    L.q4o_fp16_to_f32.argtypes = [ctypes.c_uint16]
    L.q4o_fp16_to_f32.restype = ctypes.c_float
    L.q4o_f32_to_fp16.argtypes = [ctypes.c_float]
    L.q4o_f32_to_fp16.restype = ctypes.c_uint16
    L.q4o_fp16_to_f32_array.argtypes = [p, p, i64]
    L.q4o_f32_to_fp16_array.argtypes = [p, p, i64]
    L.q4o_quantize_q8_0.argtypes = [p, p, i64]
    L.q4o_quantize_q8_0_block.argtypes = [p, p]
    L.q4o_decode_q4_0.argtypes = [p, p, p, i64]
    L.q4o_block_dot.argtypes = [p, p]
    L.q4o_block_dot.restype = ctypes.c_int32
    L.q4o_block_sums.argtypes = [p, p, i64, i64, ctypes.c_int, p]
    L.q4o_gemv.argtypes = [p, p, i64, i64, ctypes.c_int, p, p, p]
    L.q4o_gemv_rows.argtypes = [p, p, i64, ctypes.c_int, p, i64, p, p]
    L.q4o_q8w_block_dot.argtypes = [p, p]
    L.q4o_q8w_block_dot.restype = ctypes.c_int32
    L.q4o_q8w_block_sums.argtypes = [p, p, i64, i64, ctypes.c_int, p]
    L.q4o_q8w_gemv.argtypes = [p, p, i64, i64, ctypes.c_int, p, p, p]
    L.q4o_requant_block_q8_0_to_q4_0.argtypes = [p, p]
    L.q4o_requant_q8_0_to_q4_0.argtypes = [p, p, i64]
    L.q4o_attn_decode.argtypes = [p, p, p, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double, p, p]
    L.q4o_gemv_f32.argtypes = [p, p, i64, i64, ctypes.c_int, p]
    L.q4o_gemv_f32_rows.argtypes = [p, p, i64, ctypes.c_int, p, i64, p]
    L.q4o_rmsnorm.argtypes = [p, i64, p]
    L.q4o_rmsnorm.restype = ctypes.c_float
    L.q4o_chain_step.argtypes = [p, ctypes.c_int, i64, i64, i64, i64, p, p, p]
    L.q4o_set_threads.argtypes = [ctypes.c_int]
    L.q4o_max_threads.restype = ctypes.c_int
    return L


def lib():
    """The default oracle library (built from q4_oracle.c if missing or stale)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(_LIB_PATH)
    return _lib


class _Use:
    """Temporarily route this module's functions to another build of the oracle
    (used only by the test that plants mistakes in a copy of the oracle)."""

    def __init__(self, path: str):
        self.L = _bind(path)

    def __enter__(self):
        global _lib
        self.prev, _lib = _lib, self.L
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev


def using(path: str) -> _Use:
    return _Use(path)


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> None:
    lib().q4o_set_threads(int(n))


def max_threads() -> int:
    return int(lib().q4o_max_threads())


# ---------------------------------------------------------------- binary16

def fp16_to_f32(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().q4o_fp16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


def f32_to_fp16(f: np.ndarray) -> np.ndarray:
    """Returns the binary16 bit patterns (uint16)."""
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().q4o_f32_to_fp16_array(_ptr(f), _ptr(out), f.size)
    return out


# ---------------------------------------------------------------- Q8_0

def quantize_q8_0(x: np.ndarray) -> np.ndarray:
    """x float32 [..., K] (K % 32 == 0) -> uint8 [..., K/32, 34] canonical Q8_0 blocks."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    K = x.shape[-1]
    assert K % QK == 0
    out = np.empty(x.shape[:-1] + (K // QK, Q8_BLOCK_BYTES), np.uint8)
    lib().q4o_quantize_q8_0(_ptr(x), _ptr(out), x.size)
    return out


def q8_split(blocks: np.ndarray):
    """Canonical Q8_0 blocks [..., nb, 34] -> (d fp16 bits [..., nb], q int8 [..., nb*32])."""
    blocks = np.ascontiguousarray(blocks)
    d = blocks[..., 0:2].copy().view(np.uint16)[..., 0]
    q = blocks[..., 2:].copy().view(np.int8)
    return d, q.reshape(blocks.shape[:-2] + (-1,))


# ---------------------------------------------------------------- Q4_0

def decode_q4_0(w: np.ndarray):
    """Q4_0 blocks [..., 18] -> (d float32 [...], nibbles uint8 [..., 32])."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    nblk = w.size // Q4_BLOCK_BYTES
    d = np.empty(nblk, np.float32)
    nib = np.empty(nblk * QK, np.uint8)
    lib().q4o_decode_q4_0(_ptr(w), _ptr(d), _ptr(nib), nblk)
    return d.reshape(w.shape[:-1]), nib.reshape(w.shape[:-1] + (QK,))


def block_dot(q4_block: np.ndarray, q8_block: np.ndarray) -> int:
    a = np.ascontiguousarray(q4_block, dtype=np.uint8)
    b = np.ascontiguousarray(q8_block, dtype=np.uint8)
    assert a.size == Q4_BLOCK_BYTES and b.size == Q8_BLOCK_BYTES
    return int(lib().q4o_block_dot(_ptr(a), _ptr(b)))


def block_sums(w: np.ndarray, xq8: np.ndarray, rows: int, cols: int, n: int) -> np.ndarray:
    """-> int32 [n][rows][cols/32]"""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xq8 = np.ascontiguousarray(xq8, dtype=np.uint8)
    assert w.size == rows * (cols // QK) * Q4_BLOCK_BYTES
    assert xq8.size == n * (cols // QK) * Q8_BLOCK_BYTES
    s = np.empty((n, rows, cols // QK), np.int32)
    lib().q4o_block_sums(_ptr(w), _ptr(xq8), rows, cols, n, _ptr(s))
    return s


def gemv(w: np.ndarray, xq8: np.ndarray, rows: int, cols: int, n: int, want_y64: bool = False):
    """-> (y float32 [n][rows], S float64 [n][rows][, y64 float64 [n][rows]])"""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xq8 = np.ascontiguousarray(xq8, dtype=np.uint8)
    assert w.size == rows * (cols // QK) * Q4_BLOCK_BYTES
    assert xq8.size == n * (cols // QK) * Q8_BLOCK_BYTES
    y = np.empty((n, rows), np.float32)
    S = np.empty((n, rows), np.float64)
    y64 = np.empty((n, rows), np.float64) if want_y64 else None
    lib().q4o_gemv(_ptr(w), _ptr(xq8), rows, cols, n, _ptr(y), _ptr(S),
                   _ptr(y64) if want_y64 else None)
    return (y, S, y64) if want_y64 else (y, S)


def gemv_rows(w: np.ndarray, xq8: np.ndarray, cols: int, n: int, row_idx: np.ndarray):
    """Selected output rows of the full matrix w -> (y [n][len(row_idx)], S [n][len(row_idx)])."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xq8 = np.ascontiguousarray(xq8, dtype=np.uint8)
    idx = np.ascontiguousarray(row_idx, dtype=np.int64)
    rows = w.size // ((cols // QK) * Q4_BLOCK_BYTES)
    assert idx.size == 0 or (idx.min() >= 0 and idx.max() < rows)
    y = np.empty((n, idx.size), np.float32)
    S = np.empty((n, idx.size), np.float64)
    lib().q4o_gemv_rows(_ptr(w), _ptr(xq8), cols, n, _ptr(idx), idx.size, _ptr(y), _ptr(S))
    return y, S


def gemv_f32(w: np.ndarray, xq8: np.ndarray, rows: int, cols: int, n: int) -> np.ndarray:
    """The GEMV in the fixed fp32 order (milestone M16 reading) -> y float32 [n][rows]."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xq8 = np.ascontiguousarray(xq8, dtype=np.uint8)
    assert w.size == rows * (cols // QK) * Q4_BLOCK_BYTES
    assert xq8.size == n * (cols // QK) * Q8_BLOCK_BYTES
    y = np.empty((n, rows), np.float32)
    lib().q4o_gemv_f32(_ptr(w), _ptr(xq8), rows, cols, n, _ptr(y))
    return y


def gemv_f32_rows(w: np.ndarray, xq8: np.ndarray, cols: int, n: int, row_idx: np.ndarray) -> np.ndarray:
    """Selected rows of the fixed-order fp32 GEMV -> y float32 [n][len(row_idx)]."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xq8 = np.ascontiguousarray(xq8, dtype=np.uint8)
    idx = np.ascontiguousarray(row_idx, dtype=np.int64)
    rows = w.size // ((cols // QK) * Q4_BLOCK_BYTES)
    assert idx.size == 0 or (idx.min() >= 0 and idx.max() < rows)
    y = np.empty((n, idx.size), np.float32)
    lib().q4o_gemv_f32_rows(_ptr(w), _ptr(xq8), cols, n, _ptr(idx), idx.size, _ptr(y))
    return y


# ---------------------------------------------------------------- chained step

def rmsnorm(x: np.ndarray):
    """-> (x / sqrt(ss/n + 1e-6) float32, ss) with ss in the fixed order (see q4_oracle.c)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    ss = lib().q4o_rmsnorm(_ptr(x), x.size, _ptr(out))
    return out, float(ss)


def rmsnorm_f64(x: np.ndarray) -> np.ndarray:
    """The RMS norm of the chained step by its plain definition, in fp64 and with no
    prescribed summation order: x / sqrt(mean(x^2) + 1e-6) -- Qwen2.5's RMS norm with its
    epsilon of 1e-6 and no learned weight (the synthetic model's norm weights are 1); the
    pages name the "norm prologues" of milestone M19 without a formula.  Returns float64."""
    x64 = np.asarray(x, dtype=np.float64)
    return x64 / np.sqrt(np.mean(x64 * x64) + 1e-6)


def chain_layout(E: int, D: int, F: int):
    """Offsets of q, k, v, o, h1, g, u, dn, h2 within one layer's block of activations."""
    sizes = [("q", E), ("k", D), ("v", D), ("o", E), ("h1", E), ("g", F), ("u", F), ("dn", E), ("h2", E)]
    off, out = 0, {}
    for name, n in sizes:
        out[name] = (off, n)
        off += n
    return out, off


def chain_step(weights, E: int, D: int, F: int, V: int, h0: np.ndarray):
    """One chained decode step.  weights: 7*layers + 1 canonical Q4_0 arrays (q, k, v, o, gate,
    up, down per layer, then the head).  Returns (acts float32 [layers][per_layer], logits [V])."""
    assert len(weights) % 7 == 1
    layers = len(weights) // 7
    shapes = [(E, E), (D, E), (D, E), (E, E), (F, E), (F, E), (E, F)] * layers + [(V, E)]
    ws = [np.ascontiguousarray(w, dtype=np.uint8) for w in weights]
    for w, (r, c) in zip(ws, shapes):
        assert w.size == r * (c // QK) * Q4_BLOCK_BYTES
    h0 = np.ascontiguousarray(h0, dtype=np.float32)
    assert h0.size == E
    _, per = chain_layout(E, D, F)
    acts = np.empty((layers, per), np.float32)
    logits = np.empty(V, np.float32)
    ptrs = (ctypes.c_void_p * len(ws))(*[w.ctypes.data for w in ws])
    lib().q4o_chain_step(ptrs, layers, E, D, F, V, _ptr(h0), _ptr(acts), _ptr(logits))
    return acts, logits


# ---------------------------------------------------------------- Q8_0 weights

def q8w_block_dot(w_block: np.ndarray, x_block: np.ndarray) -> int:
    a = np.ascontiguousarray(w_block, dtype=np.uint8)
    b = np.ascontiguousarray(x_block, dtype=np.uint8)
    assert a.size == Q8_BLOCK_BYTES and b.size == Q8_BLOCK_BYTES
    return int(lib().q4o_q8w_block_dot(_ptr(a), _ptr(b)))


def q8w_block_sums(w: np.ndarray, xq8: np.ndarray, rows: int, cols: int, n: int) -> np.ndarray:
    """Q8_0 weights [rows][cols/32][34] x Q8_0 activations -> int32 [n][rows][cols/32]"""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xq8 = np.ascontiguousarray(xq8, dtype=np.uint8)
    assert w.size == rows * (cols // QK) * Q8_BLOCK_BYTES
    assert xq8.size == n * (cols // QK) * Q8_BLOCK_BYTES
    s = np.empty((n, rows, cols // QK), np.int32)
    lib().q4o_q8w_block_sums(_ptr(w), _ptr(xq8), rows, cols, n, _ptr(s))
    return s


def q8w_gemv(w: np.ndarray, xq8: np.ndarray, rows: int, cols: int, n: int, want_y64: bool = False):
    """Q8_0-weight GEMV -> (y float32 [n][rows], S float64 [n][rows][, y64])"""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    xq8 = np.ascontiguousarray(xq8, dtype=np.uint8)
    assert w.size == rows * (cols // QK) * Q8_BLOCK_BYTES
    assert xq8.size == n * (cols // QK) * Q8_BLOCK_BYTES
    y = np.empty((n, rows), np.float32)
    S = np.empty((n, rows), np.float64)
    y64 = np.empty((n, rows), np.float64) if want_y64 else None
    lib().q4o_q8w_gemv(_ptr(w), _ptr(xq8), rows, cols, n, _ptr(y), _ptr(S),
                       _ptr(y64) if want_y64 else None)
    return (y, S, y64) if want_y64 else (y, S)


def requant_q8_0_to_q4_0(w_q8: np.ndarray) -> np.ndarray:
    """Q8_0 blocks [..., 34] -> Q4_0 blocks [..., 18] (load-time requantization)."""
    a = np.ascontiguousarray(w_q8, dtype=np.uint8)
    assert a.shape[-1] == Q8_BLOCK_BYTES
    nblk = a.size // Q8_BLOCK_BYTES
    out = np.empty(a.shape[:-1] + (Q4_BLOCK_BYTES,), np.uint8)
    lib().q4o_requant_q8_0_to_q4_0(_ptr(a), _ptr(out), nblk)
    return out


# ---------------------------------------------------------------- attention

def attn_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None):
    """Decode attention in fp64: q [n_q][hd], k and v [L][n_kv][hd] (fp32).
    Returns (o [n_q][hd] fp64, o_abs [n_q][hd] fp64 = sum_j p_hj |v_j|)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    n_q, hd = q.shape
    L, n_kv, hd2 = k.shape
    assert hd2 == hd and v.shape == k.shape and n_q % n_kv == 0
    if scale is None:
        scale = 1.0 / np.sqrt(hd)
    o = np.empty((n_q, hd), np.float64)
    o_abs = np.empty((n_q, hd), np.float64)
    lib().q4o_attn_decode(_ptr(q), _ptr(k), _ptr(v), L, n_q, n_kv, hd, float(scale), _ptr(o), _ptr(o_abs))
    return o, o_abs
