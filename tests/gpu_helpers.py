"""Helpers for the GPU parity tests: device transfer and test-side views of the
library's documented layouts.  None of this holds the method's arithmetic."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from q4_weight_streaming_amd import _lib as q


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def packed_weights(w_canon: np.ndarray, rows: int, cols: int) -> torch.Tensor:
    """Upload canonical Q4_0 bytes and repack them on the GPU."""
    wc = to_dev(w_canon.reshape(-1))
    return q.repack_q4_0(wc, rows, cols)


def q8_canonical(x_q8: torch.Tensor, n: int, cols: int) -> np.ndarray:
    """Planar Q8_0 buffer -> canonical 34-byte blocks [n][cols/32][34] (byte moves only)."""
    b = x_q8.cpu().numpy()
    nb = cols // 32
    stride = (nb + 7) // 8 * 8                                    # d_x rows padded to 8 entries
    qv = b[: n * cols].reshape(n, nb, 32)
    dv = b[n * cols: n * cols + 2 * n * stride].reshape(n, stride, 2)[:, :nb]
    return np.concatenate([dv, qv], axis=2)


def unpack_packed(packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """Inverse of the documented packed layout -> canonical Q4_0 [rows][cols/32][18]."""
    nb = cols // 32
    G, C = -(-rows // 64), -(-nb // 8)
    p = packed.reshape(G, C, 9216)
    nib = p[:, :, :8192].reshape(G, C, 8, 64, 16) ^ 0x88          # [g][c][b][r][16]
    sc = p[:, :, 8192:].reshape(G, C, 64, 8, 2)                     # [g][c][r][b][2]
    nib = nib.transpose(0, 3, 1, 2, 4).reshape(G * 64, C * 8, 16)
    sc = sc.transpose(0, 2, 1, 3, 4).reshape(G * 64, C * 8, 2)
    out = np.concatenate([sc, nib], axis=2)
    return np.ascontiguousarray(out[:rows, :nb])


def padding_is_zero(packed: np.ndarray, rows: int, cols: int) -> bool:
    nb = cols // 32
    G, C = -(-rows // 64), -(-nb // 8)
    p = packed.reshape(G, C, 9216)
    nib = p[:, :, :8192].reshape(G, C, 8, 64, 16).transpose(0, 3, 1, 2, 4).reshape(G * 64, C * 8, 16)
    sc = p[:, :, 8192:].reshape(G, C, 64, 8, 2).transpose(0, 2, 1, 3, 4).reshape(G * 64, C * 8, 2)
    pad_rows = (nib[rows:] == 0).all() and (sc[rows:] == 0).all()
    pad_blks = (nib[:, nb:] == 0).all() and (sc[:, nb:] == 0).all()
    return bool(pad_rows and pad_blks)


def assert_within(y_gpu: np.ndarray, y_ref: np.ndarray, S: np.ndarray, rel: float = 1e-5, what: str = ""):
    """|y_gpu - y_ref| <= rel * S elementwise (S = sum_b |d_w d_x s|); S == 0 demands y == 0."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref.astype(np.float64))
    bad = err > rel * S
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} outputs off, first at {tuple(i)}: gpu={y_gpu[tuple(i)]!r} "
                             f"ref={y_ref[tuple(i)]!r} S={S[tuple(i)]!r}")
    return float((err / np.where(S > 0, S, 1)).max()) if err.size else 0.0


def unpack_packed_q8(packed: np.ndarray, rows: int, cols: int):
    """Inverse of the documented packed Q8_0 layout -> (canonical [rows][cols/32][34], padding is zero)."""
    nb = cols // 32
    G, C = -(-rows // 64), -(-nb // 8)
    p = packed.reshape(G, C, 2, 8704)
    qv = p[..., :8192].reshape(G, C, 2, 4, 2, 64, 16)             # [g][c][piece][blk][half][row][16]
    sc = p[..., 8192:].reshape(G, C, 2, 64, 4, 2)                   # [g][c][piece][row][blk][2]
    qv = qv.transpose(0, 5, 1, 2, 3, 4, 6).reshape(G * 64, C * 8, 32)
    sc = sc.transpose(0, 3, 1, 2, 4, 5).reshape(G * 64, C * 8, 2)
    full = np.concatenate([sc, qv], axis=2)
    pad_zero = bool((full[rows:] == 0).all() and (full[:, nb:] == 0).all())
    return np.ascontiguousarray(full[:rows, :nb]), pad_zero
