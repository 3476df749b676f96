"""ctypes binding of libq4stream (include/q4s.h): argument marshalling only.

Every computation runs in the HIP library.  PyTorch supplies device memory and
the current stream; this module only checks tensor placement, passes
``data_ptr()`` values and the stream handle, and turns status codes into
exceptions.  If the library is not built the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libq4stream.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "q4s.h")
MAX_N = 24
MAX_N_Q8 = 8

_lib = None


class Q4SError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn}: {status_string(status)} ({detail})")
        self.status = status


class _Mat(ctypes.Structure):
    _fields_ = [("w_packed", ctypes.c_void_p), ("x", ctypes.c_void_p), ("x_q8", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64)]


class PlanInfo(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int64) for k in
                ("n_mats", "n_tiles", "n_quant_blocks", "fused_quantize", "weight_bytes", "packed_bytes", "act_bytes",
                 "out_bytes", "dev_bytes")]

    def as_dict(self) -> dict:
        return {k: int(getattr(self, k)) for k, _ in self._fields_}


class ChainShape(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32) for k in ("layers", "hidden", "kv_dim", "ff", "vocab")]


class ChainInfo(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int64) for k in
                ("n_mats", "n_phases", "n_tiles", "workgroups", "act_words", "packed_bytes", "dev_bytes", "steps")]

    def as_dict(self) -> dict:
        return {k: int(getattr(self, k)) for k, _ in self._fields_}


CHAIN_COUNTER, CHAIN_TREE, CHAIN_TAGGED = 0, 1, 2
ERR_WAIT = 7


def lib():
    """The loaded library; raises if libq4stream.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m q4_weight_streaming_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        sig = {
            "q4s_abi_version": ([], i32),
            "q4s_status_string": ([i32], ctypes.c_char_p),
            "q4s_last_error": ([], ctypes.c_char_p),
            "q4s_q4_0_bytes": ([i64, i64], sz),
            "q4s_packed_bytes": ([i64, i64], sz),
            "q4s_q8_bytes": ([i32, i64], sz),
            "q4s_repack_q4_0": ([p, p, i64, i64, p], i32),
            "q4s_quantize_q8_0": ([p, p, i32, i64, p], i32),
            "q4s_gemv_q4_0": ([p, p, p, i64, i64, i32, p], i32),
            "q4s_block_sums": ([p, p, p, i64, i64, i32, p], i32),
            "q4s_q8_0_bytes": ([i64, i64], sz),
            "q4s_packed_q8_0_bytes": ([i64, i64], sz),
            "q4s_repack_q8_0": ([p, p, i64, i64, p], i32),
            "q4s_gemv_q8_0": ([p, p, p, i64, i64, i32, p], i32),
            "q4s_gemv_q8_0_f32": ([p, p, p, p, i64, i64, p], i32),
            "q4s_block_sums_q8_0": ([p, p, p, i64, i64, i32, p], i32),
            "q4s_requant_q8_0_to_q4_0": ([p, p, i64, i64, p], i32),
            "q4s_attn_workspace_bytes": ([i32, i64], sz),
            "q4s_attn_decode": ([p, p, p, p, i32, i32, i64, i64, p, sz, p], i32),
            "q4s_attn_decode_noalloc": ([p, p, p, p, i32, i32, i64, i64, p], i32),
            "q4s_sweep_plan_create": ([p, i32, i32, ctypes.POINTER(sz), ctypes.POINTER(p)], i32),
            "q4s_sweep_plan_upload": ([p, p, sz, p], i32),
            "q4s_sweep_run": ([p, p], i32),
            "q4s_sweep_plan_info": ([p, ctypes.POINTER(PlanInfo)], i32),
            "q4s_sweep_plan_destroy": ([p], None),
            "q4s_sweep_trace_bytes": ([p], sz),
            "q4s_sweep_set_trace": ([p, p, sz], i32),
            "q4s_chain_act_words": ([ctypes.POINTER(ChainShape)], i64),
            "q4s_chain_create": ([ctypes.POINTER(ChainShape), p, p, p, p, i32, i32, ctypes.POINTER(sz),
                                  ctypes.POINTER(p)], i32),
            "q4s_chain_upload": ([p, p, sz, p], i32),
            "q4s_chain_run": ([p, p], i32),
            "q4s_chain_check": ([p, p], i32),
            "q4s_chain_get_info": ([p, ctypes.POINTER(ChainInfo)], i32),
            "q4s_chain_destroy": ([p], None),
            "q4s_chain_trace_bytes": ([p], sz),
            "q4s_chain_set_trace": ([p, p, sz], i32),
            "q4s_chain_set_wait_limit": ([p, ctypes.c_uint32], i32),
            "q4s_chain_set_cooperative": ([p, i32], i32),
            "q4s_chain_stage_dump_bytes": ([p], sz),
            "q4s_chain_set_stage_dump": ([p, p, sz], i32),
            "q4s_bench_read": ([p, sz, i32, i32, p, p], i32),
            "q4s_bench_read_units": ([p, sz, sz, p, p], i32),
            "q4s_bench_copy": ([p, p, sz, p], i32),
            "q4s_bench_grid_barrier": ([i32, i32, i32, p, sz, p], i32),
            "q4s_bench_grid_barrier_scratch_bytes": ([i32], sz),
            "q4s_bench_grid_barrier_max_workgroups": ([], i32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        if L.q4s_abi_version() != 4:
            raise RuntimeError("libq4stream ABI version mismatch")
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/q4s.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4s_[a-z0-9_]+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().q4s_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Q4SError(fn, status, lib().q4s_last_error().decode())


def _stream(device: torch.device | None = None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype | None = None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


# ------------------------------------------------------------------ sizes

def q4_0_bytes(rows: int, cols: int) -> int:
    return int(lib().q4s_q4_0_bytes(rows, cols))


def packed_bytes(rows: int, cols: int) -> int:
    return int(lib().q4s_packed_bytes(rows, cols))


def q8_bytes(n: int, cols: int) -> int:
    return int(lib().q4s_q8_bytes(n, cols))


# ------------------------------------------------------------- operations

def repack_q4_0(w_q4_0: torch.Tensor, rows: int, cols: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Canonical Q4_0 bytes (uint8, rows*cols/32*18) -> packed uint8 tensor."""
    if w_q4_0.numel() != q4_0_bytes(rows, cols) or w_q4_0.dtype != torch.uint8:
        raise ValueError("w_q4_0 must be uint8 with rows*cols/32*18 elements")
    if out is None:
        out = torch.empty(packed_bytes(rows, cols), dtype=torch.uint8, device=w_q4_0.device)
    _check("q4s_repack_q4_0", lib().q4s_repack_q4_0(_dev(w_q4_0, "w_q4_0"), _dev(out, "out", torch.uint8),
                                                     rows, cols, _stream(w_q4_0.device)))
    return out


def quantize_q8_0(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 [n][cols] -> planar Q8_0 bytes (uint8, q8_bytes(n, cols))."""
    if x.dim() != 2:
        raise ValueError("x must be [n][cols]")
    n, cols = x.shape
    if out is None:
        out = torch.empty(q8_bytes(n, cols), dtype=torch.uint8, device=x.device)
    _check("q4s_quantize_q8_0", lib().q4s_quantize_q8_0(_dev(x, "x", torch.float32), _dev(out, "out", torch.uint8),
                                                         n, cols, _stream(x.device)))
    return out


def q8_views(x_q8: torch.Tensor, n: int, cols: int):
    """Views of a planar Q8_0 buffer: (q int8 [n][cols], d binary16 bits int16 [n][cols/32])."""
    stride = (cols // 32 + 7) // 8 * 8
    q = x_q8[: n * cols].view(torch.int8).view(n, cols)
    d = x_q8[n * cols: n * cols + 2 * n * stride].view(torch.int16).view(n, stride)[:, : cols // 32]
    return q, d


def gemv_q4_0(w_packed: torch.Tensor, x_q8: torch.Tensor, rows: int, cols: int, n: int,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """y fp32 [n][rows] = Q4_0 W [rows][cols] x Q8_0 activation rows."""
    if out is None:
        out = torch.empty((n, rows), dtype=torch.float32, device=w_packed.device)
    _check("q4s_gemv_q4_0", lib().q4s_gemv_q4_0(_dev(w_packed, "w_packed", torch.uint8),
                                                 _dev(x_q8, "x_q8", torch.uint8),
                                                 _dev(out, "out", torch.float32), rows, cols, n,
                                                 _stream(w_packed.device)))
    return out


def block_sums(w_packed: torch.Tensor, x_q8: torch.Tensor, rows: int, cols: int, n: int) -> torch.Tensor:
    """Per-block integer sums, int32 [n][rows][cols/32]."""
    out = torch.empty((n, rows, cols // 32), dtype=torch.int32, device=w_packed.device)
    _check("q4s_block_sums", lib().q4s_block_sums(_dev(w_packed, "w_packed", torch.uint8),
                                                   _dev(x_q8, "x_q8", torch.uint8),
                                                   _dev(out, "out", torch.int32), rows, cols, n,
                                                   _stream(w_packed.device)))
    return out


# ------------------------------------------------------------ Q8_0 weights

def q8_0_bytes(rows: int, cols: int) -> int:
    return int(lib().q4s_q8_0_bytes(rows, cols))


def packed_q8_0_bytes(rows: int, cols: int) -> int:
    return int(lib().q4s_packed_q8_0_bytes(rows, cols))


def repack_q8_0(w_q8_0: torch.Tensor, rows: int, cols: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Canonical Q8_0 weight bytes (uint8, rows*cols/32*34) -> packed uint8 tensor."""
    if w_q8_0.numel() != q8_0_bytes(rows, cols) or w_q8_0.dtype != torch.uint8:
        raise ValueError("w_q8_0 must be uint8 with rows*cols/32*34 elements")
    if out is None:
        out = torch.empty(packed_q8_0_bytes(rows, cols), dtype=torch.uint8, device=w_q8_0.device)
    _check("q4s_repack_q8_0", lib().q4s_repack_q8_0(_dev(w_q8_0, "w_q8_0"), _dev(out, "out", torch.uint8),
                                                     rows, cols, _stream(w_q8_0.device)))
    return out


def gemv_q8_0(w_packed: torch.Tensor, x_q8: torch.Tensor, rows: int, cols: int, n: int,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """y fp32 [n][rows] = Q8_0 W [rows][cols] x Q8_0 activation rows."""
    if out is None:
        out = torch.empty((n, rows), dtype=torch.float32, device=w_packed.device)
    _check("q4s_gemv_q8_0", lib().q4s_gemv_q8_0(_dev(w_packed, "w_packed", torch.uint8),
                                                 _dev(x_q8, "x_q8", torch.uint8),
                                                 _dev(out, "out", torch.float32), rows, cols, n,
                                                 _stream(w_packed.device)))
    return out


def gemv_q8_0_f32(w_packed: torch.Tensor, x: torch.Tensor, rows: int, cols: int,
                  out: torch.Tensor | None = None, x_q8: torch.Tensor | None = None):
    """1-row Q8_0-weight GEMV from an fp32 activation x [cols] (or [1][cols]): returns (y fp32 [1][rows],
    x_q8, its planar Q8_0 bytes), in one launch when cols <= 2048."""
    if out is None:
        out = torch.empty((1, rows), dtype=torch.float32, device=w_packed.device)
    if x_q8 is None:
        x_q8 = torch.empty(q8_bytes(1, cols), dtype=torch.uint8, device=w_packed.device)
    _check("q4s_gemv_q8_0_f32", lib().q4s_gemv_q8_0_f32(_dev(w_packed, "w_packed", torch.uint8),
                                                         _dev(x, "x", torch.float32),
                                                         _dev(x_q8, "x_q8", torch.uint8),
                                                         _dev(out, "out", torch.float32), rows, cols,
                                                         _stream(w_packed.device)))
    return out, x_q8


def block_sums_q8_0(w_packed: torch.Tensor, x_q8: torch.Tensor, rows: int, cols: int, n: int) -> torch.Tensor:
    """Per-block integer sums of the Q8_0-weight product, int32 [n][rows][cols/32]."""
    out = torch.empty((n, rows, cols // 32), dtype=torch.int32, device=w_packed.device)
    _check("q4s_block_sums_q8_0", lib().q4s_block_sums_q8_0(_dev(w_packed, "w_packed", torch.uint8),
                                                             _dev(x_q8, "x_q8", torch.uint8),
                                                             _dev(out, "out", torch.int32), rows, cols, n,
                                                             _stream(w_packed.device)))
    return out


def requant_q8_0_to_q4_0(w_q8_0: torch.Tensor, rows: int, cols: int,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """Canonical Q8_0 weight bytes -> canonical Q4_0 bytes (uint8, rows*cols/32*18)."""
    if w_q8_0.numel() != q8_0_bytes(rows, cols) or w_q8_0.dtype != torch.uint8:
        raise ValueError("w_q8_0 must be uint8 with rows*cols/32*34 elements")
    if out is None:
        out = torch.empty(q4_0_bytes(rows, cols), dtype=torch.uint8, device=w_q8_0.device)
    _check("q4s_requant_q8_0_to_q4_0",
           lib().q4s_requant_q8_0_to_q4_0(_dev(w_q8_0, "w_q8_0"), _dev(out, "out", torch.uint8), rows, cols,
                                          _stream(w_q8_0.device)))
    return out


# ---------------------------------------------------------------- attention

ATTN_HEAD_DIM = 128


def attn_workspace_bytes(n_q: int, L: int) -> int:
    return int(lib().q4s_attn_workspace_bytes(n_q, L))


def attn_decode(q: torch.Tensor, k_blk: torch.Tensor, v: torch.Tensor, L: int,
                workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention: q fp32 [n_q][128], k_blk fp32 [n_kv][l_cap/64][128][64], v fp32 [n_kv][l_cap][128]."""
    n_q = q.shape[0]
    n_kv, l_cap = v.shape[0], v.shape[1]
    if out is None:
        out = torch.empty((n_q, ATTN_HEAD_DIM), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(16, attn_workspace_bytes(n_q, L)), dtype=torch.uint8, device=q.device)
    _check("q4s_attn_decode", lib().q4s_attn_decode(
        _dev(q, "q", torch.float32), _dev(k_blk, "k_blk", torch.float32), _dev(v, "v", torch.float32),
        _dev(out, "out", torch.float32), n_q, n_kv, L, l_cap, _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(q.device)))
    return out


ATTN_SCRATCH_BYTES = 8 << 20


def attn_decode_noalloc(q: torch.Tensor, k_blk: torch.Tensor, v: torch.Tensor, L: int,
                        out: torch.Tensor) -> torch.Tensor:
    """attn_decode with the split partials in the library's static per-GPU scratch
    (q4s_attn_decode_noalloc): the call allocates nothing; `out` fp32 [n_q][128] is required."""
    n_q = q.shape[0]
    n_kv, l_cap = v.shape[0], v.shape[1]
    _check("q4s_attn_decode_noalloc", lib().q4s_attn_decode_noalloc(
        _dev(q, "q", torch.float32), _dev(k_blk, "k_blk", torch.float32), _dev(v, "v", torch.float32),
        _dev(out, "out", torch.float32), n_q, n_kv, L, l_cap, _stream(q.device)))
    return out


class Sweep:
    """A layer-stack sweep over many matrices with n activation rows each.

    mats: sequence of dicts with keys w_packed, x_q8, y, rows, cols and optional x
    (fp32 [n][cols]; when given, each run quantizes it into x_q8 first).
    """

    def __init__(self, mats, n: int):
        self.n = n
        self._keep = list(mats)            # keep tensors alive as long as the plan
        arr = (_Mat * max(1, len(mats)))()
        for i, m in enumerate(mats):
            x = m.get("x")
            arr[i] = _Mat(_dev(m["w_packed"], "w_packed", torch.uint8) if m["w_packed"].numel() else None,
                          _dev(x, "x", torch.float32) if x is not None else None,
                          _dev(m["x_q8"], "x_q8", torch.uint8) if m["x_q8"].numel() else None,
                          _dev(m["y"], "y", torch.float32) if m["y"].numel() else None,
                          int(m["rows"]), int(m["cols"]))
        need = ctypes.c_size_t(0)
        plan = ctypes.c_void_p(None)
        _check("q4s_sweep_plan_create", lib().q4s_sweep_plan_create(arr, len(mats), n, ctypes.byref(need),
                                                                     ctypes.byref(plan)))
        self._plan = plan
        dev = mats[0]["y"].device if mats else torch.device("cuda")
        self.dev_mem = torch.empty(int(need.value), dtype=torch.uint8, device=dev)
        _check("q4s_sweep_plan_upload", lib().q4s_sweep_plan_upload(self._plan, self.dev_mem.data_ptr(),
                                                                     int(need.value), _stream(dev)))
        torch.cuda.current_stream(dev).synchronize()
        self.device = dev

    def info(self) -> dict:
        inf = PlanInfo()
        _check("q4s_sweep_plan_info", lib().q4s_sweep_plan_info(self._plan, ctypes.byref(inf)))
        return inf.as_dict()

    def run(self) -> None:
        _check("q4s_sweep_run", lib().q4s_sweep_run(self._plan, _stream(self.device)))

    def set_trace(self, on: bool) -> torch.Tensor | None:
        """Record the GEMV launch's timeline in later runs; returns the zeroed int64 tensor
        [n_tiles][9] (word 0: workgroup start, 1 + w: wave w done; 100 MHz clock)."""
        if not on:
            _check("q4s_sweep_set_trace", lib().q4s_sweep_set_trace(self._plan, None, 0))
            self._trace = None
            return None
        n = int(lib().q4s_sweep_trace_bytes(self._plan)) // 8
        self._trace = torch.zeros(max(n, 1), dtype=torch.int64, device=self.device)
        _check("q4s_sweep_set_trace", lib().q4s_sweep_set_trace(self._plan, self._trace.data_ptr(), n * 8))
        return self._trace

    def close(self) -> None:
        if self._plan:
            lib().q4s_sweep_plan_destroy(self._plan)
            self._plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def chain_act_words(layers: int, hidden: int, kv_dim: int, ff: int, vocab: int) -> int:
    return int(lib().q4s_chain_act_words(ctypes.byref(ChainShape(layers, hidden, kv_dim, ff, vocab))))


def chain_layout(hidden: int, kv_dim: int, ff: int):
    """Offsets (in words) of q, k, v, o, h1, g, u, dn, h2 within one layer of the activation buffer."""
    E, D, F = hidden, kv_dim, ff
    sizes = [("q", E), ("k", D), ("v", D), ("o", E), ("h1", E), ("g", F), ("u", F), ("dn", E), ("h2", E)]
    out, off = {}, 0
    for name, n in sizes:
        out[name] = (off, n)
        off += n
    return out, off


def chain_values(acts: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Split tagged activation words (int64) into (fp32 values, int64 tags)."""
    halves = acts.contiguous().view(torch.int32).view(-1, 2)   # little-endian: [low, high]
    return halves[:, 0].contiguous().view(torch.float32), halves[:, 1].to(torch.int64) & 0xFFFFFFFF


class Chain:
    """One chained decode step (see q4s_chain_create): w_packed is the list of 7*layers + 1
    packed matrices; h0 fp32 [hidden]; acts int64 [chain_act_words]; logits fp32 [vocab]."""

    def __init__(self, layers: int, hidden: int, kv_dim: int, ff: int, vocab: int, w_packed, h0: torch.Tensor,
                 acts: torch.Tensor, logits: torch.Tensor, sync_mode: int = CHAIN_TAGGED, workgroups: int = 0):
        self.shape = ChainShape(layers, hidden, kv_dim, ff, vocab)
        self._keep = (list(w_packed), h0, acts, logits)
        ws = (ctypes.c_void_p * len(w_packed))(*[_dev(w, "w_packed", torch.uint8) for w in w_packed])
        need = ctypes.c_size_t(0)
        handle = ctypes.c_void_p(None)
        _check("q4s_chain_create", lib().q4s_chain_create(
            ctypes.byref(self.shape), ws, _dev(h0, "h0", torch.float32), _dev(acts, "acts", torch.int64),
            _dev(logits, "logits", torch.float32), sync_mode, workgroups, ctypes.byref(need), ctypes.byref(handle)))
        self._chain = handle
        self.device = h0.device
        self.dev_mem = torch.empty(int(need.value), dtype=torch.uint8, device=self.device)
        _check("q4s_chain_upload", lib().q4s_chain_upload(self._chain, self.dev_mem.data_ptr(), int(need.value),
                                                          _stream(self.device)))
        torch.cuda.current_stream(self.device).synchronize()

    def info(self) -> dict:
        inf = ChainInfo()
        _check("q4s_chain_get_info", lib().q4s_chain_get_info(self._chain, ctypes.byref(inf)))
        return inf.as_dict()

    def run(self) -> None:
        _check("q4s_chain_run", lib().q4s_chain_run(self._chain, _stream(self.device)))

    def set_trace(self, on: bool) -> torch.Tensor | None:
        """Record the phase timeline of later steps; returns the zeroed int64 trace tensor
        (layout in q4s.h: phase ends [P][W], workgroup starts [W], first-tile starts [P][W],
        first-tile prologue ends [P][W]; 100 MHz clock)."""
        if not on:
            _check("q4s_chain_set_trace", lib().q4s_chain_set_trace(self._chain, None, 0))
            self._trace = None
            return None
        n = int(lib().q4s_chain_trace_bytes(self._chain)) // 8
        self._trace = torch.zeros(n, dtype=torch.int64, device=self.device)
        _check("q4s_chain_set_trace", lib().q4s_chain_set_trace(self._chain, self._trace.data_ptr(), n * 8))
        return self._trace

    def set_stage_dump(self, on: bool) -> torch.Tensor | None:
        """Test hook: record the staged Q8_0 input of every phase of later steps; returns the
        int64 dump tensor [n_phases][C][64] (code dword | d_x fp32 bits << 32, see q4s.h)."""
        if not on:
            _check("q4s_chain_set_stage_dump", lib().q4s_chain_set_stage_dump(self._chain, None, 0))
            self._dump = None
            return None
        nbytes = int(lib().q4s_chain_stage_dump_bytes(self._chain))
        self._dump = torch.zeros(nbytes // 8, dtype=torch.int64, device=self.device)
        _check("q4s_chain_set_stage_dump", lib().q4s_chain_set_stage_dump(self._chain, self._dump.data_ptr(), nbytes))
        return self._dump

    def set_wait_limit(self, polls: int) -> None:
        _check("q4s_chain_set_wait_limit", lib().q4s_chain_set_wait_limit(self._chain, polls))

    def set_cooperative(self, on: bool) -> None:
        _check("q4s_chain_set_cooperative", lib().q4s_chain_set_cooperative(self._chain, 1 if on else 0))

    def check(self) -> None:
        """Synchronize; raise Q4SError (status 7) if a bounded wait of the last step gave up."""
        _check("q4s_chain_check", lib().q4s_chain_check(self._chain, _stream(self.device)))

    def close(self) -> None:
        if self._chain:
            lib().q4s_chain_destroy(self._chain)
            self._chain = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ----------------------------------------------------------- measurement

def bench_read(buf: torch.Tensor, loads_in_flight: int = 4, n_blocks: int = 0,
               sink: torch.Tensor | None = None) -> None:
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check("q4s_bench_read", lib().q4s_bench_read(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                                   loads_in_flight, n_blocks, _dev(sink, "sink"),
                                                   _stream(buf.device)))


def bench_read_units(buf: torch.Tensor, unit_bytes: int, sink: torch.Tensor | None = None) -> None:
    """Read buf's whole units of unit_bytes (a multiple of 1024), one wave per unit."""
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check("q4s_bench_read_units", lib().q4s_bench_read_units(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                                               unit_bytes, _dev(sink, "sink"), _stream(buf.device)))


def bench_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    _check("q4s_bench_copy", lib().q4s_bench_copy(_dev(src, "src"), _dev(dst, "dst"), nbytes,
                                                   _stream(src.device)))


def bench_grid_barrier(kind: int, n_workgroups: int, phases: int, scratch: torch.Tensor) -> None:
    """Launch a grid-barrier measurement kernel (kind 0: atomic counter, 1: per-workgroup flags)."""
    _check("q4s_bench_grid_barrier", lib().q4s_bench_grid_barrier(
        kind, n_workgroups, phases, _dev(scratch, "scratch"), scratch.numel() * scratch.element_size(),
        _stream(scratch.device)))


def grid_barrier_scratch_bytes(n_workgroups: int) -> int:
    return int(lib().q4s_bench_grid_barrier_scratch_bytes(n_workgroups))


def grid_barrier_max_workgroups() -> int:
    return int(lib().q4s_bench_grid_barrier_max_workgroups())
