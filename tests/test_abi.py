"""The C-ABI library: it loads, exports every function include/q4s.h declares,
and rejects bad arguments before touching the GPU (no device needed here)."""
import ctypes

import pytest

from q4_weight_streaming_amd import _lib as q

FAKE = 0x7F0000000000  # a 256-byte aligned address that is never dereferenced on these paths


@pytest.fixture(scope="module")
def L():
    return q.lib()


def test_exports_every_declared_function(L):
    names = q.header_functions()
    assert len(names) >= 23
    for n in names:
        assert hasattr(L, n), n
    assert L.q4s_abi_version() == 4


def test_status_strings(L):
    for s in range(8):
        assert q.status_string(s) != "unknown status"
    assert q.status_string(99) == "unknown status"


def test_sizes():
    assert q.q4_0_bytes(151936, 1536) == 131_272_704
    assert q.packed_bytes(1536, 1536) == 1_327_104          # no padding at config shapes
    assert q.packed_bytes(151936, 1536) == 131_272_704
    assert q.packed_bytes(1536, 8960) == 1536 * 280 * 18
    assert q.packed_bytes(65, 288) == 2 * 2 * 9216         # 2 groups x 2 chunks, padded
    assert q.packed_bytes(1, 32) == 9216
    assert q.packed_bytes(0, 1536) == 0 and q.packed_bytes(10, 0) == 0
    assert q.q8_bytes(1, 1536) == 1632                     # dense Q8_0 at cols % 256 == 0
    assert q.q8_bytes(8, 8960) == 8 * 8960 * 34 // 32
    assert q.q8_bytes(1, 32) == 32 + 16                    # d_x row padded to 8 entries
    assert q.q8_bytes(3, 288) == 3 * 288 + 3 * 16 * 2
    assert q.packed_bytes(3, 33) == 0 and q.q8_bytes(25, 32) == 0 and q.q4_0_bytes(-1, 32) == 0
    assert q.q8_bytes(24, 1536) == 24 * 1536 * 34 // 32
    # Q8_0 weights: the 8-bit lm_head of milestone M14 is 248 MB at 151936 x 1536
    assert q.q8_0_bytes(151936, 1536) == 247_959_552
    assert q.packed_q8_0_bytes(151936, 1536) == 247_959_552   # no padding at config shapes
    assert q.packed_q8_0_bytes(65, 288) == 2 * 2 * 17408
    assert q.packed_q8_0_bytes(1, 32) == 17408
    assert q.packed_q8_0_bytes(0, 64) == 0 and q.q8_0_bytes(3, 33) == 0


def _err(L):
    return L.q4s_last_error().decode()


def test_gemv_validation(L):
    g = L.q4s_gemv_q4_0
    assert g(FAKE, FAKE, FAKE + (1 << 30), 64, 33, 1, None) == 2        # cols % 32
    assert "cols" in _err(L)
    assert g(FAKE, FAKE, FAKE + (1 << 30), 64, 64, 25, None) == 2       # n > 24
    assert g(FAKE, FAKE, FAKE + (1 << 30), -1, 64, 1, None) == 2
    assert g(None, FAKE, FAKE + (1 << 30), 64, 64, 1, None) == 1        # null weights
    assert g(FAKE + 8, FAKE, FAKE + (1 << 30), 64, 64, 1, None) == 3    # misaligned
    assert g(FAKE, FAKE + 4, FAKE + (1 << 30), 64, 64, 1, None) == 3
    assert g(FAKE, FAKE + (1 << 20), FAKE + 64, 64, 64, 1, None) == 4   # y inside w
    assert "overlap" in _err(L)
    assert g(None, None, None, 0, 64, 1, None) == 0                     # rows == 0: no-op
    assert g(None, None, None, 64, 64, 0, None) == 0                    # n == 0: no-op
    assert _err(L) == ""


def test_other_entry_points_validate(L):
    assert L.q4s_repack_q4_0(FAKE + 1, FAKE + (1 << 30), 64, 64, None) == 3   # 2-byte alignment
    assert L.q4s_repack_q4_0(FAKE, FAKE, 64, 64, None) == 4                     # in place
    assert L.q4s_repack_q4_0(None, None, 0, 64, None) == 0
    assert L.q4s_quantize_q8_0(FAKE, FAKE + 8, 1, 64, None) == 3
    assert L.q4s_quantize_q8_0(FAKE, FAKE, 1, 64, None) == 4
    assert L.q4s_quantize_q8_0(None, FAKE, 1, 64, None) == 1
    assert L.q4s_quantize_q8_0(FAKE + 4, FAKE + (1 << 30), 1, 64, None) == 3   # x needs 16 bytes
    assert L.q4s_quantize_q8_0(FAKE, FAKE + (1 << 30), 1, 48, None) == 2
    assert L.q4s_block_sums(FAKE, FAKE + (1 << 28), FAKE + 2, 64, 64, 1, None) == 3
    assert L.q4s_bench_read(FAKE, 24, 4, 0, FAKE + (1 << 30), None) == 2
    assert L.q4s_bench_read(FAKE, 32, 3, 0, FAKE + (1 << 30), None) == 2
    assert L.q4s_bench_copy(FAKE, FAKE + 16, 64, None) == 4
    assert L.q4s_bench_read_units(FAKE, 1 << 20, 1000, FAKE + (1 << 30), None) == 2   # unit not a multiple of 1 KB
    assert L.q4s_bench_read_units(FAKE, 1 << 20, 0, FAKE + (1 << 30), None) == 2
    assert L.q4s_bench_read_units(FAKE + 4, 1 << 20, 9216, FAKE + (1 << 30), None) == 3
    assert L.q4s_bench_read_units(None, 0, 9216, None, None) == 0                      # nothing to read
    assert L.q4s_sweep_run(None, None) == 1
    assert L.q4s_bench_grid_barrier(0, 4, 0, FAKE, 1 << 20, None) == 2      # phases >= 1
    assert L.q4s_bench_grid_barrier(10, 4, 10, FAKE, 1 << 20, None) == 2     # unknown kind
    assert q.grid_barrier_scratch_bytes(4) == (64 + 16 * 16384) * 4
    # Q8_0 weights
    g = L.q4s_gemv_q8_0
    assert g(FAKE, FAKE, FAKE + (1 << 30), 64, 33, 1, None) == 2
    assert g(FAKE, FAKE, FAKE + (1 << 30), 64, 64, 9, None) == 2        # n > 8 for Q8_0 weights
    assert g(FAKE + 8, FAKE, FAKE + (1 << 30), 64, 64, 1, None) == 3
    assert g(FAKE, FAKE + (1 << 20), FAKE + 17408 - 4, 64, 64, 1, None) == 4   # y overlaps packed Q8_0
    assert g(None, None, None, 0, 64, 1, None) == 0
    assert L.q4s_repack_q8_0(FAKE + 1, FAKE + (1 << 30), 64, 64, None) == 3
    assert L.q4s_repack_q8_0(FAKE, FAKE, 64, 64, None) == 4
    assert L.q4s_block_sums_q8_0(FAKE, FAKE + (1 << 28), FAKE + 2, 64, 64, 1, None) == 3
    assert L.q4s_requant_q8_0_to_q4_0(FAKE, FAKE + 1, 64, 64, None) == 3
    # Q8_0 weights from an fp32 activation (quantized in the launch)
    f = L.q4s_gemv_q8_0_f32
    W, X, XQ, Y = FAKE, FAKE + (1 << 24), FAKE + (1 << 26), FAKE + (1 << 28)
    assert f(W, X, XQ, Y, 64, 33, None) == 2                             # cols % 32
    assert f(W, X + 4, XQ, Y, 64, 64, None) == 3                         # x needs 16 bytes
    assert f(W, X, XQ + 8, Y, 64, 64, None) == 3                         # x_q8 needs 16 bytes
    assert f(W, None, XQ, Y, 64, 64, None) == 1
    assert f(W, X, XQ, X + 64, 64, 64, None) == 4                        # y overlaps x
    assert f(W, X, W + 16, Y, 64, 64, None) == 4                         # x_q8 overlaps w_packed
    assert f(W, XQ, XQ, Y, 64, 64, None) == 4                            # x overlaps x_q8
    assert f(None, None, None, None, 0, 64, None) == 0
    assert L.q4s_requant_q8_0_to_q4_0(FAKE, FAKE + 64, 64, 64, None) == 4
    assert L.q4s_requant_q8_0_to_q4_0(None, FAKE, 64, 64, None) == 1
    assert L.q4s_requant_q8_0_to_q4_0(None, None, 0, 64, None) == 0
    # decode attention
    a = L.q4s_attn_decode
    W = q.attn_workspace_bytes(12, 100)
    assert W == 2 * 12 * 130 * 4 and q.attn_workspace_bytes(12, 0) == 0
    assert q.attn_workspace_bytes(3, 64) == 392 * 4                    # 3*130 rounded up to 4 floats
    ok = (FAKE, FAKE + (1 << 24), FAKE + (1 << 26), FAKE + (1 << 28), 12, 2, 100, 128, FAKE + (1 << 29), W, None)
    assert a(*ok[:7], 130, *ok[8:]) == 2                                # l_cap not a multiple of 64
    assert a(*ok[:4], 12, 5, *ok[6:]) == 2                              # 5 does not divide 12
    assert a(*ok[:4], 18, 2, *ok[6:]) == 2                              # group of 9
    assert a(*ok[:6], 129, 128, *ok[8:]) == 2                           # L > l_cap
    assert a(FAKE, FAKE + (1 << 24) + 4, *ok[2:]) == 3                  # k_blk needs 16 bytes
    assert a(*ok[:6], 0, 128, *ok[8:]) == 2
    assert a(*ok[:9], W - 4, None) == 2                                 # workspace too small
    assert a(FAKE + 4, *ok[1:]) == 3                                    # q needs 16 bytes
    assert a(*ok[:3], FAKE, *ok[4:]) == 4                               # o overlaps q
    assert a(*ok[:8], FAKE + (1 << 28) + 64, W, None) == 4              # workspace overlaps o
    # the allocation-free variant: the same checks, and its scratch limit, all before any HIP call
    nz = L.q4s_attn_decode_noalloc
    assert nz(*ok[:6], 129, 128, None) == 2                              # L > l_cap
    assert nz(FAKE + 4, *ok[1:8], None) == 3                             # q needs 16 bytes
    assert nz(*ok[:3], FAKE, *ok[4:8], None) == 4                        # o overlaps q
    big = 86016 + 64                                                     # one split past 8 MiB at 12 heads
    assert q.attn_workspace_bytes(12, big) > q.ATTN_SCRATCH_BYTES >= q.attn_workspace_bytes(12, big - 64)
    assert nz(*ok[:6], big, big, None) == 2
    assert "static scratch" in _err(L)


def _plan(L, mats, n):
    arr = (q._Mat * len(mats))(*[q._Mat(*m) for m in mats])
    need = ctypes.c_size_t(0)
    plan = ctypes.c_void_p(None)
    st = L.q4s_sweep_plan_create(arr, len(mats), n, ctypes.byref(need), ctypes.byref(plan))
    return st, plan, need.value


def test_sweep_plan_host_side(L):
    from q4_weight_streaming_amd import synth
    shapes = synth.qwen25_1p5b()
    mats, base = [], FAKE
    for s in shapes:                                      # disjoint fake regions per buffer
        w = base; base += (q.packed_bytes(s.rows, s.cols) + 4095) // 4096 * 4096
        x = base; base += (q.q8_bytes(1, s.cols) + 4095) // 4096 * 4096
        y = base; base += (4 * s.rows + 4095) // 4096 * 4096
        mats.append((w, None, x, y, s.rows, s.cols))
    st, plan, need = _plan(L, mats, 1)
    assert st == 0, _err(L)
    info = q.PlanInfo()
    assert L.q4s_sweep_plan_info(plan, ctypes.byref(info)) == 0
    d = info.as_dict()
    assert d["n_mats"] == 197
    assert d["weight_bytes"] == 868_257_792 == d["packed_bytes"]
    # at n = 1 a single-split matrix (at most 8 chunks) has one tile per row group: q,o 24; k,v 4;
    # gate,up 140; down 24 group sets of one row group (4-way K split) per layer; lm_head 2374
    assert d["n_tiles"] == 28 * (24 + 4 + 4 + 24 + 140 + 140 + 24) + 2374
    assert d["n_quant_blocks"] == 0 and d["dev_bytes"] == need and d["fused_quantize"] == 0
    assert d["out_bytes"] == 4 * sum(s.rows for s in shapes)
    L.q4s_sweep_plan_destroy(plan)
    # at n = 2 every tile is a group set: q,o 6; k,v 1; gate,up 35; down 24 per layer; lm_head 594
    mats2, base2 = [], base
    for s in shapes:
        w = base2; base2 += (q.packed_bytes(s.rows, s.cols) + 4095) // 4096 * 4096
        x = base2; base2 += (q.q8_bytes(2, s.cols) + 4095) // 4096 * 4096
        y = base2; base2 += (8 * s.rows + 4095) // 4096 * 4096
        mats2.append((w, None, x, y, s.rows, s.cols))
    st, plan, _ = _plan(L, mats2, 2)
    assert st == 0, _err(L)
    assert L.q4s_sweep_plan_info(plan, ctypes.byref(info)) == 0
    assert info.n_tiles == 28 * (6 + 1 + 1 + 6 + 35 + 35 + 24) + 594
    L.q4s_sweep_plan_destroy(plan)
    # with fp32 activations at n = 1 the plan quantizes inside the GEMV launch
    fx = base
    mats_x = []
    for (w, _, x, y, rows, cols) in mats:
        mats_x.append((w, fx, x, y, rows, cols))
        fx += (4 * cols + 4095) // 4096 * 4096
    st, plan, _ = _plan(L, mats_x, 1)
    assert st == 0, _err(L)
    assert L.q4s_sweep_plan_info(plan, ctypes.byref(info)) == 0
    assert info.fused_quantize == 1 and info.n_quant_blocks == sum(s.cols // 32 for s in shapes)
    L.q4s_sweep_plan_destroy(plan)
    # an output aliasing another matrix's input is rejected
    bad = list(mats)
    bad[1] = (mats[1][0], None, mats[1][2], mats[0][0], mats[1][4], mats[1][5])
    st, plan, _ = _plan(L, bad, 1)
    assert st == 4 and not plan.value
    st, plan, _ = _plan(L, mats[:3], 25)
    assert st == 2
    st, plan, _ = _plan(L, [(FAKE, None, FAKE + 8, FAKE + (1 << 30), 64, 64)], 1)
    assert st == 3 and "matrix 0" in _err(L)


def _chain(L, shape, ws, h0, acts, logits, mode=2, wg=0):
    arr = (ctypes.c_void_p * max(1, len(ws)))(*ws)
    need = ctypes.c_size_t(0)
    h = ctypes.c_void_p(None)
    st = L.q4s_chain_create(ctypes.byref(shape), arr, h0, acts, logits, mode, wg, ctypes.byref(need),
                            ctypes.byref(h))
    return st, h, need.value


def test_chain_host_side(L):
    """Plan building and validation of the chained step (no GPU: upload is not called)."""
    Lr, E, D, F, V = 28, 1536, 256, 8960, 151936
    shape = q.ChainShape(Lr, E, D, F, V)
    assert L.q4s_chain_act_words(ctypes.byref(shape)) == 28 * (5 * 1536 + 2 * 256 + 2 * 8960)
    assert q.chain_layout(E, D, F)[1] == 5 * 1536 + 2 * 256 + 2 * 8960
    dims = [(E, E), (D, E), (D, E), (E, E), (F, E), (F, E), (E, F)] * Lr + [(V, E)]
    ws, base = [], FAKE
    for r, c in dims:
        ws.append(base)
        base += (q.packed_bytes(r, c) + 4095) // 4096 * 4096
    h0 = base; base += 1 << 16
    acts = base; base += (8 * L.q4s_chain_act_words(ctypes.byref(shape)) + 4095) // 4096 * 4096
    logits = base
    st, h, need = _chain(L, shape, ws, h0, acts, logits)
    assert st == 0, _err(L)
    info = q.ChainInfo()
    assert L.q4s_chain_get_info(h, ctypes.byref(info)) == 0
    d = info.as_dict()
    assert d["n_mats"] == 197 and d["n_phases"] == 113 and d["workgroups"] == 0 and d["steps"] == 0
    assert d["packed_bytes"] == 868_257_792 and d["dev_bytes"] == need
    # laid out for 256 workgroups: q/k/v (32 row groups) and o (24): one row group per tile;
    # gate + up (280 groups): two per tile (140); down (four K splits of <= 16 chunks, tagged
    # phases): one tile per K range and row group (96); the head (2374 groups): group sets of 4 (594)
    assert d["n_tiles"] == 28 * (32 + 24 + 140 + 96) + 594
    assert L.q4s_chain_run(h, None) == 5                  # not uploaded
    L.q4s_chain_destroy(h)
    # for 64 workgroups gate + up fall back to group sets of 4; the device image does not change
    st, h, need64 = _chain(L, shape, ws, h0, acts, logits, wg=64)
    assert st == 0 and need64 == need
    assert L.q4s_chain_get_info(h, ctypes.byref(info)) == 0
    assert info.n_tiles == 28 * (32 + 24 + 70 + 96) + 594
    L.q4s_chain_destroy(h)
    # with barriers between phases down keeps one tile per row group (its four K ranges on 4 waves)
    st, h, _ = _chain(L, shape, ws, h0, acts, logits, mode=q.CHAIN_TREE)
    assert st == 0 and L.q4s_chain_get_info(h, ctypes.byref(info)) == 0
    assert info.n_tiles == 28 * (32 + 24 + 140 + 24) + 594
    L.q4s_chain_destroy(h)
    # bad shapes, modes, counts, pointers and aliasing
    for bad in (q.ChainShape(2, 100, 64, 256, 10), q.ChainShape(2, 128, 0, 256, 10),
                q.ChainShape(2, 128, 64, 250, 10), q.ChainShape(-1, 128, 64, 256, 10),
                q.ChainShape(2, 128, 64, 256, 0), q.ChainShape(2, 32800, 64, 256, 10),
                q.ChainShape(2, 128, 64, 32800, 10)):
        assert L.q4s_chain_act_words(ctypes.byref(bad)) == 0
        assert _chain(L, bad, ws, h0, acts, logits)[0] == 2
    assert _chain(L, shape, ws, h0, acts, logits, mode=3)[0] == 2
    assert _chain(L, shape, ws, h0, acts, logits, wg=-1)[0] == 2
    assert _chain(L, shape, ws, h0 + 4, acts, logits)[0] == 3          # h0 not 16-byte aligned
    assert _chain(L, shape, ws, h0, acts + 8, logits)[0] == 3
    assert _chain(L, shape, ws, None, acts, logits)[0] == 1
    wbad = list(ws)
    wbad[5] = None
    st, _, _ = _chain(L, shape, wbad, h0, acts, logits)
    assert st == 1 and "matrix 5" in _err(L)
    assert _chain(L, shape, ws, h0, ws[3], logits)[0] == 4             # acts over a weight
    assert _chain(L, shape, ws, h0, acts, h0)[0] == 4                  # logits over h0
    assert _chain(L, shape, ws, h0, acts, acts + 64)[0] == 4           # logits inside acts
    # the head alone
    one = q.ChainShape(0, 128, 64, 64, 200)
    st, h, _ = _chain(L, one, [FAKE], FAKE + (1 << 20), FAKE + (1 << 21), FAKE + (1 << 22))
    assert st == 0, _err(L)
    assert L.q4s_chain_get_info(h, ctypes.byref(info)) == 0 and info.n_phases == 1 and info.act_words == 0
    L.q4s_chain_destroy(h)


def test_library_refuses_when_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(q, "_lib", None)
    monkeypatch.setattr(q, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        q.lib()
