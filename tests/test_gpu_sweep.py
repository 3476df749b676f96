"""GPU parity of the layer-stack sweep at the full workload sizes, in the same
launch configuration the benchmark times (one plan, quantize + GEMV launches).

  * Qwen2.5-1.5B-shaped set (197 matrices, 868 MB), N=1: every output against
    the oracle; the sweep equals the standalone GEMV bit for bit.
  * the same set at N=8 (multi-token verify) and N=24: every output against the
    oracle, and each row equals the N=1 sweep of that activation bit for bit.
  * lm_head alone (151936 x 1536): every output against the oracle.
  * Qwen2.5-7B-shaped set (3.98 GB), N=1 and N=8: every output against the oracle.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import assert_within, dev, packed_weights, q8_canonical, require_gpu, to_dev
from q4_weight_streaming_amd import _lib as q
from q4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu


def _stack(cfg, shapes, n, act_cfg=None, keep_host=True):
    """Generate, upload and repack a weight stack; returns host weights, device tensors."""
    host_w, host_x, mats = [], [], []
    for m, s in enumerate(shapes):
        w = synth.q4_0_weights(s.rows, s.cols, synth.generator(cfg, m, 0, 0))
        x = synth.activation(n, s.cols, synth.generator(cfg if act_cfg is None else act_cfg, m, 0, 1))
        wp = packed_weights(w, s.rows, s.cols)
        mats.append({"w_packed": wp, "x": to_dev(x),
                     "x_q8": torch.empty(q.q8_bytes(n, s.cols), dtype=torch.uint8, device=dev()),
                     "y": torch.empty((n, s.rows), dtype=torch.float32, device=dev()),
                     "rows": s.rows, "cols": s.cols})
        if keep_host:
            host_w.append(w)
        host_x.append(x)
    torch.cuda.synchronize()
    return host_w, host_x, mats


@pytest.fixture(scope="module")
def qwen15():
    require_gpu()
    return _stack(1, synth.qwen25_1p5b(), 1)


def test_sweep_small_mixed_equals_standalone(oracle):
    require_gpu()
    shapes = [synth.MatShape("a", 257, 1536), synth.MatShape("b", 64, 8960), synth.MatShape("c", 1, 32),
              synth.MatShape("d", 130, 4128), synth.MatShape("e", 0, 64), synth.MatShape("f", 90, 0)]
    for n in (1, 4, 8, 16, 24):
        _, hx, mats = _stack(77, shapes, n)
        sw = q.Sweep(mats, n)
        sw.run()
        torch.cuda.synchronize()
        for m, x in zip(mats, hx):
            xq = q.quantize_q8_0(to_dev(x))
            used = n * m["cols"]                              # q; d_x compared below without padding
            assert torch.equal(q.q8_views(xq, n, m["cols"])[1], q.q8_views(m["x_q8"], n, m["cols"])[1])
            assert torch.equal(xq[:used], m["x_q8"][:used])
            y = q.gemv_q4_0(m["w_packed"], xq, m["rows"], m["cols"], n)
            assert torch.equal(y, m["y"])
        assert (mats[5]["y"] == 0).all()


def test_sweep_fused_quantize_equals_two_launches(oracle):
    # n = 1 with every activation given as fp32: one launch whose waves quantize
    # the chunks they stream; x_q8 and y equal the separate quantize + GEMV bit
    # for bit (rows over 32768 columns and padded d_x rows included)
    require_gpu()
    shapes = [synth.MatShape("a", 257, 1536), synth.MatShape("b", 64, 8960), synth.MatShape("c", 1, 32),
              synth.MatShape("d", 130, 4128), synth.MatShape("e", 90, 96), synth.MatShape("f", 70, 18944),
              synth.MatShape("g", 3, 33792), synth.MatShape("h", 200, 3072)]
    _, hx, mats = _stack(78, shapes, 1)
    for m in mats:
        m["x_q8"].fill_(0xA5)                                # every byte must be written
    sw = q.Sweep(mats, 1)
    info = sw.info()
    assert info["fused_quantize"] == 1
    assert info["n_quant_blocks"] == sum(s.cols // 32 for s in shapes)
    sw.run()
    torch.cuda.synchronize()
    for m, x in zip(mats, hx):
        xq = q.quantize_q8_0(to_dev(x))
        assert torch.equal(xq, m["x_q8"])                    # q, d_x and the zeroed padding
        assert np.array_equal(q.q8_views(xq, 1, m["cols"])[0].cpu().numpy().view(np.uint8).reshape(-1),
                              oracle.quantize_q8_0(x)[0, :, 2:].reshape(-1))
        y = q.gemv_q4_0(m["w_packed"], xq, m["rows"], m["cols"], 1)
        assert torch.equal(y, m["y"])


MANY_ROW_SHAPES = [synth.MatShape("a", 257, 1536), synth.MatShape("b", 64, 8960), synth.MatShape("c", 1, 32),
                   synth.MatShape("d", 130, 4128), synth.MatShape("e", 90, 96), synth.MatShape("f", 70, 18944),
                   synth.MatShape("g", 3, 33792), synth.MatShape("h", 200, 3072), synth.MatShape("i", 65, 2080)]


def _new_activations(mats, n, cfg):
    """Overwrite every x with a fresh seeded activation; returns the host copies."""
    hx = []
    for i, m in enumerate(mats):
        x = synth.activation(n, m["cols"], synth.generator(cfg, i, 0, 1))
        m["x"].copy_(to_dev(x))
        hx.append(x)
    torch.cuda.synchronize()
    return hx


def _check_standalone(mats, hx, n, names):
    for m, x, name in zip(mats, hx, names):
        xq = q.quantize_q8_0(to_dev(x))
        assert torch.equal(xq, m["x_q8"]), name                # q, d_x and the zeroed padding
        y = q.gemv_q4_0(m["w_packed"], xq, m["rows"], m["cols"], n)
        assert torch.equal(y, m["y"]), name


@pytest.mark.parametrize("n", [2, 3, 5, 8])
def test_sweep_many_rows_equals_standalone(oracle, n):
    # 2..8 rows with every activation given as fp32: a quantize launch, then one GEMV launch
    # over all matrices; x_q8 and y equal the standalone quantize + GEMV bit for bit -- one,
    # two and four K splits, partial chunks and row groups, segments past 16 chunks, padded
    # d_x rows -- and the Q8_0 bytes equal the oracle's; three steps over fresh activations
    # (a GEMV that read the previous step's codes would differ)
    require_gpu()
    shapes = MANY_ROW_SHAPES
    hw, hx, mats = _stack(81 + n, shapes, n)
    for m in mats:
        m["x_q8"].fill_(0xA5)                                # every byte must be written
        m["y"].fill_(float("nan"))
    sw = q.Sweep(mats, n)
    info = sw.info()
    assert info["fused_quantize"] == 0
    assert info["n_quant_blocks"] == n * sum(s.cols // 32 for s in shapes)
    sw.run()
    torch.cuda.synchronize()
    for m, x, sh in zip(mats, hx, shapes):
        assert np.array_equal(q8_canonical(m["x_q8"], n, m["cols"]), oracle.quantize_q8_0(x)), sh.name
    _check_standalone(mats, hx, n, [s.name for s in shapes])
    for i in (0, 3, 8):                                       # and against the fp64 oracle
        y_ref, S = oracle.gemv(hw[i], oracle.quantize_q8_0(hx[i]), shapes[i].rows, shapes[i].cols, n)
        assert_within(mats[i]["y"].cpu().numpy(), y_ref, S, what=shapes[i].name)
    for step in (1, 2):
        hx = _new_activations(mats, n, 181 + 10 * step + n)
        sw.run()
        torch.cuda.synchronize()
        _check_standalone(mats, hx, n, [f"{s.name} step {step}" for s in shapes])


def test_sweep_many_rows_graph_replay():
    # the 8-row sweep (quantize launch + GEMV launch) captured in a graph: each replay, with
    # eager activation updates and synchronizations between replays, equals the standalone
    # quantize + GEMV bit for bit, and an eager step in between stays exact
    require_gpu()
    n = 8
    shapes = MANY_ROW_SHAPES[:6]
    _, hx, mats = _stack(95, shapes, n, keep_host=False)
    sw = q.Sweep(mats, n)
    sw.run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw.run()
    torch.cuda.synchronize()
    for r in range(4):
        hx = _new_activations(mats, n, 400 + r)
        for m in mats:
            m["y"].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _check_standalone(mats, hx, n, [f"{s.name} replay {r}" for s in shapes])
        if r == 1:
            hx = _new_activations(mats, n, 410)
            sw.run()
            torch.cuda.synchronize()
            _check_standalone(mats, hx, n, [f"{s.name} eager" for s in shapes])


def _adversarial_blocks(rng, nblk):
    """Q8_0 blocks whose maxima span the quantizer's division-free range and its guards, with
    near-ties (k + 1/2) d nudged by an ulp either way, all-zero blocks and the maximum anywhere."""
    f32 = np.float32
    amax = (f32(2.0) ** rng.uniform(-100, 22, nblk).astype(np.float32)).astype(np.float32)
    amax[::7] = f32(127 * 2.0 ** -125)
    amax[3::11] = f32(7.9e6)
    d = (amax / f32(127)).astype(np.float32)
    k = rng.integers(-126, 126, size=(nblk, 23)).astype(np.float32)
    ties = ((k + f32(0.5)) * d[:, None]).astype(np.float32)
    ties = np.where(rng.random(ties.shape) < 0.4, np.nextafter(ties, f32(np.inf)), ties)
    ties = np.where(rng.random(ties.shape) < 0.4, np.nextafter(ties, f32(-np.inf)), ties)
    rand = ((rng.random((nblk, 8)) * 2 - 1) * amax[:, None]).astype(np.float32)
    x = np.clip(np.concatenate([ties, rand], 1), -amax[:, None], amax[:, None])
    sign = np.where(rng.random((nblk, 1)) < 0.5, f32(-1), f32(1))
    blocks = np.concatenate([amax[:, None] * sign, x], 1).astype(np.float32)
    blocks = np.take_along_axis(blocks, rng.permuted(np.tile(np.arange(32), (nblk, 1)), axis=1), 1)
    blocks[::13] = 0
    return blocks


@pytest.mark.parametrize("n", [1, 4, 8, 16])
def test_sweep_quantizers_near_ties_and_extreme_scales(oracle, n):
    # the sweep's quantizers (one row: inside the GEMV launch; 2..24 rows: the batched quantize
    # launch, storing with the non-temporal hint up to 8 rows and without past 8) on adversarial
    # activations: x_q8 equals the oracle's Q8_0 bytes, y the GEMV of those bytes
    require_gpu()
    rng = np.random.default_rng(300 + n)
    shapes = [synth.MatShape("a", 130, 4096), synth.MatShape("b", 64, 1056)]
    hw, _, mats = _stack(90 + n, shapes, n)
    hx = []
    for m, sh in zip(mats, shapes):
        x = _adversarial_blocks(rng, n * sh.cols // 32).reshape(n, sh.cols)
        hx.append(x)
        m["x"] = to_dev(x)
    sw = q.Sweep(mats, n)
    assert sw.info()["fused_quantize"] == int(n == 1)
    sw.run()
    torch.cuda.synchronize()
    for m, w, x, sh in zip(mats, hw, hx, shapes):
        ref = oracle.quantize_q8_0(x)
        assert np.array_equal(q8_canonical(m["x_q8"], n, sh.cols), ref), sh.name
        y = q.gemv_q4_0(m["w_packed"], m["x_q8"], sh.rows, sh.cols, n)
        assert torch.equal(y, m["y"]), sh.name


def test_lm_head_fused_sweep_full_parity(oracle):
    # the lone head as the benchmark times it: a 1-row sweep of one 151936 x 1536 matrix given
    # as fp32, i.e. one launch of 8-wave split tiles quantizing as they stream; every output
    # against the oracle, the Q8_0 bytes bit for bit
    require_gpu()
    rows, cols = 151936, 1536
    w = synth.q4_0_weights(rows, cols, synth.generator(2, 0, 1, 0))
    x = synth.activation(1, cols, synth.generator(2, 0, 1, 1), outliers=0)
    m = {"w_packed": packed_weights(w, rows, cols), "x": to_dev(x),
         "x_q8": torch.full((q.q8_bytes(1, cols),), 0xA5, dtype=torch.uint8, device=dev()),
         "y": torch.full((1, rows), float("nan"), dtype=torch.float32, device=dev()), "rows": rows, "cols": cols}
    sw = q.Sweep([m], 1)
    info = sw.info()
    assert info["fused_quantize"] == 1 and info["n_tiles"] == rows // 64
    sw.run()
    torch.cuda.synchronize()
    xq = oracle.quantize_q8_0(x)
    assert np.array_equal(q8_canonical(m["x_q8"], 1, cols), xq)
    y_ref, S = oracle.gemv(w, xq, rows, cols, 1)
    assert_within(m["y"].cpu().numpy(), y_ref, S, what="lm_head sweep")


@pytest.mark.parametrize("n,split", [(1, True), (1, False), (8, False)])
def test_sweep_timeline(n, split):
    # a traced run records every workgroup's start and its waves' ends (100 MHz clock, ends
    # after the start) and leaves the results bit for bit as an untraced run's
    require_gpu()
    shapes = ([synth.MatShape("a", 257, 1536), synth.MatShape("b", 130, 2048)] if split else
              [synth.MatShape("a", 257, 1536), synth.MatShape("b", 64, 8960), synth.MatShape("c", 90, 4128)])
    _, _, mats = _stack(95 + n, shapes, n)
    sw = q.Sweep(mats, n)
    sw.run()
    torch.cuda.synchronize()
    ref = [m["y"].clone() for m in mats]
    tr = sw.set_trace(True)
    sw.run()
    torch.cuda.synchronize()
    sw.set_trace(False)
    nt = sw.info()["n_tiles"]
    t = tr.cpu().numpy().reshape(nt, 9)
    waves = 8 if split else 4
    assert (t[:, 0] > 0).all() and (t[:, 1:1 + waves] >= t[:, :1]).all()
    assert (t[:, 1 + waves:] == 0).all()
    span_us = (t[:, 1:1 + waves].max() - t[:, 0].min()) / 100.0
    assert 0 < span_us < 1e5
    for m, r in zip(mats, ref):
        assert torch.equal(m["y"], r)


def _one_row_tiles(shapes):
    """Tiles of a 1-row plan: a row group each for matrices of at most 8 chunks, else group sets."""
    n = 0
    for sh in shapes:
        if sh.rows == 0 or sh.cols == 0:
            continue
        g, c = -(-sh.rows // 64), -(-(sh.cols // 32) // 8)
        ks = 1 if c <= 8 else (2 if c <= 16 else 4)
        n += g if ks == 1 else -(-g // (4 // ks))
    return n


def test_sweep_one_row_prequantized_mixed_equals_standalone(oracle):
    # n = 1 over activations quantized by the sweep's own quantize launch (one matrix brings its
    # x_q8 already quantized, so the plan is not fused): matrices of at most 8 chunks run as
    # split tiles, the others (2 and 4 K splits) as group sets, in one GEMV launch; every y
    # equals the standalone GEMV bit for bit
    require_gpu()
    shapes = [synth.MatShape("a", 257, 1536), synth.MatShape("b", 64, 8960), synth.MatShape("c", 1, 32),
              synth.MatShape("d", 130, 4128), synth.MatShape("e", 90, 96), synth.MatShape("f", 200, 3072),
              synth.MatShape("g", 3, 33792), synth.MatShape("h", 65, 2048)]
    hw, hx, mats = _stack(80, shapes, 1)
    mats[7]["x_q8"] = q.quantize_q8_0(mats[7].pop("x"))
    for m in mats:
        m["y"].fill_(float("nan"))
    sw = q.Sweep(mats, 1)
    info = sw.info()
    assert info["fused_quantize"] == 0
    assert info["n_tiles"] == _one_row_tiles(shapes)
    sw.run()
    sw.run()
    torch.cuda.synchronize()
    for m, x, sh in zip(mats, hx, shapes):
        xq = q.quantize_q8_0(to_dev(x))
        assert torch.equal(xq, m["x_q8"]), sh.name
        y = q.gemv_q4_0(m["w_packed"], xq, m["rows"], m["cols"], 1)
        assert torch.equal(y, m["y"]), sh.name
    # and against the oracle's fixed-order GEMV for one single-split and one split-K matrix
    for i in (0, 5):
        y_ref, S = oracle.gemv(hw[i], oracle.quantize_q8_0(hx[i]), shapes[i].rows, shapes[i].cols, 1)
        assert_within(mats[i]["y"].cpu().numpy(), y_ref, S, what=shapes[i].name)


@pytest.mark.parametrize("n", [1, 4])
def test_sweep_not_fused_with_a_prequantized_activation(n):
    # a matrix without x reads its x_q8 as given: the plan keeps two launches
    require_gpu()
    shapes = [synth.MatShape("a", 65, 1536), synth.MatShape("b", 3, 2048)]
    _, hx, mats = _stack(79, shapes, n)
    mats[1]["x_q8"] = q.quantize_q8_0(mats[1].pop("x"))
    sw = q.Sweep(mats, n)
    assert sw.info()["fused_quantize"] == 0
    sw.run()
    torch.cuda.synchronize()
    for m, x in zip(mats, hx):
        y = q.gemv_q4_0(m["w_packed"], q.quantize_q8_0(to_dev(x)), m["rows"], m["cols"], n)
        assert torch.equal(y, m["y"])


def test_qwen15_n1_full_parity(oracle, qwen15):
    hw, hx, mats = qwen15
    sw = q.Sweep(mats, 1)
    info = sw.info()
    assert info["weight_bytes"] == 868_257_792
    for m in mats:
        m["y"].fill_(float("nan"))
    sw.run()
    sw.run()                                    # repeated runs give the same bytes
    torch.cuda.synchronize()
    worst = 0.0
    for i, (w, x, m) in enumerate(zip(hw, hx, mats)):
        y_ref, S = oracle.gemv(w, oracle.quantize_q8_0(x), m["rows"], m["cols"], 1)
        worst = max(worst, assert_within(m["y"].cpu().numpy(), y_ref, S, what=f"matrix {i}"))
    print(f"worst |y - y_ref| / S = {worst:.3e}")
    # sweep == standalone GEMV, bit for bit
    for i in (0, 1, 4, 6, 196):
        m = mats[i]
        y = q.gemv_q4_0(m["w_packed"], m["x_q8"], m["rows"], m["cols"], 1)
        assert torch.equal(y, m["y"])


@pytest.mark.parametrize("n", [8, 24])
def test_qwen15_multi_row_verify(oracle, qwen15, n):
    hw, _, mats1 = qwen15
    shapes = synth.qwen25_1p5b()
    mats8, hx8 = [], []
    for mi, (s, m1) in enumerate(zip(shapes, mats1)):
        x = synth.activation(n, s.cols, synth.generator(3, mi, 0, 1))
        hx8.append(x)
        mats8.append({"w_packed": m1["w_packed"], "x": to_dev(x),
                      "x_q8": torch.empty(q.q8_bytes(n, s.cols), dtype=torch.uint8, device=dev()),
                      "y": torch.empty((n, s.rows), dtype=torch.float32, device=dev()),
                      "rows": s.rows, "cols": s.cols})
    q.Sweep(mats8, n).run()
    torch.cuda.synchronize()
    # every output of every matrix against the fp64 oracle
    worst = 0.0
    for i, s in enumerate(shapes):
        y_ref, S = oracle.gemv(hw[i], oracle.quantize_q8_0(hx8[i]), s.rows, s.cols, n)
        worst = max(worst, assert_within(mats8[i]["y"].cpu().numpy(), y_ref, S, what=f"matrix {i}"))
    print(f"worst |y - y_ref| / S = {worst:.3e}")
    # each row of the n-row sweep equals the 1-row sweep of that activation
    for t in (0, 5, n - 1):
        mats_t = [{"w_packed": m["w_packed"], "x": m["x"][t:t + 1].contiguous(),
                   "x_q8": torch.empty(q.q8_bytes(1, m["cols"]), dtype=torch.uint8, device=dev()),
                   "y": torch.empty((1, m["rows"]), dtype=torch.float32, device=dev()),
                   "rows": m["rows"], "cols": m["cols"]} for m in mats8]
        q.Sweep(mats_t, 1).run()
        torch.cuda.synchronize()
        for m8, mt in zip(mats8, mats_t):
            assert torch.equal(m8["y"][t], mt["y"][0])


def test_lm_head_full_parity(oracle):
    require_gpu()
    rows, cols = 151936, 1536
    w = synth.q4_0_weights(rows, cols, synth.generator(2, 0, 0, 0))
    x = synth.activation(1, cols, synth.generator(2, 0, 0, 1), outliers=0)
    y = q.gemv_q4_0(packed_weights(w, rows, cols), q.quantize_q8_0(to_dev(x)), rows, cols, 1)
    y_ref, S = oracle.gemv(w, oracle.quantize_q8_0(x), rows, cols, 1)
    assert_within(y.cpu().numpy(), y_ref, S, what="lm_head")


@pytest.mark.parametrize("n", [1, 8])
def test_qwen7b_full_parity(oracle, n):
    # the 7B-shaped sweep as the benchmark times it: every output of every matrix against the
    # fp64 oracle
    require_gpu()
    shapes = synth.qwen25_7b()
    hw, hx, mats = _stack(4, shapes, n)
    sw = q.Sweep(mats, n)
    assert sw.info()["weight_bytes"] == 3_977_035_776
    sw.run()
    torch.cuda.synchronize()
    worst = 0.0
    for i, s in enumerate(shapes):
        y_ref, S = oracle.gemv(hw[i], oracle.quantize_q8_0(hx[i]), s.rows, s.cols, n)
        worst = max(worst, assert_within(mats[i]["y"].cpu().numpy(), y_ref, S, what=f"7B matrix {i}"))
    print(f"worst |y - y_ref| / S = {worst:.3e}")
    del mats
    torch.cuda.empty_cache()
