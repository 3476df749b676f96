"""GPU parity of the chained decode step (q4s_chain_*).

Against the plain definitions (the parity bar): every phase's staged Q8_0 input,
exported by the step itself, is the Q8_0 quantization of the GPU's own fp32
input -- bit for bit where that input is a stored vector (o reads q, down reads
g * u), and, behind an RMS norm, equal to the quantization of the fp64 norm of
the GPU's own vector except at rare elements within the fp32 norm's error bound
of a rounding boundary; every GEMV output is within 1e-5 * sum|terms| of the
fp64 GEMV of that staged input; the residual sums are single fp32 additions.
Checked at the Qwen2.5-1.5B shape (28 layers, 868 MB) and the 7B shape.

Order and determinism (the same arithmetic in a fixed order): every intermediate
vector and the logits equal the oracle's fixed-order transcription of the
step (q4o_chain_step: the kernel's fp32 order of the milestone M16 reading, the
Q8_0 quantizer and the RMS norm's lane-partial order) bit for bit, in all three
phase-synchronisation modes, at small, ragged and full shapes, with the
persistent workgroup count both one per compute unit and below the number of
tiles of a phase.  Gate and up run as one paired matrix whose tiles hand g * u
to down as Q8_0 words (every tile layout: two groups per tile, group sets of
one and two K splits), and as two matrices when their rows have four K splits."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, packed_weights, require_gpu, to_dev
from q4_weight_streaming_amd import _lib as q
from q4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu

MODES = [q.CHAIN_COUNTER, q.CHAIN_TREE, q.CHAIN_TAGGED]
MODE_IDS = ["counter", "tree", "tagged"]


def _inputs(cfg, layers, E, D, F, V, scale=1.0, outliers=8):
    shapes = [(E, E), (D, E), (D, E), (E, E), (F, E), (F, E), (E, F)] * layers + [(V, E)]
    ws = [synth.q4_0_weights(r, c, synth.generator(cfg, m, 0, 0)) for m, (r, c) in enumerate(shapes)]
    h0 = (scale * synth.activation(1, E, synth.generator(cfg, 999, 0, 1), outliers=outliers)[0]).astype(np.float32)
    return shapes, ws, h0


def _device(shapes, ws, h0, layers, E, D, F, V):
    wp = [packed_weights(w, r, c) for w, (r, c) in zip(ws, shapes)]
    words = q.chain_act_words(layers, E, D, F, V)
    acts = torch.empty(max(words, 1), dtype=torch.int64, device=dev())
    logits = torch.empty(V, dtype=torch.float32, device=dev())
    torch.cuda.synchronize()
    return wp, to_dev(h0), acts, logits


def _run(wp, h0d, acts, logits, layers, E, D, F, V, mode, workgroups, steps=1):
    ch = q.Chain(layers, E, D, F, V, wp, h0d, acts, logits, sync_mode=mode, workgroups=workgroups)
    for _ in range(steps):
        ch.run()
    ch.check()
    info = ch.info()
    ch.close()
    words = q.chain_act_words(layers, E, D, F, V)
    vals, tags = q.chain_values(acts[:words])
    return vals.cpu().numpy(), tags.cpu().numpy(), logits.cpu().numpy().copy(), info


def _compare(oracle_acts, oracle_logits, vals, logits, layers, E, D, F, what):
    lay, per = q.chain_layout(E, D, F)
    got = vals.reshape(layers, per) if layers else vals[:0]
    for l in range(layers):
        for name, (off, n) in lay.items():
            a, b = got[l, off:off + n], oracle_acts[l, off:off + n]
            bad = np.flatnonzero(a != b)
            assert bad.size == 0, f"{what}: layer {l} {name}: {bad.size} of {n} differ, first at {bad[0]}: {a[bad[0]]!r} vs {b[bad[0]]!r}"
    bad = np.flatnonzero(logits != oracle_logits)
    assert bad.size == 0, f"{what}: {bad.size} logits differ, first at {bad[0]}"


@pytest.mark.parametrize("workgroups", [0, 5], ids=["per_cu", "wg5"])
@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_chain_small_bit_exact(oracle, mode, workgroups):
    require_gpu()
    L, E, D, F, V = 2, 256, 64, 384, 320
    shapes, ws, h0 = _inputs(40, L, E, D, F, V)
    ref_acts, ref_logits = oracle.chain_step(ws, E, D, F, V, h0)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    vals, tags, lg, info = _run(wp, h0d, acts, logits, L, E, D, F, V, mode, workgroups)
    assert info["n_phases"] == 4 * L + 1 and info["steps"] == 1
    assert (tags == 1).all()
    _compare(ref_acts, ref_logits, vals, lg, L, E, D, F, f"mode {mode}")


@pytest.mark.parametrize("workgroups", [0, 5], ids=["per_cu", "wg5"])
@pytest.mark.parametrize("E,F", [(768, 2304), (1280, 1024)], ids=["ranges_3_4_5", "ranges_5_4"])
def test_chain_split_range_lengths(oracle, E, F, workgroups):
    """Split tiles whose K ranges hold 3, 4 and 5 chunks (hidden 768: 3 chunks; ff 2304: 9
    chunks in two K splits of 4 and 5; hidden 1280: 5 chunks; ff 1024: 4), each range's chain
    read and added as one batch of exactly its chunks; on 256 and on 5 workgroups (coarser
    layouts): bit-exact against the oracle's fixed order, tagged phases."""
    require_gpu()
    L, D, V = 2, 64, 320
    shapes, ws, h0 = _inputs(44, L, E, D, F, V)
    ref_acts, ref_logits = oracle.chain_step(ws, E, D, F, V, h0)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    vals, tags, lg, info = _run(wp, h0d, acts, logits, L, E, D, F, V, q.CHAIN_TAGGED, workgroups)
    assert info["n_phases"] == 4 * L + 1
    assert (tags == 1).all()
    _compare(ref_acts, ref_logits, vals, lg, L, E, D, F, f"E={E} F={F}")


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_chain_ragged_shapes(oracle, mode):
    """hidden 96 and ff 160 (partial chunks), kv_dim 5 and vocab 77 (partial row groups),
    three layers, three workgroups (fewer than the tiles of most phases)."""
    require_gpu()
    L, E, D, F, V = 3, 96, 5, 160, 77
    shapes, ws, h0 = _inputs(41, L, E, D, F, V)
    ref_acts, ref_logits = oracle.chain_step(ws, E, D, F, V, h0)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    vals, tags, lg, _ = _run(wp, h0d, acts, logits, L, E, D, F, V, mode, 3)
    assert (tags == 1).all()
    _compare(ref_acts, ref_logits, vals, lg, L, E, D, F, "ragged")


@pytest.mark.parametrize("mode", [q.CHAIN_TREE, q.CHAIN_TAGGED], ids=["tree", "tagged"])
def test_chain_wide_hidden_unpaired(oracle, mode):
    """hidden 4352 (17 chunks: four K splits), so gate and up cannot run as one paired
    matrix and down quantizes g * u itself; ff 96 (one partial chunk)."""
    require_gpu()
    L, E, D, F, V = 1, 4352, 32, 96, 64
    shapes, ws, h0 = _inputs(43, L, E, D, F, V, scale=0.05, outliers=0)
    ref_acts, ref_logits = oracle.chain_step(ws, E, D, F, V, h0)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    vals, tags, lg, info = _run(wp, h0d, acts, logits, L, E, D, F, V, mode, 0)
    assert info["n_phases"] == 4 * L + 1
    assert (tags == 1).all()
    _compare(ref_acts, ref_logits, vals, lg, L, E, D, F, "wide hidden")


@pytest.mark.parametrize("workgroups", [0, 5], ids=["per_cu", "wg5"])
def test_chain_norm_vector_shared_at_its_limit(oracle, workgroups):
    """Tagged phases read a norm phase's vector once per workgroup into LDS when it
    has at most 4096 elements: hidden 4096 fills that copy (16 chunks).  With 5
    workgroups each one runs many tiles of every norm phase, so most tiles find
    the phase's vector already claimed and wait for it instead of loading it;
    two layers make each workgroup claim a new phase after an old one."""
    require_gpu()
    L, E, D, F, V = 2, 4096, 64, 384, 320
    shapes, ws, h0 = _inputs(49, L, E, D, F, V, scale=0.05, outliers=0)
    ref_acts, ref_logits = oracle.chain_step(ws, E, D, F, V, h0)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    vals, tags, lg, info = _run(wp, h0d, acts, logits, L, E, D, F, V, q.CHAIN_TAGGED, workgroups, steps=2)
    assert (tags == 2).all()
    _compare(ref_acts, ref_logits, vals, lg, L, E, D, F, f"hidden 4096, {workgroups} workgroups")


@pytest.mark.parametrize("F,workgroups",[(4608, 0), (4608, 5), (17408, 0), (17408, 5), (32768, 0), (32768, 5)],
                         ids=["ranges4_per_cu", "ranges4_wg5", "ranges17_per_cu", "ranges17_wg5",
                              "ranges32_per_cu", "ranges32_wg5"])
def test_chain_k_range_tiles_bit_exact(oracle, F, workgroups):
    """Tagged phases: down with four K splits runs one tile per (K range, row group), ranges
    1..3 handing their sums to range 0 as tagged words.  F = 4608: ranges of 4-5 chunks; F =
    17408: 17 chunks, two fp32 segments per range; F = 32768 (the largest ff a chain accepts):
    32-chunk ranges that fill the terms table and exactly two 16-chunk segments, 8 chunks per
    wave.  With 5 workgroups each runs several such tiles in turn (range 0 last).  Results
    equal the oracle's bit for bit."""
    require_gpu()
    L, E, D, V = 2, 256, 64, 320
    shapes, ws, h0 = _inputs(47, L, E, D, F, V)
    ref_acts, ref_logits = oracle.chain_step(ws, E, D, F, V, h0)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    vals, tags, lg, info = _run(wp, h0d, acts, logits, L, E, D, F, V, q.CHAIN_TAGGED, workgroups, steps=2)
    assert (tags == 2).all()
    _compare(ref_acts, ref_logits, vals, lg, L, E, D, F, f"K-range tiles, {workgroups} workgroups")


def test_chain_plain_launch_equals_cooperative(oracle):
    """The step launched without the cooperative-launch call (one workgroup per CU, on an
    otherwise idle GPU) gives the same bits as the cooperative launch and the oracle."""
    require_gpu()
    L, E, D, F, V = 2, 256, 64, 384, 320
    shapes, ws, h0 = _inputs(48, L, E, D, F, V)
    ref_acts, ref_logits = oracle.chain_step(ws, E, D, F, V, h0)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    ch = q.Chain(L, E, D, F, V, wp, h0d, acts, logits, sync_mode=q.CHAIN_TAGGED, workgroups=0)
    ch.set_cooperative(False)
    ch.run()
    ch.run()
    ch.check()
    ch.close()
    words = q.chain_act_words(L, E, D, F, V)
    vals, tags = q.chain_values(acts[:words])
    assert (tags.cpu().numpy() == 2).all()
    _compare(ref_acts, ref_logits, vals.cpu().numpy(), logits.cpu().numpy(), L, E, D, F, "plain launch")


def test_chain_head_only(oracle):
    require_gpu()
    L, E, D, F, V = 0, 128, 64, 64, 200
    shapes, ws, h0 = _inputs(42, L, E, D, F, V)
    _, ref_logits = oracle.chain_step(ws, E, D, F, V, h0)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    _, _, lg, info = _run(wp, h0d, acts, logits, L, E, D, F, V, q.CHAIN_TAGGED, 0)
    assert info["n_phases"] == 1
    np.testing.assert_array_equal(lg, ref_logits)


def test_chain_repeated_steps_are_identical(oracle):
    """Three steps on one chain: every word carries the third step's tag, same values."""
    require_gpu()
    L, E, D, F, V = 2, 256, 64, 384, 320
    shapes, ws, h0 = _inputs(43, L, E, D, F, V)
    ref_acts, ref_logits = oracle.chain_step(ws, E, D, F, V, h0)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    vals, tags, lg, info = _run(wp, h0d, acts, logits, L, E, D, F, V, q.CHAIN_TAGGED, 0, steps=3)
    assert info["steps"] == 3 and (tags == 3).all()
    _compare(ref_acts, ref_logits, vals, lg, L, E, D, F, "third step")


@pytest.fixture(scope="module")
def qwen15_chain(oracle):
    require_gpu()
    L, E, D, F, V = 28, 1536, 256, 8960, 151936
    shapes, ws, h0 = _inputs(44, L, E, D, F, V)
    ref = oracle.chain_step(ws, E, D, F, V, h0)
    dv = _device(shapes, ws, h0, L, E, D, F, V)
    return (L, E, D, F, V), ref, dv, (shapes, ws, h0)


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_chain_qwen15_full_bit_exact(qwen15_chain, mode):
    """The Qwen2.5-1.5B-shaped chain (28 layers, 868 MB of weights), one workgroup per
    compute unit: all 28 x 9 vectors and the 151936 logits equal the oracle's."""
    (L, E, D, F, V), (ref_acts, ref_logits), (wp, h0d, acts, logits), _ = qwen15_chain
    vals, tags, lg, info = _run(wp, h0d, acts, logits, L, E, D, F, V, mode, 0)
    assert info["n_phases"] == 113 and (tags == 1).all()
    assert np.isfinite(lg).all()
    _compare(ref_acts, ref_logits, vals, lg, L, E, D, F, f"1.5B mode {mode}")


@pytest.mark.parametrize("mode", [q.CHAIN_TREE, q.CHAIN_TAGGED], ids=["tree", "tagged"])
def test_chain_trace_timeline(oracle, mode):
    """With a trace buffer, a step records every workgroup's end of every phase after the
    launch start; under a barrier every workgroup's ends are non-decreasing; results unchanged."""
    require_gpu()
    L, E, D, F, V = 2, 256, 64, 384, 320
    shapes, ws, h0 = _inputs(45, L, E, D, F, V)
    ref_acts, ref_logits = oracle.chain_step(ws, E, D, F, V, h0)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    ch = q.Chain(L, E, D, F, V, wp, h0d, acts, logits, sync_mode=mode, workgroups=6)
    tr = ch.set_trace(True)
    ch.run()
    ch.check()
    info = ch.info()
    t = tr.cpu().numpy()
    P, wg = info["n_phases"], info["workgroups"]
    assert P == 9 and wg == 6 and t.size == (3 * P + 1) * wg
    ends, wstart = t[:P * wg].reshape(P, wg), t[P * wg:P * wg + wg]
    tstart = t[P * wg + wg:2 * P * wg + wg].reshape(P, wg)
    tready = t[2 * P * wg + wg:].reshape(P, wg)
    start = wstart.min()
    assert (wstart > 0).all() and (ends >= wstart[None, :]).all()
    has = tstart > 0                     # workgroups with a tile in the phase
    assert has.any(axis=1).all() and ((tready > 0) == has).all()
    assert (tstart[has] >= start).all() and (tready[has] >= tstart[has]).all() and (ends[has] >= tready[has]).all()
    if mode != q.CHAIN_TAGGED:
        assert (np.diff(ends, axis=0) >= 0).all()
    ch.set_trace(False)
    ch.close()
    vals, _ = q.chain_values(acts[:q.chain_act_words(L, E, D, F, V)])
    _compare(ref_acts, ref_logits, vals.cpu().numpy(), logits.cpu().numpy(), L, E, D, F, "traced")


@pytest.mark.parametrize("mode", MODES, ids=MODE_IDS)
def test_chain_wait_limit_zero_reports_and_recovers(oracle, mode):
    """With a wait limit of 0 polls a wait that finds its input not yet ready gives up: the
    step still ends (no hang), q4s_chain_check reports Q4S_ERR_WAIT; with the default limit
    restored the next step is bit-exact again."""
    require_gpu()
    L, E, D, F, V = 4, 256, 64, 384, 320
    shapes, ws, h0 = _inputs(46, L, E, D, F, V)
    ref_acts, ref_logits = oracle.chain_step(ws, E, D, F, V, h0)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    ch = q.Chain(L, E, D, F, V, wp, h0d, acts, logits, sync_mode=mode, workgroups=0)
    ch.set_wait_limit(0)
    ch.run()
    with pytest.raises(q.Q4SError) as e:
        ch.check()
    assert e.value.status == q.ERR_WAIT
    ch.set_wait_limit(1 << 20)
    ch.run()
    ch.check()
    ch.close()
    vals, tags = q.chain_values(acts[:q.chain_act_words(L, E, D, F, V)])
    assert (tags.cpu().numpy() == 2).all()
    _compare(ref_acts, ref_logits, vals.cpu().numpy(), logits.cpu().numpy(), L, E, D, F, "after recovery")


@pytest.fixture(scope="module")
def qwen7b_chain(oracle):
    require_gpu()
    L, E, D, F, V = 28, 3584, 512, 18944, 152064
    shapes, ws, h0 = _inputs(47, L, E, D, F, V)
    ref = oracle.chain_step(ws, E, D, F, V, h0)
    dv = _device(shapes, ws, h0, L, E, D, F, V)
    return (L, E, D, F, V), ref, dv, (shapes, ws, h0)


def test_chain_qwen7b_full_bit_exact(qwen7b_chain):
    """The Qwen2.5-7B-shaped chain (28 layers, 3.98 GB), tagged sync: every vector and logit
    equals the oracle's (ff 18944: four K splits of 18-19 chunks, two segments each)."""
    (L, E, D, F, V), (ref_acts, ref_logits), (wp, h0d, acts, logits), _ = qwen7b_chain
    vals, tags, lg, info = _run(wp, h0d, acts, logits, L, E, D, F, V, q.CHAIN_TAGGED, 0)
    assert info["n_phases"] == 113 and (tags == 1).all() and np.isfinite(lg).all()
    _compare(ref_acts, ref_logits, vals, lg, L, E, D, F, "7B tagged")


# ------------------------------------------------------------- against the definitions

U = 2.0 ** -24


def _staged_blocks(oracle, dump, p, C, K):
    """Phase p's staged activation from the stage dump (words [phase][chunk][lane]: code
    dword | fp32 bits of the block's d_x << 32) as canonical Q8_0 blocks uint8 [K/32][34]
    (byte moves; the d_x values are binary16 values, so their conversion is exact)."""
    d = dump.reshape(-1, C, 64)[p, :(K + 255) // 256]
    lo = (d & 0xFFFFFFFF).astype(np.uint32)
    hi = ((d >> 32) & 0xFFFFFFFF).astype(np.uint32)
    nb = K // 32
    codes = lo.reshape(-1).view(np.uint8)[:K].reshape(nb, 32)
    dx = hi.reshape(-1)[::8][:nb].view(np.float32)        # lanes 8b .. 8b+7 carry block b's d_x
    blocks = np.empty((nb, 34), np.uint8)
    blocks[:, :2] = oracle.f32_to_fp16(dx).view(np.uint8).reshape(nb, 2)
    blocks[:, 2:] = codes
    return blocks


def _norm_code_mismatches(oracle, h, blocks, what):
    """Staged codes of a normalized input against the quantization of the fp64 norm of the
    GPU's own h (rounded to fp32).  A block may differ only where the fp32 norm's error can
    move a rounding decision: the GPU's normalized values are within delta (relative) of the
    fp64 ones, delta = 2 * ((n/64 + 6)/2 + 4) * 2^-24 (twice the bound pinned on the CPU), so
    its d_x must lie between binary16(d(1 - delta')) and binary16(d(1 + delta')), d =
    max|x|/127, delta' = delta + 2^-23, and each code within 0.5 + 127 (2 delta + 3 * 2^-24) of
    x/d.  Returns the number of differing blocks."""
    n = h.size
    x64 = oracle.rmsnorm_f64(h)
    ref = oracle.quantize_q8_0(x64.astype(np.float32)).reshape(-1, 34)
    bad = np.flatnonzero((ref != blocks).any(axis=1))
    delta = 2 * ((n / 64 + 6) / 2 + 4) * U
    xb = x64.reshape(-1, 32)
    for b in bad:
        d64 = np.abs(xb[b]).max() / 127.0
        lo = oracle.fp16_to_f32(oracle.f32_to_fp16(np.float32([d64 * (1 - delta - 2 * U)])))[0]
        hi = oracle.fp16_to_f32(oracle.f32_to_fp16(np.float32([d64 * (1 + delta + 2 * U)])))[0]
        dg = oracle.fp16_to_f32(blocks[b, :2].copy().view(np.uint16))[0]
        assert lo <= dg <= hi, f"{what}: block {b} d_x {dg!r} outside [{lo!r}, {hi!r}]"
        qg = blocks[b, 2:].view(np.int8).astype(np.float64)
        assert np.all(np.abs(qg - xb[b] / d64) <= 0.5 + 127 * (2 * delta + 3 * U)), f"{what}: block {b} codes"
    return bad.size


def _check_gemv(oracle, w, blocks, rows, cols, y, what):
    y_ref, S = oracle.gemv(w, blocks.reshape(1, -1), rows, cols, 1)
    err = np.abs(y.astype(np.float64) - y_ref[0])
    assert np.all(err <= 1e-5 * S[0]), f"{what}: max |y - y_ref| / S = {float((err / S[0]).max()):.3e}"


def _check_chain_definition(oracle, dims, host, vals, logits, dump):
    """Every phase of one chained step against the plain definitions (see the module doc)."""
    L, E, D, F, V = dims
    shapes, ws, h0 = host
    C = max((E + 255) // 256, (F + 255) // 256)
    lay, per = q.chain_layout(E, D, F)
    got = vals.reshape(L, per) if L else vals[:0]

    def vec(l, name):
        off, n = lay[name]
        return got[l, off:off + n]

    mism, norm_blocks = 0, 0
    h = h0.astype(np.float32)
    for l in range(L):
        wq, wk, wv, wo, wg, wu, wd = ws[7 * l:7 * l + 7]
        # q, k, v read Q8(norm h)
        xb = _staged_blocks(oracle, dump, 4 * l, C, E)
        mism += _norm_code_mismatches(oracle, h, xb, f"layer {l} qkv")
        norm_blocks += E // 32
        _check_gemv(oracle, wq, xb, E, E, vec(l, "q"), f"layer {l} q")
        _check_gemv(oracle, wk, xb, D, E, vec(l, "k"), f"layer {l} k")
        _check_gemv(oracle, wv, xb, D, E, vec(l, "v"), f"layer {l} v")
        # o reads Q8(q); h1 = h + o
        xb = _staged_blocks(oracle, dump, 4 * l + 1, C, E)
        assert np.array_equal(xb, oracle.quantize_q8_0(vec(l, "q")).reshape(-1, 34)), f"layer {l}: o's input"
        _check_gemv(oracle, wo, xb, E, E, vec(l, "o"), f"layer {l} o")
        assert np.array_equal(vec(l, "h1"), h + vec(l, "o")), f"layer {l}: h1 != h + o"
        h1 = vec(l, "h1")
        # gate and up read Q8(norm h1)
        xb = _staged_blocks(oracle, dump, 4 * l + 2, C, E)
        mism += _norm_code_mismatches(oracle, h1, xb, f"layer {l} gate/up")
        norm_blocks += E // 32
        _check_gemv(oracle, wg, xb, F, E, vec(l, "g"), f"layer {l} gate")
        _check_gemv(oracle, wu, xb, F, E, vec(l, "u"), f"layer {l} up")
        # down reads Q8(g * u); h2 = h1 + dn
        xb = _staged_blocks(oracle, dump, 4 * l + 3, C, F)
        assert np.array_equal(xb, oracle.quantize_q8_0(vec(l, "g") * vec(l, "u")).reshape(-1, 34)), \
            f"layer {l}: down's input"
        _check_gemv(oracle, wd, xb, E, F, vec(l, "dn"), f"layer {l} down")
        assert np.array_equal(vec(l, "h2"), h1 + vec(l, "dn")), f"layer {l}: h2 != h1 + dn"
        h = vec(l, "h2")
    xb = _staged_blocks(oracle, dump, 4 * L, C, E)
    mism += _norm_code_mismatches(oracle, h, xb, "head")
    norm_blocks += E // 32
    _check_gemv(oracle, ws[7 * L], xb, V, E, logits, "head")
    # behind a norm the staged codes are the fp64 definition's except at rare boundary blocks
    assert mism <= 0.02 * norm_blocks + 2, f"{mism} of {norm_blocks} normalized blocks differ"
    return mism, norm_blocks


def _run_with_dump(wp, h0d, acts, logits, dims):
    L, E, D, F, V = dims
    ch = q.Chain(L, E, D, F, V, wp, h0d, acts, logits, sync_mode=q.CHAIN_TAGGED, workgroups=0)
    dump = ch.set_stage_dump(True)
    ch.run()
    ch.check()
    ch.set_stage_dump(False)
    ch.close()
    vals, tags = q.chain_values(acts[:q.chain_act_words(L, E, D, F, V)])
    assert (tags.cpu().numpy() == 1).all()
    return vals.cpu().numpy(), logits.cpu().numpy().copy(), dump.cpu().numpy()


@pytest.mark.parametrize("dims,cfg", [((2, 256, 64, 384, 320), 48), ((3, 96, 5, 160, 77), 49)],
                         ids=["small", "ragged"])
def test_chain_small_against_definition(oracle, dims, cfg):
    require_gpu()
    L, E, D, F, V = dims
    shapes, ws, h0 = _inputs(cfg, L, E, D, F, V)
    wp, h0d, acts, logits = _device(shapes, ws, h0, L, E, D, F, V)
    vals, lg, dump = _run_with_dump(wp, h0d, acts, logits, dims)
    _check_chain_definition(oracle, dims, (shapes, ws, h0), vals, lg, dump)


def test_chain_qwen15_against_definition(oracle, qwen15_chain):
    """The Qwen2.5-1.5B-shaped chain (tagged phases, one workgroup per compute unit), every
    phase of all 28 layers and the head against the plain definitions."""
    dims, _, (wp, h0d, acts, logits), host = qwen15_chain
    vals, lg, dump = _run_with_dump(wp, h0d, acts, logits, dims)
    mism, blocks = _check_chain_definition(oracle, dims, host, vals, lg, dump)
    print(f"1.5B chain: {mism} of {blocks} normalized Q8_0 blocks at a rounding boundary", flush=True)


def test_chain_qwen7b_against_definition(oracle, qwen7b_chain):
    """The Qwen2.5-7B-shaped chain, every phase against the plain definitions."""
    dims, _, (wp, h0d, acts, logits), host = qwen7b_chain
    vals, lg, dump = _run_with_dump(wp, h0d, acts, logits, dims)
    mism, blocks = _check_chain_definition(oracle, dims, host, vals, lg, dump)
    print(f"7B chain: {mism} of {blocks} normalized Q8_0 blocks at a rounding boundary", flush=True)
