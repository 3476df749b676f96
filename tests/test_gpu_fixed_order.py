"""Order and determinism checks: the GEMV entry points equal the oracle's
fixed-order fp32 GEMV (a transcription of the kernels' own summation order, the
reading of milestone M16: one rounded expression per block and one
accumulation order) bit for bit: 1-row dot4 path, 2..8-row MFMA path and
9..24-row tiled path, at shapes covering one, two and four K splits, segments
and ragged tails.  The parity bar itself -- within 1e-5 * sum|terms| of the fp64
definition -- is checked in test_gpu_kernels.py and test_gpu_sweep.py."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, packed_weights, q8_canonical, require_gpu, to_dev
from q4_weight_streaming_amd import _lib as q
from q4_weight_streaming_amd import synth

pytestmark = pytest.mark.gpu

SHAPES = [(256, 1536), (1536, 8960), (130, 18944), (70, 800), (64, 2304), (9, 17408)]


@pytest.mark.parametrize("n", [1, 3, 8, 17])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_gemv_equals_fixed_order_oracle(oracle, rows, cols, n):
    require_gpu()
    w = synth.q4_0_weights(rows, cols, synth.generator(60, rows, cols, 0))
    x = synth.activation(n, cols, synth.generator(60, rows, cols, 1))
    wp = packed_weights(w, rows, cols)
    xq = q.quantize_q8_0(to_dev(x))
    y = q.gemv_q4_0(wp, xq, rows, cols, n)
    xq8 = oracle.quantize_q8_0(x)
    assert np.array_equal(q8_canonical(xq, n, cols), xq8)      # the GPU's bytes are the oracle's
    ref = oracle.gemv_f32(w, xq8, rows, cols, n)
    got = y.cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} of {got.size} differ, first {bad[0]}: {got[tuple(bad[0])]!r} vs {ref[tuple(bad[0])]!r}"


SINGLE_SPLIT = [(257, 1536), (64, 32), (130, 96), (70, 2048), (1, 800), (200, 288), (65, 640), (3, 1824)]


@pytest.mark.parametrize("fused", [True, False])
def test_single_split_sweep_equals_fixed_order_oracle(oracle, fused):
    """A 1-row sweep whose matrices all have one K split (at most 8 chunks) runs
    one 4-wave workgroup per row group, the chunks spread over the waves and the
    fp32 chains taken from exact block sums in LDS: chunk counts 1..8 (waves
    without a chunk), padding blocks, ragged row groups; with the activation
    quantized inside the launch or given as Q8_0."""
    require_gpu()
    mats, hw, hx = [], [], []
    for i, (rows, cols) in enumerate(SINGLE_SPLIT):
        w = synth.q4_0_weights(rows, cols, synth.generator(61, i, 0, 0))
        x = synth.activation(1, cols, synth.generator(61, i, 0, 1))
        m = {"w_packed": packed_weights(w, rows, cols),
             "x_q8": torch.empty(q.q8_bytes(1, cols), dtype=torch.uint8, device=dev()),
             "y": torch.full((1, rows), float("nan"), dtype=torch.float32, device=dev()),
             "rows": rows, "cols": cols}
        if fused:
            m["x"] = to_dev(x)
        else:
            m["x_q8"] = q.quantize_q8_0(to_dev(x))
        mats.append(m)
        hw.append(w)
        hx.append(x)
    sw = q.Sweep(mats, 1)
    assert sw.info()["fused_quantize"] == int(fused)
    sw.run()
    torch.cuda.synchronize()
    for (rows, cols), m, w, x in zip(SINGLE_SPLIT, mats, hw, hx):
        xq8 = oracle.quantize_q8_0(x)
        assert np.array_equal(q8_canonical(m["x_q8"], 1, cols), xq8)
        ref = oracle.gemv_f32(w, xq8, rows, cols, 1)
        got = m["y"].cpu().numpy()
        bad = np.argwhere(got.view(np.uint32) != ref.view(np.uint32))
        assert bad.size == 0, f"{rows}x{cols}: {len(bad)} of {got.size} differ, first {bad[0]}"
