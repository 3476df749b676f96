"""The GEMV entry points equal the oracle's fixed-order fp32 GEMV (the reading of
milestone M16: one rounded expression per block and one accumulation order)
bit for bit: 1-row dot4 path, 2..8-row MFMA path and 9..24-row tiled path, at
shapes covering one, two and four K splits, segments and ragged tails."""
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
    ref = oracle.gemv_f32(w, q8_canonical(xq, n, cols), rows, cols, n)
    got = y.cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} of {got.size} differ, first {bad[0]}: {got[tuple(bad[0])]!r} vs {ref[tuple(bad[0])]!r}"
