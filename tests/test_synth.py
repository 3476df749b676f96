"""The seeded input generators: determinism, distributions and workload shapes."""
import numpy as np

from q4_weight_streaming_amd import synth


def test_weights_deterministic_and_shaped():
    a = synth.q4_0_weights(64, 256, synth.generator(0, 1, 2))
    b = synth.q4_0_weights(64, 256, synth.generator(0, 1, 2))
    c = synth.q4_0_weights(64, 256, synth.generator(0, 1, 3))
    assert a.shape == (64, 8, 18) and a.dtype == np.uint8
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_weight_distribution():
    w = synth.q4_0_weights(512, 4096, synth.generator(5, 0))
    d = w[:, :, 0:2].copy().view("<f2")[:, :, 0].astype(np.float64)
    assert d.min() >= 0
    # E|N(0, s)| / 8 = s * sqrt(2/pi) / 8
    assert abs(d.mean() - 0.02 * np.sqrt(2 / np.pi) / 8) < 2e-5
    assert (d < 2.0 ** -14).mean() > 0.005        # subnormal scales occur
    nib = np.concatenate([w[..., 2:] & 15, w[..., 2:] >> 4], -1)
    counts = np.bincount(nib.ravel(), minlength=16) / nib.size
    assert np.all(np.abs(counts - 1 / 16) < 2e-3)


def test_activation_outliers_shared_across_rows():
    x = synth.activation(8, 1536, synth.generator(1, 4, 0, 1))
    assert x.dtype == np.float32 and x.shape == (8, 1536)
    big = np.abs(x).mean(axis=0) > 8
    assert big.sum() == 8
    y = synth.activation(8, 1536, synth.generator(1, 4, 0, 1), outliers=0)
    assert (np.abs(y).mean(axis=0) > 8).sum() == 0


def test_stack_shapes():
    s15 = synth.qwen25_1p5b()
    s7 = synth.qwen25_7b()
    assert len(s15) == len(s7) == 197
    assert sum(s.q4_bytes for s in s7) == 3_977_035_776
    assert s15[-1].rows == 151936 and s7[-1].rows == 152064
    assert [s.name for s in s15[:7]] == ["l0.q", "l0.k", "l0.v", "l0.o", "l0.gate", "l0.up",
                                         "l0.down"]
