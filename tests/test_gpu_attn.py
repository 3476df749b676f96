"""GPU parity of decode attention (split-KV partials + combine) against the
fp64 oracle.  Tolerance: |o - o_exact| <= 1e-4 * sum_j p_j |v_j| elementwise.
Derivation: the fp32 score of 128 products carries at most ~34 * 2^-24 of
scale * sum_d |q_d k_d| (about 2e-5 for unit-normal data at 1/sqrt(128)); a
score error e changes each weight p_j by a factor exp(+-e), and expf, the
64-term split sums and the combine over up to 512 splits add a few 1e-6 more.
Every call goes through the C ABI of libq4stream."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, require_gpu, to_dev
from q4_weight_streaming_amd import _lib as q

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _cache(L, n_q, n_kv, seed, spread=1.0):
    rng = np.random.default_rng(seed)
    qv = rng.standard_normal((n_q, 128)).astype(np.float32)
    k = (rng.standard_normal((L, n_kv, 128)) * spread).astype(np.float32)
    v = rng.standard_normal((L, n_kv, 128)).astype(np.float32)
    return qv, k, v


def _gpu_layout(k, v, pad):
    """Canonical [L][n_kv][128] -> k_blk [n_kv][l_cap/64][128][64], v [n_kv][l_cap][128], l_cap = L
    rounded up to 64 plus `pad` blocks' worth of positions; NaN past L (byte moves only)."""
    L, n_kv, _ = k.shape
    l_cap = (L + 63) // 64 * 64 + 64 * pad
    kb = np.full((n_kv, l_cap, 128), np.nan, np.float32)
    kb[:, :L] = k.transpose(1, 0, 2)
    kb = np.ascontiguousarray(kb.reshape(n_kv, l_cap // 64, 64, 128).transpose(0, 1, 3, 2))
    vp = np.full((n_kv, l_cap, 128), np.nan, np.float32)
    vp[:, :L] = v.transpose(1, 0, 2)
    return to_dev(kb), to_dev(vp)


def _run(qv, k, v, pad=1):
    kt, vp = _gpu_layout(k, v, pad)
    return q.attn_decode(to_dev(qv), kt, vp, k.shape[0]).cpu().numpy()


def _check(o, oracle_out):
    o64, oabs = oracle_out
    err = np.abs(o.astype(np.float64) - o64)
    assert np.all(np.isfinite(o))
    assert np.all(err <= 1e-4 * oabs + 1e-30), float((err / np.maximum(oabs, 1e-300)).max())


@pytest.mark.parametrize("L", [1, 5, 63, 64, 65, 200, 1000, 4097])
@pytest.mark.parametrize("n_q,n_kv", [(12, 2), (4, 4), (8, 1), (14, 2)])
def test_attn_matches_oracle(oracle, L, n_q, n_kv):
    qv, k, v = _cache(L, n_q, n_kv, seed=L * 31 + n_q)
    _check(_run(qv, k, v), oracle.attn_decode(qv, k, v))


def test_attn_full_context(oracle):
    # Qwen2.5-1.5B heads at the 32768-position context
    qv, k, v = _cache(32768, 12, 2, seed=7)
    _check(_run(qv, k, v, pad=0), oracle.attn_decode(qv, k, v))


@pytest.mark.parametrize("L,n_q,n_kv", [(40000, 2, 1), (70001, 4, 2)])
def test_attn_beyond_one_combine_batch(oracle, L, n_q, n_kv):
    # more than 512 splits: each of the combine's 64 slices takes its splits in several load batches
    qv, k, v = _cache(L, n_q, n_kv, seed=L + n_q)
    _check(_run(qv, k, v), oracle.attn_decode(qv, k, v))


def test_attn_peaked_scores(oracle):
    qv, k, v = _cache(3000, 12, 2, seed=8, spread=4.0)     # sharper softmax
    _check(_run(qv, k, v), oracle.attn_decode(qv, k, v))


def test_attn_one_position_is_exact():
    qv, k, v = _cache(1, 12, 2, seed=9)
    o = _run(qv, k, v)
    for h in range(12):
        assert np.array_equal(o[h], v[0, h // 6])


def test_attn_dominant_position_is_exact():
    # one position wins by a score margin of ~2000: every other weight is exp(-2000) = 0
    L = 700
    qv = np.zeros((12, 128), np.float32)
    qv[:, 0] = 100.0
    rng = np.random.default_rng(10)
    k = rng.uniform(-1, 1, (L, 2, 128)).astype(np.float32)
    k[:, :, 0] = 0.0
    k[333, :, 0] = 20.0 * np.sqrt(128.0)
    v = rng.standard_normal((L, 2, 128)).astype(np.float32)
    o = _run(qv, k, v)
    for h in range(12):
        assert np.array_equal(o[h], v[333, h // 6])


def test_attn_deterministic():
    qv, k, v = _cache(5000, 12, 2, seed=11)
    kt, vp = _gpu_layout(k, v, 0)
    a = q.attn_decode(to_dev(qv), kt, vp, 5000)
    b = q.attn_decode(to_dev(qv), kt, vp, 5000)
    assert torch.equal(a, b)
