"""Pins of the oracle's decode attention (minfer README, nano-inference page:
the attention kernels of milestones M5, M12 and M15; the model details give 12
query heads over 2 key/value heads of dimension 128)."""
import numpy as np
import pytest

from conftest import load_golden

GOLD = load_golden("attn_small.txt")[0]


def _rand(L, n_q=12, n_kv=2, hd=128, seed=0, spread=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_q, hd)).astype(np.float32)
    k = (rng.standard_normal((L, n_kv, hd)) * spread).astype(np.float32)
    v = rng.standard_normal((L, n_kv, hd)).astype(np.float32)
    return q, k, v


def test_attn_golden(oracle):
    f = lambda key: np.array([float(t) for t in GOLD[key]], np.float32)
    n_q, n_kv, hd = int(GOLD["n_q"][0]), int(GOLD["n_kv"][0]), int(GOLD["hd"][0])
    q = f("q").reshape(n_q, hd)
    k = f("k").reshape(-1, n_kv, hd)
    v = f("v").reshape(-1, n_kv, hd)
    o, _ = oracle.attn_decode(q, k, v, scale=float(GOLD["scale"][0]))
    assert np.allclose(o.reshape(-1), [float(t) for t in GOLD["o"]], rtol=1e-6, atol=0)


def test_attn_single_position_returns_v(oracle):
    q, k, v = _rand(1, seed=1)
    o, o_abs = oracle.attn_decode(q, k, v)
    for h in range(12):
        assert np.array_equal(o[h], v[0, h // 6].astype(np.float64))
        assert np.array_equal(o_abs[h], np.abs(v[0, h // 6]).astype(np.float64))


def test_attn_equal_keys_average_values(oracle):
    q, k, v = _rand(37, seed=2)
    k[:] = k[0]                                           # every score equal: uniform weights
    o, _ = oracle.attn_decode(q, k, v)
    mean = v.astype(np.float64).mean(axis=0)              # [n_kv][hd]
    for h in range(12):
        assert np.allclose(o[h], mean[h // 6], rtol=1e-12, atol=1e-15)


def test_attn_one_dominant_key_closed_form(oracle):
    L, hd = 9, 128
    q = np.zeros((12, hd), np.float32)
    q[:, 0] = 4.0
    k = np.zeros((L, 2, hd), np.float32)
    k[3, :, 0] = 8.0                                      # score 4*8/sqrt(128) for key 3, 0 for the rest
    rng = np.random.default_rng(3)
    v = rng.standard_normal((L, 2, hd)).astype(np.float32)
    o, _ = oracle.attn_decode(q, k, v)
    d = 32.0 / np.sqrt(128.0)
    p3 = np.exp(d) / (np.exp(d) + (L - 1))
    for h in range(12):
        g = h // 6
        rest = (v[:, g].astype(np.float64).sum(axis=0) - v[3, g]) / (L - 1)
        expect = p3 * v[3, g] + (1 - p3) * rest
        assert np.allclose(o[h], expect, rtol=1e-12, atol=1e-14)


def test_attn_large_scores_stay_finite(oracle):
    # scores of +-2000 overflow exp unless the maximum is subtracted first
    L, hd = 4, 128
    q = np.zeros((12, hd), np.float32)
    q[:, 0] = 100.0
    k = np.zeros((L, 2, hd), np.float32)
    k[:, :, 0] = np.array([-1.0, 2.0, 1.0, 0.0], np.float32)[:, None] * 20.0 * np.sqrt(128.0)
    rng = np.random.default_rng(4)
    v = rng.standard_normal((L, 2, hd)).astype(np.float32)
    o, _ = oracle.attn_decode(q, k, v)
    assert np.all(np.isfinite(o))
    for h in range(12):                                   # key 1 wins by a margin of 2000
        assert np.array_equal(o[h], v[1, h // 6].astype(np.float64))


def test_attn_gqa_groups(oracle):
    # query heads 0-5 read key/value head 0, heads 6-11 head 1
    q, k, v = _rand(20, seed=5)
    v[:, 1] = 0.0
    o, _ = oracle.attn_decode(q, k, v)
    assert np.all(o[6:] == 0.0) and np.all(np.abs(o[:6]).sum(axis=1) > 0)
    q2 = q.copy()
    q2[7] = q2[1]
    k2 = k.copy()
    k2[:, 1] = k2[:, 0]
    v2 = v.copy()
    v2[:, 1] = v2[:, 0]
    o2, _ = oracle.attn_decode(q2, k2, v2)
    assert np.array_equal(o2[7], o2[1])                   # same query, same (copied) kv head


def test_attn_scale_moves_between_query_and_keys(oracle):
    q, k, v = _rand(25, seed=6)
    a, _ = oracle.attn_decode(q, 2 * k, v, scale=0.05)
    b, _ = oracle.attn_decode(q, k, v, scale=0.10)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
    c, _ = oracle.attn_decode(q, k, v)                    # default scale 1/sqrt(hd)
    d, _ = oracle.attn_decode(q, k, v, scale=1 / np.sqrt(128.0))
    assert np.array_equal(c, d)


@pytest.mark.parametrize("L,n_q,n_kv,hd", [(7, 12, 2, 128), (3, 4, 4, 8), (50, 6, 1, 16)])
def test_attn_matches_bruteforce(oracle, L, n_q, n_kv, hd):
    q, k, v = _rand(L, n_q, n_kv, hd, seed=L + hd, spread=2.0)
    o, o_abs = oracle.attn_decode(q, k, v)
    g = n_q // n_kv
    for h in range(n_q):                                  # pure-Python loops, fp64
        kk, vv = k[:, h // g].astype(np.float64), v[:, h // g].astype(np.float64)
        s = [sum(float(q[h, i]) * kk[j, i] for i in range(hd)) / np.sqrt(hd) for j in range(L)]
        m = max(s)
        e = [np.exp(x - m) for x in s]
        p = [x / sum(e) for x in e]
        for i in range(hd):
            assert abs(o[h, i] - sum(p[j] * vv[j, i] for j in range(L))) <= 1e-13 * (1 + abs(o[h, i]))
            assert abs(o_abs[h, i] - sum(p[j] * abs(vv[j, i]) for j in range(L))) <= 1e-13 * (1 + o_abs[h, i])
