"""The allocation-free decode attention (q4s_attn_decode_noalloc: split partials in the
library's static per-GPU scratch array) against q4s_attn_decode with a caller workspace:
bit-identical outputs on two calls in a row, the second smaller than the first, and
within the attention tolerance of the fp64 oracle (|o - o_exact| <= 1e-4 * sum_j p_j |v_j|,
derived in test_gpu_attn.py).  Every call goes through the C ABI of libq4stream."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, require_gpu, to_dev
from q4_weight_streaming_amd import _lib as q

pytestmark = pytest.mark.gpu


def _inputs(L, n_q, n_kv, seed):
    rng = np.random.default_rng(seed)
    qv = rng.standard_normal((n_q, 128)).astype(np.float32)
    k = rng.standard_normal((L, n_kv, 128)).astype(np.float32)
    v = rng.standard_normal((L, n_kv, 128)).astype(np.float32)
    l_cap = (L + 63) // 64 * 64
    kb = np.zeros((n_kv, l_cap, 128), np.float32)
    kb[:, :L] = k.transpose(1, 0, 2)
    kb = np.ascontiguousarray(kb.reshape(n_kv, l_cap // 64, 64, 128).transpose(0, 1, 3, 2))
    vp = np.zeros((n_kv, l_cap, 128), np.float32)
    vp[:, :L] = v.transpose(1, 0, 2)
    return (qv, k, v), (to_dev(qv), to_dev(kb), to_dev(vp))


def test_noalloc_matches_workspace_entry_point(oracle):
    require_gpu()
    # the first call fills far more of the scratch than the second, so stale partials
    # of the first would show in the second
    for L, n_q, n_kv, seed in [(32768, 12, 2, 11), (1000, 12, 2, 12), (65, 8, 1, 13)]:
        print(f"noalloc attention L={L} n_q={n_q} n_kv={n_kv}", flush=True)
        host, (qd, kd, vd) = _inputs(L, n_q, n_kv, seed)
        ref = q.attn_decode(qd, kd, vd, L)
        got = torch.full((n_q, 128), float("nan"), dtype=torch.float32, device=dev())
        q.attn_decode_noalloc(qd, kd, vd, L, out=got)
        torch.cuda.synchronize()
        r, g = ref.cpu().numpy(), got.cpu().numpy()
        assert np.array_equal(r.view(np.uint32), g.view(np.uint32)), "differs from q4s_attn_decode"
        o64, oabs = oracle.attn_decode(*host)
        assert np.all(np.abs(g.astype(np.float64) - o64) <= 1e-4 * oabs + 1e-30)


def test_noalloc_rejects_beyond_scratch():
    require_gpu()
    n_q, n_kv = 12, 2
    L = 86016 + 64                    # one split more than the 8 MiB scratch holds for 12 heads
    assert q.attn_workspace_bytes(n_q, L) > q.ATTN_SCRATCH_BYTES >= q.attn_workspace_bytes(n_q, L - 64)
    qd = torch.zeros((n_q, 128), dtype=torch.float32, device=dev())
    kd = torch.zeros((n_kv, L // 64, 128, 64), dtype=torch.float32, device=dev())
    vd = torch.zeros((n_kv, L, 128), dtype=torch.float32, device=dev())
    out = torch.zeros((n_q, 128), dtype=torch.float32, device=dev())
    with pytest.raises(q.Q4SError) as e:
        q.attn_decode_noalloc(qd, kd, vd, L, out=out)
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert not out.any()              # nothing was enqueued
