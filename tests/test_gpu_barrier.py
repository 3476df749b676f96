"""The grid-barrier measurement kernel completes every phase on the GPU (its
bounded poll never gives up when all workgroups are resident)."""
import pytest
import torch

from gpu_helpers import dev, require_gpu
from q4_weight_streaming_amd import _lib as q

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", list(range(10)))
@pytest.mark.parametrize("frac", [1, 4])
def test_grid_barrier_completes(kind, frac):
    require_gpu()
    n = q.grid_barrier_max_workgroups() // frac
    assert n >= 64
    scratch = torch.full((q.grid_barrier_scratch_bytes(n) // 4,), 7, dtype=torch.int32, device=dev())
    q.bench_grid_barrier(kind, n, 200, scratch)
    torch.cuda.synchronize()
    w = scratch.cpu()
    assert w[1].item() == 0                                    # nobody gave up waiting
    lines = w[64:32 * (n + 2)].view(n, 32)[:, 0]
    if kind in (0, 3, 9):
        assert w[0].item() == 200 * n                          # every arrival counted
    elif kind == 1:
        assert w[0].item() == 200                              # the last release
        assert (lines == 200).all()                            # every workgroup's last phase
    elif kind in (2, 7, 8):
        fan = min(16, n)
        assert w[0].item() == 200 and w[32].item() == 200 * fan
        assert lines[:fan].sum().item() == 200 * n             # every arrival counted once
    else:
        fan = min(16, n)
        slot = {4: 256, 5: 1024, 6: 16384}[kind]
        slots = w[64:64 + 16 * slot].view(16, slot)[:fan]
        assert w[32].item() == 200 * fan
        assert slots[:, 0].sum().item() == 200 * n            # every arrival counted once
        assert (slots[:, 32] == 200).all()                     # every release copy stored
