"""The clock probe (a measurement aid beside the attention path) reports a
plausible shader clock through the C ABI, idle and beside a running
forward."""

import pytest
import torch

import exact_attention_113_amd as fa
from exact_attention_113_amd import _lib
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _probe(side, out, iters=50000):
    with torch.cuda.stream(side):
        _lib.check("fa_clock_probe", _lib.load().fa_clock_probe(out.data_ptr(), iters,
                                                                 side.cuda_stream))
    side.synchronize()
    cycles, ticks = int(out[0].item()), int(out[1].item())
    assert cycles > 0 and ticks > 0
    return cycles / ticks * 100.0


def test_clock_probe_idle_and_beside_a_forward():
    out = torch.zeros(4, dtype=torch.int64, device=DEV)
    side = torch.cuda.Stream()
    idle = _probe(side, out)
    print(f"clock idle {idle:.0f} MHz")
    # The MI355X's shader clock is at most 2.4 GHz; allow for counter jitter.
    assert 500.0 < idle < 2600.0
    q, k, v = workloads.make_random((1, 32, 2048, 128), seed=3, dtype="bf16", count=3, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(1, 32, 2048, dtype=torch.float32, device=DEV)
    for _ in range(30):
        fa.forward(q, k, v, causal=True, out=o, lse=lse)
    busy = _probe(side, out)
    torch.cuda.synchronize()
    print(f"clock beside the forward {busy:.0f} MHz")
    assert 500.0 < busy < 2600.0
