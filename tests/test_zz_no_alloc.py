"""The allocation-free backward (fa_backward_noalloc) through the C ABI
against fa_backward with a caller workspace: two calls in a row on one GPU,
the second smaller (and in the other half-precision type), so the second
runs on the scratch the first left behind. The gradients must be bitwise
those of the workspace entry point (the same kernels on the same inputs)."""

import pytest
import torch

import exact_attention_113_amd as fa
import workloads
from exact_attention_113_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _stream():
    return torch.cuda.current_stream().cuda_stream or None


def _case(B, H, N, D, dtype, causal, seed):
    q, k, v, do = workloads.make_random((B, H, N, D), seed=seed, dtype=dtype, count=4,
                                        device=DEV)
    scale = D ** -0.5
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    ref = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    got = tuple(torch.full_like(q, 3.0) for _ in range(3))
    code = {"bf16": _lib.FA_BF16, "fp16": _lib.FA_FP16}[dtype]
    st = _lib.load().fa_backward_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(), B, H, N, D, scale,
        int(causal), code, _stream())
    assert st == _lib.FA_OK, _lib.last_error()
    torch.cuda.synchronize()
    for tag, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"{tag} differs from fa_backward (B{B} H{H} N{N} D{D})"


def test_two_calls_second_smaller():
    _case(4, 8, 1000, 128, "bf16", True, 4101)
    _case(1, 3, 77, 64, "fp16", False, 4102)


def test_largest_size_and_rejection():
    """2^21 rows (the whole scratch) is accepted; one more row is refused
    with FA_ERR_UNSUPPORTED before anything is launched."""
    B, H, N, D = 1, 256, 8192, 64
    q, k, v, do = workloads.make_random((B, H, N, D), seed=4103, dtype="bf16", count=4,
                                        device=DEV)
    o, lse = fa.forward(q, k, v, causal=True)
    ref = fa.backward(q, k, v, o, lse, do, causal=True)
    got = tuple(torch.empty_like(q) for _ in range(3))
    lib = _lib.load()
    args = [q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
            lse.data_ptr(), got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr()]
    st = lib.fa_backward_noalloc(*args, B, H, N, D, D ** -0.5, 1, _lib.FA_BF16, _stream())
    assert st == _lib.FA_OK, _lib.last_error()
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    st = lib.fa_backward_noalloc(*args, B, H, N + 1, D, D ** -0.5, 1, _lib.FA_BF16, _stream())
    assert st == _lib.FA_ERR_UNSUPPORTED
    assert "scratch" in _lib.last_error()
