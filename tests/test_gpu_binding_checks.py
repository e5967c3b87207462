"""Wrong caller buffers are rejected by every Python entry point before a
kernel is launched (ValueError), so no kernel can write past them."""

import pytest
import torch

import exact_attention_113_amd as fa
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _dense():
    return workloads.make_random((1, 2, 64, 64), seed=1, dtype="bf16", count=4, device=DEV)


def test_forward_rejects_wrong_out_and_lse():
    q, k, v, _ = _dense()
    bad_out = [torch.empty(1, 2, 63, 64, dtype=torch.bfloat16, device=DEV),
               torch.empty(1, 2, 64, 64, dtype=torch.float16, device=DEV),
               torch.empty(1, 2, 64, 64, dtype=torch.bfloat16)]
    for o in bad_out:
        with pytest.raises(ValueError):
            fa.forward(q, k, v, out=o)
    bad_lse = [torch.empty(1, 2, 63, dtype=torch.float32, device=DEV),
               torch.empty(1, 2, 64, dtype=torch.float16, device=DEV),
               torch.empty(1, 2, 64, dtype=torch.float32)]
    for lse in bad_lse:
        with pytest.raises(ValueError):
            fa.forward(q, k, v, lse=lse)


def test_backward_rejects_wrong_lse_and_workspace():
    q, k, v, do = _dense()
    o, lse = fa.forward(q, k, v, causal=True)
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse.cpu(), do, causal=True)
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse[:, :, :-1], do, causal=True)
    need = fa.backward_workspace_bytes(1, 2, 64, 64)
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse, do, causal=True,
                    workspace=torch.empty(need - 1, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        fa.backward(q, k, v, o, lse, do, causal=True,
                    out=(torch.empty_like(q), torch.empty_like(k),
                         torch.empty(1, 2, 64, 32, dtype=torch.bfloat16, device=DEV)))
    torch.cuda.synchronize()


def test_varlen_rejects_wrong_out_lse_and_offsets():
    total, H, Hkv, D = 50, 4, 2, 64
    g = torch.Generator().manual_seed(2)
    q = torch.randn(total, H, D, generator=g).to(torch.bfloat16).to(DEV)
    k = torch.randn(total, Hkv, D, generator=g).to(torch.bfloat16).to(DEV)
    v = torch.randn(total, Hkv, D, generator=g).to(torch.bfloat16).to(DEV)
    cu = torch.tensor([0, 20, 50], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        fa.forward_varlen(q, k, v, cu, 30, out=torch.empty(total - 1, H, D, dtype=q.dtype,
                                                          device=DEV))
    with pytest.raises(ValueError):
        fa.forward_varlen(q, k, v, cu, 30, lse=torch.empty(total, H, dtype=torch.float32,
                                                          device=DEV))
    with pytest.raises(ValueError):
        fa.forward_varlen(q, k, v, cu.cpu(), 30)


def test_decode_rejects_wrong_out_lse_and_workspace():
    B, s_q, H, Hkv, cap, D = 2, 1, 8, 2, 2048, 128
    g = torch.Generator().manual_seed(3)
    q = torch.randn(B, s_q, H, D, generator=g).to(torch.bfloat16).to(DEV)
    kc = torch.randn(B, cap, Hkv, D, generator=g).to(torch.bfloat16).to(DEV)
    vc = torch.randn(B, cap, Hkv, D, generator=g).to(torch.bfloat16).to(DEV)
    lens = torch.tensor([2000, 100], dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        fa.decode(q, kc, vc, lens, out=torch.empty(B, s_q, H, 64, dtype=q.dtype, device=DEV))
    with pytest.raises(ValueError):
        fa.decode(q, kc, vc, lens, lse=torch.empty(B, s_q, H, dtype=torch.float32, device=DEV))
    need = fa.decode_workspace_bytes(B, s_q, H, Hkv, cap, D)
    assert need > 0
    with pytest.raises(ValueError):
        fa.decode(q, kc, vc, lens, workspace=torch.empty(need - 1, dtype=torch.uint8,
                                                         device=DEV))
    with pytest.raises(ValueError):
        fa.decode(q, kc, vc, lens.cpu())
