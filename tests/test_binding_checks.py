"""The binding's checks on caller-supplied buffers (host logic, no GPU):
a tensor handed to a kernel as a raw pointer must have the expected shape,
dtype, device and layout, and a workspace enough bytes, or the call raises
before anything is launched."""

import pytest
import torch

import exact_attention_113_amd as fa

CPU = torch.device("cpu")


def test_buffer_accepted():
    fa._check_buffer("out", torch.empty(2, 3, 5, 64), (2, 3, 5, 64), torch.float32, CPU)


@pytest.mark.parametrize("bad, why", [
    (torch.empty(2, 3, 4, 64), "shape"),
    (torch.empty(2, 3, 5, 64, dtype=torch.float16), "dtype"),
    (torch.empty(2, 3, 64, 5).transpose(2, 3), "contiguous"),
    (torch.empty(2 * 3 * 5 * 64), "shape"),
])
def test_buffer_rejected(bad, why):
    with pytest.raises(ValueError, match=why):
        fa._check_buffer("out", bad, (2, 3, 5, 64), torch.float32, CPU)


def test_buffer_wrong_device():
    with pytest.raises(ValueError, match="must be on"):
        fa._check_buffer("lse", torch.empty(2, 3, 5), (2, 3, 5), torch.float32,
                         torch.device("cuda:0"))


def test_buffer_not_a_tensor():
    with pytest.raises(TypeError):
        fa._check_buffer("lse", None, (2, 3, 5), torch.float32, CPU)


def test_workspace_checks():
    fa._check_workspace("ws", torch.empty(100, dtype=torch.uint8), 100, CPU)
    with pytest.raises(ValueError, match="bytes"):
        fa._check_workspace("ws", torch.empty(99, dtype=torch.uint8), 100, CPU)
    with pytest.raises(ValueError, match="uint8"):
        fa._check_workspace("ws", torch.empty(100, dtype=torch.float32), 100, CPU)
    with pytest.raises(ValueError, match="uint8"):
        fa._check_workspace("ws", torch.empty(10, 10, dtype=torch.uint8), 100, CPU)


@pytest.mark.parametrize("k_heads", [0, 3, 16])
def test_grouped_heads_must_divide(k_heads):
    """k and v may have H_kv heads only when H_kv divides H (checked before
    any device or library call)."""
    q = torch.zeros((1, 8, 16, 64))
    k = torch.zeros((1, k_heads, 16, 64))
    with pytest.raises(ValueError, match="H_kv"):
        fa.forward(q, k, k.clone())
    with pytest.raises(ValueError, match="H_kv"):
        fa.backward(q, k, k.clone(), q, torch.zeros((1, 8, 16)), q)


def test_grouped_heads_need_equal_k_and_v():
    q = torch.zeros((1, 8, 16, 64))
    with pytest.raises(ValueError):
        fa.forward(q, torch.zeros((1, 2, 16, 64)), torch.zeros((1, 4, 16, 64)))
    with pytest.raises(ValueError):
        fa.forward(q, torch.zeros((1, 2, 8, 64)), torch.zeros((1, 2, 8, 64)))
