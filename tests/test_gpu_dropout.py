"""Attention dropout on the GPU against the fp64 oracle: the keep decisions
themselves, forward and backward parity, the p = 0 path, repeatability, and
a sampled head of the training shape."""

import numpy as np
import pytest
import torch

import exact_attention_113_amd as fa
import oracle.attention as orc
import oracle.rng as rng
import workloads
from gpu_util import assert_close, assert_lse_close, compare_heads, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def rand(shape, seed, dtype="bf16", count=3):
    return workloads.make_random(shape, seed=seed, dtype=dtype, count=count, device=DEV)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pr", [0.1, 0.5])
def test_keep_decisions_exact(causal, pr):
    """V = identity: O[i, j] = P[i, j] / (1 - p') where kept and 0 where
    dropped, so the zero pattern of O is the keep mask; it must equal the
    oracle's bit for bit (two heads, 64 rows crossing 4x4 block edges)."""
    B, H, N, D = 1, 2, 64, 64
    q, k, _ = rand((B, H, N, D), 11)
    v = torch.eye(N, D, dtype=torch.bfloat16, device=DEV).expand(B, H, N, D).contiguous()
    o, _ = fa.forward(q, k, v, causal=causal, scale=0.02, dropout_p=pr, seed=77, offset=3)
    torch.cuda.synchronize()
    got = (o != 0).cpu().numpy()
    for h in range(H):
        keep = rng.keep_mask(h, np.arange(N), np.arange(N), pr, 77, 3)
        if causal:
            keep &= np.tril(np.ones((N, N), dtype=bool))
        assert np.array_equal(got[0, h], keep), f"head {h}: keep mask differs"


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [77, 300])
def test_forward_dropout(dtype, D, causal, N):
    B, H = 2, 2
    q, k, v = rand((B, H, N, D), 100 + N + D, dtype)
    seed = 0x0123_4567_89AB_CDEF
    o, lse = fa.forward(q, k, v, causal=causal, scale=D ** -0.5, dropout_p=0.3, seed=seed,
                        offset=9)
    torch.cuda.synchronize()
    ro, rl = orc.attention_forward_dropout(to64(q), to64(k), to64(v), D ** -0.5, causal, 0.3,
                                           seed, 9)
    assert_close(f"dropout fwd {dtype} D{D} N{N} causal={causal}", to64(o), ro, dtype)
    assert_lse_close("dropout lse", to64(lse), rl)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_backward_dropout(causal, D):
    B, H, N = 1, 2, 300
    q, k, v, do = rand((B, H, N, D), 200 + D, count=4)
    kw = dict(causal=causal, scale=D ** -0.5, dropout_p=0.25, seed=31337, offset=1)
    o, lse = fa.forward(q, k, v, **kw)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    rq, rk, rv = orc.attention_backward_dropout(to64(q), to64(k), to64(v), to64(do), D ** -0.5,
                                                causal, 0.25, 31337, 1)
    for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        assert_close(f"dropout {name} D{D} causal={causal}", to64(g), r, "bf16")


def test_below_half_a_step_is_the_plain_path():
    """p below 0.5/256 rounds to no dropout: bit-identical to fa.forward."""
    q, k, v = rand((1, 4, 200, 128), 5)
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2, l2 = fa.forward(q, k, v, causal=True, dropout_p=0.001, seed=5)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_repeatable_and_offset_changes_bits():
    q, k, v, do = rand((1, 2, 256, 128), 6, count=4)
    kw = dict(causal=True, dropout_p=0.2, seed=1)
    o1, l1 = fa.forward(q, k, v, **kw, offset=0)
    o2, _ = fa.forward(q, k, v, **kw, offset=0)
    o3, _ = fa.forward(q, k, v, **kw, offset=1)
    g1 = fa.backward(q, k, v, o1, l1, do, **kw, offset=0)
    g2 = fa.backward(q, k, v, o1, l1, do, **kw, offset=0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert not torch.equal(o1, o3)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.timeout(900)
def test_training_shape_heads():
    """The training shape (B4 H16 N8192 D128 causal) with p = 0.1: every one
    of the 64 heads, forward and gradients against the oracle at full
    length."""
    w = workloads.bf16_training()
    q, k, v, do = workloads.make_inputs(w, device=DEV)
    kw = dict(causal=True, scale=w.scale, dropout_p=0.1, seed=2024, offset=7)
    o, lse = fa.forward(q, k, v, **kw)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def fwd(q1, k1, v1, head):
        return orc.attention_forward_dropout(q1, k1, v1, w.scale, True, 0.1, 2024, 7,
                                             bh0=head[0] * w.H + head[1])

    def bwd(q1, k1, v1, do1, head):
        return orc.attention_backward_dropout(q1, k1, v1, do1, w.scale, True, 0.1, 2024, 7,
                                              bh0=head[0] * w.H + head[1])

    compare_heads("train dropout", (q, k, v), fwd, [("O", o, 0)], "bf16", heads,
                  lse=(lse, 1), pass_head=True)
    compare_heads("train dropout", (q, k, v, do), bwd,
                  [("dQ", dq, 0), ("dK", dk, 1), ("dV", dv, 2)], "bf16", heads, pass_head=True)


@pytest.mark.parametrize("causal", [False, True])
def test_forward_dropout_large_grid_d64(causal):
    """D = 64 with dropout on a grid of 512 256-row tiles (the forward path that
    keeps four K and four V tiles and synchronises once per two tiles), with a
    ragged last tile: two heads against the oracle, whose bits are keyed by
    each head's own (batch, head) index."""
    B, H, N, D = 8, 16, 1000, 64
    q, k, v = rand((B, H, N, D), 4242 + int(causal))
    kw = dict(causal=causal, scale=0.125, dropout_p=0.2, seed=77, offset=3)
    o, lse = fa.forward(q, k, v, **kw)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (B - 1, H - 3)]:
        sl = lambda t: to64(t[b:b + 1, h:h + 1])
        ro, rl = orc.attention_forward_dropout(sl(q), sl(k), sl(v), 0.125, causal, 0.2, 77, 3,
                                               bh0=b * H + h)
        assert_close(f"dropout D64 large grid causal={causal} ({b},{h})", sl(o), ro, "bf16")
        assert_lse_close("dropout D64 large grid", sl(lse), rl)
