"""Grouped K/V heads in the dense layout (fa_forward_gqa / fa_backward_gqa
through the binding): query head h of [B, H, N, D] reads K/V head
h // (H // H_kv) of [B, H_kv, N, D], and dK, dV of a K/V head sum over its
query heads. Every head against the fp64 oracle: a dense batch of B
sequences of N tokens is the packed batch with offsets 0, N, 2N, .., so the
oracle's grouped-head functions (attention_forward_varlen,
attention_backward_varlen) give the reference after a change of layout;
with dropout, the oracle's dropout functions run per query head with that
head's K/V head and random-bit index b * H + h. The bars are the fixed ones
(these are not named workloads, so the max-abs bar widens only where the
reference's own rounding to the dtype exceeds 1e-2: dK and dV of a K/V head
shared by 8 query heads reach magnitudes whose bf16 half-ulp is above it)."""

import numpy as np
import pytest
import torch

import exact_attention_113_amd as fa
import workloads
from gpu_util import assert_close, assert_lse_close, orc, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def packed(t):
    """[B, H, N, D] -> fp64 [B*N, H, D]."""
    B, H, N, D = t.shape
    return to64(t.permute(0, 2, 1, 3).reshape(B * N, H, D))


def dense(x, B, N):
    """fp64 [B*N, H, D] -> [B, H, N, D]."""
    return x.reshape(B, N, x.shape[1], x.shape[2]).transpose(0, 2, 1, 3)


def inputs(B, H, H_kv, N, D, dtype, seed):
    q, do = workloads.make_random((B, H, N, D), seed=seed, dtype=dtype, count=2, device=DEV)
    k, v = workloads.make_random((B, H_kv, N, D), seed=seed + 1, dtype=dtype, count=2,
                                 device=DEV)
    return q, k, v, do


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H_kv", [4, 2, 1])
@pytest.mark.parametrize("causal", [False, True])
def test_forward(dtype, D, H_kv, causal):
    B, H, N = 2, 8, 333
    q, k, v, _ = inputs(B, H, H_kv, N, D, dtype, seed=3000 + D + H_kv)
    scale = D ** -0.5
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    cu = np.arange(B + 1) * N
    ro, rl = orc.attention_forward_varlen(packed(q), packed(k), packed(v), cu, scale, causal)
    name = f"gqa fwd {dtype} D{D} H{H}/{H_kv} causal={causal}"
    assert_close(name + " O", to64(o), dense(ro, B, N), dtype)
    assert_lse_close(name, to64(lse), rl.reshape(H, B, N).transpose(1, 0, 2))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H_kv,N", [(4, 200), (1, 333), (2, 1024)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward(dtype, D, H_kv, N, causal):
    B, H = 2, 8
    q, k, v, do = inputs(B, H, H_kv, N, D, dtype, seed=4000 + D + H_kv + N)
    scale = D ** -0.5
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    cu = np.arange(B + 1) * N
    rq, rk, rv = orc.attention_backward_varlen(packed(q), packed(k), packed(v), packed(do), cu,
                                               scale, causal)
    name = f"gqa bwd {dtype} D{D} H{H}/{H_kv} N{N} causal={causal}"
    assert_close(name + " dQ", to64(dq), dense(rq, B, N), dtype)
    assert_close(name + " dK", to64(dk), dense(rk, B, N), dtype)
    assert_close(name + " dV", to64(dv), dense(rv, B, N), dtype)


def test_groups_of_one_match_the_plain_entry_points_bitwise():
    """H_kv = H through fa_forward_gqa / fa_backward_gqa is the plain path."""
    from exact_attention_113_amd import _lib
    B, H, N, D = 1, 4, 300, 64
    q, k, v, do = inputs(B, H, H, N, D, "bf16", seed=77)
    o, lse = fa.forward(q, k, v, causal=True)
    g = fa.backward(q, k, v, o, lse, do, causal=True)
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    lib = _lib.load()
    st = lib.fa_forward_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(),
                            lse2.data_ptr(), B, H, H, N, D, D ** -0.5, 1, _lib.FA_BF16, 0.0, 0, 0,
                            None)
    assert st == 0
    ws = torch.empty(fa.backward_workspace_bytes(B, H, N, D), dtype=torch.uint8, device=DEV)
    g2 = [torch.empty_like(t) for t in (q, k, v)]
    st = lib.fa_backward_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             do.data_ptr(), lse.data_ptr(), *[t.data_ptr() for t in g2],
                             ws.data_ptr(), ws.numel(), B, H, H, N, D, D ** -0.5, 1,
                             _lib.FA_BF16, 0.0, 0, 0, None)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    for a, b in zip(g, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_dropout(causal):
    B, H, H_kv, N, D = 2, 4, 2, 160, 64
    p, seed, offset = 0.2, 1234, 7
    q, k, v, do = inputs(B, H, H_kv, N, D, "bf16", seed=5000)
    scale = D ** -0.5
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, dropout_p=p, seed=seed,
                        offset=offset)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale, dropout_p=p,
                             seed=seed, offset=offset)
    torch.cuda.synchronize()
    g = H // H_kv
    q64, k64, v64, g64 = (to64(t) for t in (q, k, v, do))
    ro = np.empty_like(q64)
    rl = np.empty((B, H, N))
    rq = np.empty_like(q64)
    rk = np.zeros_like(k64)
    rv = np.zeros_like(v64)
    for b in range(B):
        for h in range(H):
            hk = h // g
            args = (q64[b:b + 1, h:h + 1], k64[b:b + 1, hk:hk + 1], v64[b:b + 1, hk:hk + 1])
            fo, fl = orc.attention_forward_dropout(*args, scale, causal, p, seed, offset,
                                                   bh0=b * H + h)
            bq, bk, bv = orc.attention_backward_dropout(*args, g64[b:b + 1, h:h + 1], scale,
                                                        causal, p, seed, offset, bh0=b * H + h)
            ro[b, h], rl[b, h], rq[b, h] = fo[0, 0], fl[0, 0], bq[0, 0]
            rk[b, hk] += bk[0, 0]
            rv[b, hk] += bv[0, 0]
    name = f"gqa dropout H{H}/{H_kv} causal={causal}"
    assert_close(name + " O", to64(o), ro, "bf16")
    assert_lse_close(name, to64(lse), rl)
    assert_close(name + " dQ", to64(dq), rq, "bf16")
    assert_close(name + " dK", to64(dk), rk, "bf16")
    assert_close(name + " dV", to64(dv), rv, "bf16")
