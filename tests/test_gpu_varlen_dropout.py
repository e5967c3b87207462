"""Dropout on packed variable-length batches with grouped K/V heads
(fa_forward_varlen_dropout / fa_backward_varlen_dropout through the
binding) against the fp64 oracle: each (sequence b, query head h) is
attention_forward_dropout / attention_backward_dropout on that sequence's
rows with K/V head h // (H // H_kv) and the random bits of head b * H + h
(rows and keys counted from the sequence's first token); dK and dV of a K/V
head sum over its query heads. Also: a packed batch of equal lengths gives
the dense dropout results bit for bit."""

import numpy as np
import pytest
import torch

import exact_attention_113_amd as fa
import oracle.attention as orc
import workloads
from gpu_util import assert_close, assert_lse_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
P, SEED, OFFSET = 0.2, 987654321, 3


def packed(lengths, H, H_kv, D, seed):
    total = sum(lengths)
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn((total, H, D), generator=g).to(torch.bfloat16)
    k = torch.randn((total, H_kv, D), generator=g).to(torch.bfloat16)
    v = torch.randn((total, H_kv, D), generator=g).to(torch.bfloat16)
    do = torch.randn((total, H, D), generator=g).to(torch.bfloat16)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    return q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), cu


def oracle(q, k, v, do, cu, scale, causal):
    q, k, v, do = (to64(t) for t in (q, k, v, do))
    total, H, D = q.shape
    g = H // k.shape[1]
    o, dq = np.zeros_like(q), np.zeros_like(q)
    dk, dv = np.zeros_like(k), np.zeros_like(v)
    lse = np.zeros((H, total))
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        if s1 <= s0:
            continue
        for h in range(H):
            hk = h // g
            args = [t[s0:s1, c][None, None] for t, c in ((q, h), (k, hk), (v, hk))]
            fo, fl = orc.attention_forward_dropout(*args, scale, causal, P, SEED, OFFSET,
                                                   bh0=b * H + h)
            bq, bk, bv = orc.attention_backward_dropout(*args, do[s0:s1, h][None, None], scale,
                                                        causal, P, SEED, OFFSET, bh0=b * H + h)
            o[s0:s1, h], lse[h, s0:s1], dq[s0:s1, h] = fo[0, 0], fl[0, 0], bq[0, 0]
            dk[s0:s1, hk] += bk[0, 0]
            dv[s0:s1, hk] += bv[0, 0]
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H_kv", [4, 1])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_dropout(D, H_kv, causal):
    lengths = [1, 7, 0, 65, 300, 129]
    q, k, v, do, cu = packed(lengths, 4, H_kv, D, seed=800 + D + H_kv)
    scale = D ** -0.5
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    kw = dict(causal=causal, scale=scale, dropout_p=P, seed=SEED, offset=OFFSET)
    o, lse = fa.forward_varlen(q, k, v, cu_t, max(lengths), **kw)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, lse, do, cu_t, max(lengths), **kw)
    torch.cuda.synchronize()
    ro, rl, rq, rk, rv = oracle(q, k, v, do, cu, scale, causal)
    name = f"packed dropout D{D} H4/{H_kv} causal={causal}"
    assert_close(name + " O", to64(o), ro, "bf16")
    assert_lse_close(name, to64(lse), rl)
    assert_close(name + " dQ", to64(dq), rq, "bf16")
    assert_close(name + " dK", to64(dk), rk, "bf16")
    assert_close(name + " dV", to64(dv), rv, "bf16")


def test_equal_lengths_match_dense_dropout_bitwise():
    B, H, N, D = 2, 4, 200, 128
    q, k, v = workloads.make_random((B, H, N, D), seed=61, dtype="bf16", device=DEV)
    do = workloads.make_random((B, H, N, D), seed=62, dtype="bf16", count=1, device=DEV)[0]
    kw = dict(causal=True, scale=D ** -0.5, dropout_p=P, seed=SEED, offset=OFFSET)
    o, lse = fa.forward(q, k, v, **kw)
    g = fa.backward(q, k, v, o, lse, do, **kw)

    def pk(t):
        return t.permute(0, 2, 1, 3).reshape(B * N, H, D).contiguous()
    cu = torch.tensor([0, N, 2 * N], dtype=torch.int32, device=DEV)
    op, lp = fa.forward_varlen(pk(q), pk(k), pk(v), cu, N, **kw)
    gp = fa.backward_varlen(pk(q), pk(k), pk(v), op, lp, pk(do), cu, N, **kw)
    torch.cuda.synchronize()
    assert torch.equal(op, pk(o))
    assert torch.equal(lp, lse.permute(1, 0, 2).reshape(H, B * N))
    for a, b in zip(gp, g):
        assert torch.equal(a, pk(b))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H_kv", [8, 2])
@pytest.mark.parametrize("causal", [False, True])
def test_packed_dropout_whole_batch_order(D, H_kv, causal):
    """Eight query heads: the forward's grid of only real tiles, heaviest
    first over the batch, and (full attention, unit-major grids) the
    backward's grids of only real tiles, with dropout."""
    lengths = [1, 7, 0, 65, 300, 129, 700]
    q, k, v, do, cu = packed(lengths, 8, H_kv, D, seed=820 + D + H_kv + int(causal))
    scale = D ** -0.5
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    kw = dict(causal=causal, scale=scale, dropout_p=P, seed=SEED, offset=OFFSET)
    o, lse = fa.forward_varlen(q, k, v, cu_t, max(lengths), **kw)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, lse, do, cu_t, max(lengths), **kw)
    torch.cuda.synchronize()
    ro, rl, rq, rk, rv = oracle(q, k, v, do, cu, scale, causal)
    name = f"packed dropout D{D} H8/{H_kv} causal={causal}"
    assert_close(name + " O", to64(o), ro, "bf16")
    assert_lse_close(name, to64(lse), rl)
    assert_close(name + " dQ", to64(dq), rq, "bf16")
    assert_close(name + " dK", to64(dk), rk, "bf16")
    assert_close(name + " dV", to64(dv), rv, "bf16")


def test_equal_lengths_match_dense_dropout_bitwise_eight_heads():
    """The same with eight heads and full attention, where the packed grids
    hold only real tiles (forward and both backward kernels)."""
    B, H, N, D = 2, 8, 600, 128
    q, k, v = workloads.make_random((B, H, N, D), seed=63, dtype="bf16", device=DEV)
    do = workloads.make_random((B, H, N, D), seed=64, dtype="bf16", count=1, device=DEV)[0]
    kw = dict(causal=False, scale=D ** -0.5, dropout_p=P, seed=SEED, offset=OFFSET)
    o, lse = fa.forward(q, k, v, **kw)
    g = fa.backward(q, k, v, o, lse, do, **kw)

    def pk(t):
        return t.permute(0, 2, 1, 3).reshape(B * N, H, D).contiguous()
    cu = torch.tensor([0, N, 2 * N], dtype=torch.int32, device=DEV)
    op, lp = fa.forward_varlen(pk(q), pk(k), pk(v), cu, N, **kw)
    gp = fa.backward_varlen(pk(q), pk(k), pk(v), op, lp, pk(do), cu, N, **kw)
    torch.cuda.synchronize()
    assert torch.equal(op, pk(o))
    assert torch.equal(lp, lse.permute(1, 0, 2).reshape(H, B * N))
    for a, b in zip(gp, g):
        assert torch.equal(a, pk(b))
