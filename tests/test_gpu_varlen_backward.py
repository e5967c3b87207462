"""Backward of packed variable-length batches with grouped K/V heads on the
GPU against the fp64 oracle's exact gradients (each sequence and query head
its own problem; a shared K/V head's gradients summed over its group)."""

import numpy as np
import pytest
import torch

import exact_attention_113_amd as fa
import oracle.attention as orc
import workloads
from gpu_util import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def packed(lengths, H, H_kv, D, dtype, seed, extra=0):
    """Packed q, k, v, dO for the given lengths (plus `extra` tokens after
    the last sequence, covered by none) and the offsets."""
    total = sum(lengths) + extra
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    q = torch.randn((total, H, D), generator=g).to(td)
    k = torch.randn((total, H_kv, D), generator=g).to(td)
    v = torch.randn((total, H_kv, D), generator=g).to(td)
    do = torch.randn((total, H, D), generator=g).to(td)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    return q.to(DEV), k.to(DEV), v.to(DEV), do.to(DEV), cu


def run(q, k, v, do, cu, causal, scale, out=None):
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    n_max = max(max(b - a for a, b in zip(cu[:-1], cu[1:])), 1)
    o, lse = fa.forward_varlen(q, k, v, cu_t, n_max, causal=causal, scale=scale)
    grads = fa.backward_varlen(q, k, v, o, lse, do, cu_t, n_max, causal=causal, scale=scale,
                               out=out)
    torch.cuda.synchronize()
    return grads


def covered_rows(cu, total):
    m = np.zeros(total, dtype=bool)
    for a, b in zip(cu[:-1], cu[1:]):
        m[a:b] = True
    return m


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H_kv", [4, 2, 1])
def test_ragged_packed_gqa(dtype, D, causal, H_kv):
    lengths = [1, 7, 0, 65, 300, 129, 256]
    q, k, v, do, cu = packed(lengths, 4, H_kv, D, dtype, seed=700 + D + H_kv)
    scale = D ** -0.5
    dq, dk, dv = run(q, k, v, do, cu, causal, scale)
    ref = orc.attention_backward_varlen(to64(q), to64(k), to64(v), to64(do), cu, scale, causal)
    m = covered_rows(cu, q.shape[0])
    name = f"{dtype} D{D} causal={causal} H4/{H_kv}"
    for tag, got, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(f"{name} {tag}", to64(got)[m], r[m], dtype)


def test_uncovered_rows_untouched_and_scale_sign():
    """Tokens after the last sequence keep the caller's values; a negative
    scale takes the sign-flipped path of both kernels."""
    lengths = [200, 33]
    q, k, v, do, cu = packed(lengths, 4, 2, 64, "bf16", seed=711, extra=50)
    sentinel = 7.0
    out = tuple(torch.full_like(t, sentinel) for t in (q, k, v))
    dq, dk, dv = run(q, k, v, do, cu, True, -0.2, out=out)
    ref = orc.attention_backward_varlen(to64(q), to64(k), to64(v), to64(do), cu, -0.2, True)
    m = covered_rows(cu, q.shape[0])
    for tag, got, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert_close(f"scale=-0.2 {tag}", to64(got)[m], r[m], "bf16")
        assert bool((got[~torch.from_numpy(m).to(DEV)] == sentinel).all()), tag


def test_equal_lengths_match_dense_bitwise():
    """Equal-length sequences with H_kv = H run the dense entry point's
    arithmetic in the same order: gradients agree bit for bit."""
    B, H, N, D = 3, 4, 333, 128
    q, k, v, do = workloads.make_random((B, H, N, D), seed=53, dtype="bf16", count=4, device=DEV)
    o, lse = fa.forward(q, k, v, causal=True, scale=0.1)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=True, scale=0.1)
    pk = [t.permute(0, 2, 1, 3).reshape(B * N, H, D).contiguous() for t in (q, k, v, do)]
    cu = [0, N, 2 * N, 3 * N]
    g = run(*pk, cu, True, 0.1)
    torch.cuda.synchronize()
    for tag, a, b in zip(("dQ", "dK", "dV"), g, (dq, dk, dv)):
        assert torch.equal(a, b.permute(0, 2, 1, 3).reshape(B * N, H, D)), tag


def test_gqa_against_repeated_heads():
    """Grouped heads: dQ is bitwise that of the kernel run with each K/V head
    repeated over its group; dK and dV equal the group sums of the repeated
    run's per-head gradients to rounding."""
    lengths = [513, 96, 1000]
    q, k, v, do, cu = packed(lengths, 8, 2, 128, "bf16", seed=713)
    dq, dk, dv = run(q, k, v, do, cu, True, 0.09)
    ke = k.repeat_interleave(4, dim=1).contiguous()
    ve = v.repeat_interleave(4, dim=1).contiguous()
    dq2, dk2, dv2 = run(q, ke, ve, do, cu, True, 0.09)
    assert torch.equal(dq, dq2)
    for tag, got, rep in (("dK", dk, dk2), ("dV", dv, dv2)):
        summed = rep.double().reshape(rep.shape[0], 2, 4, -1).sum(dim=2)
        assert_close(f"group sum {tag}", to64(got), summed.cpu().numpy(), "bf16")


def test_prefill_batch_workload_sampled():
    """The packed prefill batch (16 sequences of 256..4096 tokens, 32 query
    over 8 K/V heads, causal): sampled (sequence, K/V head) gradients, with
    the dQ of the group's query heads, against the oracle at the full size."""
    w = workloads.varlen_gqa()
    q, k, v, cu_t, do = workloads.make_varlen_inputs(w, device=DEV, grad=True)
    cu = w.cu_seqlens()
    n_max = max(w.lengths)
    o, lse = fa.forward_varlen(q, k, v, cu_t, n_max, causal=True, scale=w.scale)
    dq, dk, dv = fa.backward_varlen(q, k, v, o, lse, do, cu_t, n_max, causal=True,
                                    scale=w.scale)
    torch.cuda.synchronize()
    G = w.H // w.H_kv
    for b, hk in [(6, 3), (3, 7), (0, 0)]:
        s0, s1 = cu[b], cu[b + 1]
        hs = slice(hk * G, hk * G + G)
        rq, rk, rv = orc.attention_backward_varlen(
            to64(q[s0:s1, hs]), to64(k[s0:s1, hk:hk + 1]), to64(v[s0:s1, hk:hk + 1]),
            to64(do[s0:s1, hs]), [0, s1 - s0], w.scale, True)
        name = f"seq {b} (n={s1 - s0}) K/V head {hk}"
        assert_close(name + " dQ", to64(dq[s0:s1, hs]), rq, "bf16")
        # dK and dV sum the contributions of four query heads, so their
        # largest entries reach 4..8, where rounding the exact value to bf16
        # alone costs up to 1/64: the max-abs bar is widened by twice that
        # representation floor (the relative RMS bar stays fixed).
        assert_close(name + " dK", to64(dk[s0:s1, hk:hk + 1]), rk, "bf16")
        assert_close(name + " dV", to64(dv[s0:s1, hk:hk + 1]), rv, "bf16")


def test_autograd_varlen():
    """attention_varlen's autograd path returns the entry points' gradients."""
    lengths = [130, 77]
    q, k, v, do, cu = packed(lengths, 4, 1, 64, "fp16", seed=717)
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    qr, kr, vr = (t.clone().requires_grad_() for t in (q, k, v))
    o = fa.attention_varlen(qr, kr, vr, cu_t, 130, causal=True)
    o.backward(do)
    g = run(q, k, v, do, cu, True, 64 ** -0.5)
    torch.cuda.synchronize()
    for tag, a, b in zip(("dQ", "dK", "dV"), (qr.grad, kr.grad, vr.grad), g):
        assert torch.equal(a, b), tag
