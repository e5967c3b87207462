"""Packed variable-length batches with grouped K/V heads (GQA/MQA) on the GPU
against the fp64 oracle's definition (each sequence and head on its own)."""

import numpy as np
import pytest
import torch

import exact_attention_113_amd as fa
import oracle.attention as orc
import workloads
from gpu_util import assert_close, assert_lse_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def packed(lengths, H, H_kv, D, dtype, seed, extra=0):
    total = sum(lengths) + extra
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    td = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    q = torch.randn((total, H, D), generator=g).to(td)
    k = torch.randn((total, H_kv, D), generator=g).to(td)
    v = torch.randn((total, H_kv, D), generator=g).to(td)
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    return q.to(DEV), k.to(DEV), v.to(DEV), cu


def run_and_check(name, q, k, v, cu, causal, scale, dtype):
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    lengths = [b - a for a, b in zip(cu[:-1], cu[1:])]
    o, lse = fa.forward_varlen(q, k, v, cu_t, max(lengths), causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = orc.attention_forward_varlen(to64(q), to64(k), to64(v), cu, scale, causal)
    covered = np.zeros(q.shape[0], dtype=bool)
    for a, b in zip(cu[:-1], cu[1:]):
        covered[a:b] = True
    assert_close(name + " O", to64(o)[covered], ro[covered], dtype)
    assert_lse_close(name, to64(lse)[:, covered], rl[:, covered])
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H_kv", [4, 2, 1])
def test_ragged_packed_gqa(dtype, D, causal, H_kv):
    lengths = [1, 7, 0, 65, 300, 129, 256]
    q, k, v, cu = packed(lengths, 4, H_kv, D, dtype, seed=300 + D + H_kv)
    run_and_check(f"{dtype} D{D} causal={causal} H4/{H_kv}", q, k, v, cu, causal, D ** -0.5,
                  dtype)


def test_equal_lengths_match_dense_bitwise():
    """A packed batch of equal-length sequences with H_kv = H runs the same
    arithmetic as the dense entry point: results agree bit for bit."""
    B, H, N, D = 3, 4, 333, 128
    q, k, v = workloads.make_random((B, H, N, D), seed=51, dtype="bf16", device=DEV)
    o, lse = fa.forward(q, k, v, causal=True, scale=0.1)
    pk = [t.permute(0, 2, 1, 3).reshape(B * N, H, D).contiguous() for t in (q, k, v)]
    cu = torch.tensor([0, N, 2 * N, 3 * N], dtype=torch.int32, device=DEV)
    o2, lse2 = fa.forward_varlen(*pk, cu, N, causal=True, scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(o2, o.permute(0, 2, 1, 3).reshape(B * N, H, D))
    assert torch.equal(lse2, lse.permute(1, 0, 2).reshape(H, B * N))


def test_gqa_equals_repeated_heads():
    """Grouped heads read exactly what repeating each K/V head over its group
    would: bitwise equal to the packed kernel with expanded K and V."""
    lengths = [513, 96, 1000]
    q, k, v, cu = packed(lengths, 8, 2, 128, "bf16", seed=61)
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    o, lse = fa.forward_varlen(q, k, v, cu_t, 1000, causal=True)
    ke = k.repeat_interleave(4, dim=1).contiguous()
    ve = v.repeat_interleave(4, dim=1).contiguous()
    o2, lse2 = fa.forward_varlen(q, ke, ve, cu_t, 1000, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


def test_prefill_batch_workload_sampled():
    """The benchmark's packed prefill batch (16 sequences of 256..4096 tokens,
    32 query over 8 K/V heads): sampled sequences and heads against the oracle
    at the full size."""
    w = workloads.varlen_gqa()
    q, k, v, cu_t = workloads.make_varlen_inputs(w, device=DEV)
    cu = w.cu_seqlens()
    o, lse = fa.forward_varlen(q, k, v, cu_t, max(w.lengths), causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (6, 31), (11, 13)]:
        s0, s1 = cu[b], cu[b + 1]
        hk = h // (w.H // w.H_kv)
        ro, rl = orc.attention_forward(to64(q[s0:s1, h])[None, None], to64(k[s0:s1, hk])[None, None],
                                       to64(v[s0:s1, hk])[None, None], w.scale, True)
        assert_close(f"seq {b} head {h} O", to64(o[s0:s1, h])[None, None], ro, "bf16")
        assert_lse_close(f"seq {b} head {h}", to64(lse[h, s0:s1])[None, None], rl)


@pytest.mark.parametrize("D", [64, 128])
def test_uncovered_rows_untouched(D):
    """Tokens after the last sequence keep the caller's O and LSE; the rows of
    each sequence are written up to its end and no further (a sequence of 200
    tokens ends inside a 256-row tile, the next starts right after it)."""
    lengths = [200, 33, 300]
    q, k, v, cu = packed(lengths, 4, 2, D, "bf16", seed=733 + D, extra=70)
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    o = torch.full_like(q, 7.0)
    lse = torch.full((4, q.shape[0]), 7.0, dtype=torch.float32, device=DEV)
    fa.forward_varlen(q, k, v, cu_t, max(lengths), causal=True, scale=0.1, out=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = orc.attention_forward_varlen(to64(q), to64(k), to64(v), cu, 0.1, True)
    n = cu[-1]
    assert_close("covered O", to64(o)[:n], ro[:n], "bf16")
    assert_lse_close("covered", to64(lse)[:, :n], rl[:, :n])
    assert bool((o[n:] == 7).all()) and bool((lse[:, n:] == 7).all())


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_long_packed_sequences_short_grid(D, causal):
    """A few long sequences (so few 256-row tiles that the forward splits each
    row group's keys between two waves) with grouped heads, every head against
    the oracle: tiles end inside a sequence and the next one starts mid-tile."""
    lengths = [700, 1333, 1, 517]
    q, k, v, cu = packed(lengths, 4, 2, D, "bf16", seed=900 + D + int(causal))
    run_and_check(f"long packed D{D} causal={causal}", q, k, v, cu, causal, D ** -0.5, "bf16")


@pytest.mark.parametrize("causal", [False, True])
def test_packed_large_grid_d64(causal):
    """A packed batch big enough for the whole-key-range D = 64 path (four K and
    four V tiles, one barrier per two tiles): 16 sequences of 900..2100 tokens,
    32 query over 8 K/V heads; sampled sequences and heads against the oracle."""
    g = np.random.default_rng(2048 + int(causal))
    lengths = [int(x) for x in g.integers(900, 2101, size=16)]
    q, k, v, cu = packed(lengths, 32, 8, 64, "bf16", seed=2049 + int(causal))
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    o, lse = fa.forward_varlen(q, k, v, cu_t, max(lengths), causal=causal, scale=0.125)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (7, 19), (15, 31)]:
        s0, s1 = cu[b], cu[b + 1]
        hk = h // 4
        ro, rl = orc.attention_forward(to64(q[s0:s1, h])[None, None],
                                       to64(k[s0:s1, hk])[None, None],
                                       to64(v[s0:s1, hk])[None, None], 0.125, causal)
        assert_close(f"packed D64 seq {b} head {h}", to64(o[s0:s1, h])[None, None], ro, "bf16")
        assert_lse_close(f"packed D64 seq {b} head {h}", to64(lse[h, s0:s1])[None, None], rl)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("H_kv", [8, 2, 1])
def test_whole_batch_order_every_row(D, causal, H_kv):
    """Eight query heads take the grid of only real tiles, heaviest first over
    the batch (with four heads above, the per-sequence order): every row of
    every sequence against the oracle, from outputs filled with a sentinel so
    that a tile left out or written twice elsewhere shows; the tokens after
    the last sequence keep the sentinel."""
    lengths = [1, 7, 0, 65, 300, 129, 256, 700]
    q, k, v, cu = packed(lengths, 8, H_kv, D, "bf16", seed=4100 + D + H_kv + int(causal), extra=45)
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    o = torch.full_like(q, 7.0)
    lse = torch.full((8, q.shape[0]), 7.0, dtype=torch.float32, device=DEV)
    fa.forward_varlen(q, k, v, cu_t, max(lengths), causal=causal, scale=D ** -0.5, out=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = orc.attention_forward_varlen(to64(q), to64(k), to64(v), cu, D ** -0.5, causal)
    n = cu[-1]
    name = f"whole-batch order D{D} causal={causal} H8/{H_kv}"
    assert_close(name + " O", to64(o)[:n], ro[:n], "bf16")
    assert_lse_close(name, to64(lse)[:, :n], rl[:, :n])
    assert bool((o[n:] == 7).all()) and bool((lse[:, n:] == 7).all())


def test_whole_batch_order_matches_dense_bitwise():
    """Equal lengths with eight heads (the whole-batch order) give the dense
    entry point's results bit for bit."""
    B, H, N, D = 3, 8, 700, 128
    q, k, v = workloads.make_random((B, H, N, D), seed=57, dtype="bf16", device=DEV)
    o, lse = fa.forward(q, k, v, causal=True, scale=0.1)
    pk = [t.permute(0, 2, 1, 3).reshape(B * N, H, D).contiguous() for t in (q, k, v)]
    cu = torch.tensor([0, N, 2 * N, 3 * N], dtype=torch.int32, device=DEV)
    o2, lse2 = fa.forward_varlen(*pk, cu, N, causal=True, scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(o2, o.permute(0, 2, 1, 3).reshape(B * N, H, D))
    assert torch.equal(lse2, lse.permute(1, 0, 2).reshape(H, B * N))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_whole_batch_order_long_every_row(D, causal):
    """The whole-batch order on the whole-key-range kernel (enough 256-row
    tiles that keys are not split): every row against the oracle, sentinel
    outputs as above."""
    lengths = [1, 2000, 0, 3000, 777, 2500, 129]
    q, k, v, cu = packed(lengths, 8, 2, D, "bf16", seed=4200 + D + int(causal), extra=11)
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    o = torch.full_like(q, 7.0)
    lse = torch.full((8, q.shape[0]), 7.0, dtype=torch.float32, device=DEV)
    fa.forward_varlen(q, k, v, cu_t, max(lengths), causal=causal, scale=D ** -0.5, out=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = orc.attention_forward_varlen(to64(q), to64(k), to64(v), cu, D ** -0.5, causal)
    n = cu[-1]
    name = f"whole-batch order, long, D{D} causal={causal} H8/2"
    assert_close(name + " O", to64(o)[:n], ro[:n], "bf16")
    assert_lse_close(name, to64(lse)[:, :n], rl[:, :n])
    assert bool((o[n:] == 7).all()) and bool((lse[:, n:] == 7).all())


@pytest.mark.parametrize("causal", [False, True])
def test_whole_batch_order_four_way_split(causal):
    """The whole-batch order on the D = 64 four-way key split (64-row tiles):
    every row against the oracle, sentinel outputs as above."""
    lengths = [1, 0, 500, 77]
    q, k, v, cu = packed(lengths, 8, 2, 64, "bf16", seed=4300 + int(causal), extra=9)
    cu_t = torch.tensor(cu, dtype=torch.int32, device=DEV)
    o = torch.full_like(q, 7.0)
    lse = torch.full((8, q.shape[0]), 7.0, dtype=torch.float32, device=DEV)
    fa.forward_varlen(q, k, v, cu_t, max(lengths), causal=causal, scale=0.125, out=o, lse=lse)
    torch.cuda.synchronize()
    ro, rl = orc.attention_forward_varlen(to64(q), to64(k), to64(v), cu, 0.125, causal)
    n = cu[-1]
    name = f"whole-batch order, four-way split, causal={causal}"
    assert_close(name + " O", to64(o)[:n], ro[:n], "bf16")
    assert_lse_close(name, to64(lse)[:, :n], rl[:, :n])
    assert bool((o[n:] == 7).all()) and bool((lse[:, n:] == 7).all())
