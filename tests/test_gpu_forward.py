"""Forward parity on the GPU: the HIP kernels through the C ABI against the
fp64 CPU oracle on the same seeded inputs."""

import numpy as np
import pytest
import torch

import exact_attention_113_amd as fa
import workloads
from gpu_util import (all_heads, assert_close, assert_lse_close, compare_heads, forward_oracle,
                      oracle_forward, pick, to64)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(q, k, v, causal, scale):
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def check(name, q, k, v, causal, scale, dtype, heads, strict=False):
    o, lse = run(q, k, v, causal, scale)
    ro, rl = oracle_forward(q, k, v, scale, causal, heads)
    assert_close(name + " O", pick(o, heads), ro, dtype, strict=strict)
    assert_lse_close(name, pick(lse, heads), rl)
    return o, lse


def check_every_head(name, q, k, v, causal, scale, dtype):
    """Every (batch, head) of O and LSE of a named workload against the
    oracle (threads over heads), at the fixed bars."""
    o, lse = run(q, k, v, causal, scale)
    B, H = q.shape[:2]
    compare_heads(name, (q, k, v), forward_oracle(scale, causal), [("O", o, 0)], dtype,
                  all_heads(B, H), lse=(lse, 1), strict=True)
    return o, lse


def test_fp32_b1h2_n256_d64():
    w = workloads.fp32_small()
    q, k, v = workloads.make_inputs(w, device=DEV)
    check(w.name, q, k, v, w.causal, w.scale, w.dtype, all_heads(w.B, w.H), strict=True)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 1500), (1, 16, 2176)], ids=["split", "unsplit"])
def test_fp32_both_grids(shape, causal, D):
    """fp32 grids of a few query tiles split each row group's keys over
    several waves and merge their states; grids of more than one 128-row
    tile per CU run one wave per row group. Both with a ragged last tile,
    every head against the oracle."""
    B, H, N = shape
    q, k, v = workloads.make_random((B, H, N, D), seed=17 + N + D, dtype="fp32", device=DEV)
    o, lse = run(q, k, v, causal, D ** -0.5)
    compare_heads(f"fp32 {shape} D{D} causal={causal}", (q, k, v),
                  forward_oracle(D ** -0.5, causal), [("O", o, 0)], "fp32", all_heads(B, H),
                  lse=(lse, 1), strict=True)


def test_bf16_b2h8_n512_d64():
    w = workloads.bf16_short()
    q, k, v = workloads.make_inputs(w, device=DEV)
    check(w.name, q, k, v, w.causal, w.scale, w.dtype, all_heads(w.B, w.H), strict=True)


def test_fp16_causal_b1h32_n4096_d128():
    w = workloads.fp16_causal_4k()
    q, k, v = workloads.make_inputs(w, device=DEV)
    o, _ = check_every_head(w.name, q, k, v, w.causal, w.scale, w.dtype)
    # Causal row 0 attends to key 0 only, so O[0] = V[0] exactly.
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    assert torch.isfinite(o).all()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("w", workloads.bf16_causal_sweep(), ids=lambda w: w.name)
def test_bf16_causal_sweep(w):
    q, k, v = workloads.make_inputs(w, device=DEV)
    o, _ = check_every_head(w.name, q, k, v, w.causal, w.scale, w.dtype)
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    assert torch.isfinite(o).all()


@pytest.mark.timeout(600)
def test_bf16_training_forward_b4h16_n8192():
    w = workloads.bf16_training()
    q, k, v = workloads.make_inputs(w, with_grad_out=False, device=DEV)
    o, _ = check_every_head(w.name + " fwd", q, k, v, w.causal, w.scale, w.dtype)
    assert torch.equal(o[:, :, 0], v[:, :, 0])


ODD_N = [1, 2, 7, 31, 33, 63, 65, 127, 129, 200, 1000]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths(dtype, D, causal):
    for N in ODD_N:
        q, k, v = workloads.make_random((2, 3, N, D), seed=1000 + N, dtype=dtype, device=DEV)
        check(f"{dtype} D{D} causal={causal} N{N}", q, k, v, causal, D ** -0.5, dtype,
              all_heads(2, 3))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("scale", [0.0, -0.3, 0.02, 1.0])
def test_scales(dtype, scale):
    for causal in (False, True):
        q, k, v = workloads.make_random((1, 2, 300, 64), seed=7, dtype=dtype, device=DEV)
        o, lse = check(f"{dtype} scale={scale} causal={causal}", q, k, v, causal, scale, dtype,
                       all_heads(1, 2))
        if scale == 0.0:
            # Uniform weights: LSE = ln(number of visible keys).
            n = np.arange(1, 301) if causal else np.full(300, 300)
            np.testing.assert_allclose(to64(lse)[0, 0], np.log(n), atol=1e-5)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_large_inputs(dtype):
    """Inputs x4 make raw scores of order 100: softmax in fp32 must not
    overflow the 16-bit types."""
    q, k, v = workloads.make_random((1, 2, 256, 128), seed=9, dtype=dtype, mult=4.0, device=DEV)
    for causal in (False, True):
        check(f"{dtype} x4 causal={causal}", q, k, v, causal, 128 ** -0.5, dtype, all_heads(1, 2))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_constant_v(dtype):
    q, k, _ = workloads.make_random((1, 2, 333, 64), seed=11, dtype=dtype, device=DEV)
    c = torch.linspace(-2, 2, 64).to(q.dtype).to(DEV)
    v = c.expand(1, 2, 333, 64).contiguous()
    for causal in (False, True):
        o, _ = run(q, k, v, causal, 0.125)
        tol = 1e-5 if dtype == "fp32" else 2e-2
        assert float((o.float() - v.float()).abs().max()) <= tol


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_deterministic(dtype):
    q, k, v = workloads.make_random((2, 4, 1000, 128), seed=13, dtype=dtype, device=DEV)
    for causal in (False, True):
        o1, l1 = run(q, k, v, causal, 0.1)
        o2, l2 = run(q, k, v, causal, 0.1)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
def test_guard_bands(dtype, D):
    """Outputs written in place inside larger buffers: nothing outside the
    O and LSE regions changes."""
    B, H, N = 2, 3, 77
    q, k, v = workloads.make_random((B, H, N, D), seed=15, dtype=dtype, device=DEV)
    n_o, n_l, pad = B * H * N * D, B * H * N, 4096
    obuf = torch.full((n_o + 2 * pad,), 7.0, dtype=q.dtype, device=DEV)
    lbuf = torch.full((n_l + 2 * pad,), 7.0, dtype=torch.float32, device=DEV)
    o = obuf[pad:pad + n_o].view(B, H, N, D)
    lse = lbuf[pad:pad + n_l].view(B, H, N)
    fa.forward(q, k, v, causal=True, scale=0.1, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((obuf[:pad] == 7).all()) and bool((obuf[pad + n_o:] == 7).all())
    assert bool((lbuf[:pad] == 7).all()) and bool((lbuf[pad + n_l:] == 7).all())
    ro, rl = oracle_forward(q, k, v, 0.1, True, all_heads(B, H))
    assert_close("guarded O", pick(o, all_heads(B, H)), ro, dtype)


def test_autograd_forward_matches():
    q, k, v = workloads.make_random((1, 2, 64, 64), seed=17, dtype="bf16", device=DEV)
    o = fa.attention(q, k, v, causal=True)
    o2, _ = run(q, k, v, True, 0.125)
    assert torch.equal(o, o2)


def test_long_sequence_sampled_rows():
    """A 131072-token causal sequence (two heads, D = 128): the last query
    tile streams 2048 key tiles. Sampled rows are checked against the
    oracle's definition, row i being the attention of query i over keys
    0..i."""
    import oracle.attention as orc
    B, H, N, D = 1, 2, 131072, 128
    q, k, v = workloads.make_random((B, H, N, D), seed=77, dtype="bf16", device=DEV)
    o, lse = run(q, k, v, True, D ** -0.5)
    for h, i in [(0, 0), (0, 255), (1, 256), (1, 65535), (0, 100003), (1, N - 1)]:
        # Query i against a cache of its i + 1 visible keys (one new token).
        ro, rl = orc.attention_decode(to64(q[0, h, i:i + 1])[None, :, None],
                                      to64(k[0, h, :i + 1])[None, :, None],
                                      to64(v[0, h, :i + 1])[None, :, None], [i + 1], D ** -0.5)
        assert_close(f"head {h} row {i} O", to64(o[0, h, i]), ro[0, 0, 0], "bf16")
        assert_lse_close(f"head {h} row {i}", to64(lse[0, h, i:i + 1]), rl[0, 0])


def test_offsets_beyond_2g_elements():
    """4096 sequences x 32 heads of 128 tokens (D = 128): each tensor holds
    2^31 elements, so the last heads start past 32-bit element offsets.
    Forward and backward of sampled heads against the oracle. The inputs are
    drawn on the device from a seeded generator (4 GiB each)."""
    from gpu_util import oracle_backward
    B, H, N, D = 4096, 32, 128, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(99)
    q, k, v, do = (torch.randn((B, H, N, D), generator=g, device=DEV).to(torch.bfloat16)
                   for _ in range(4))
    o, lse = fa.forward(q, k, v, causal=True)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    heads = [(0, 0), (2048, 5), (4095, 31)]
    ro, rl = oracle_forward(q, k, v, D ** -0.5, True, heads)
    assert_close("O", pick(o, heads), ro, "bf16")
    assert_lse_close("LSE", pick(lse, heads), rl)
    for tag, got, r in zip(("dQ", "dK", "dV"), (dq, dk, dv),
                           oracle_backward(q, k, v, do, D ** -0.5, True, heads)):
        assert_close(tag, pick(got, heads), r, "bf16")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(4, 16, 2048), (8, 16, 1000)])
def test_large_grid_d64(causal, shape):
    """D = 64 on grids of at least 512 256-row tiles, the path that keeps four
    K and four V tiles and synchronises once per two tiles (one shape with a
    ragged last tile): sampled heads against the oracle."""
    B, H, N = shape
    q, k, v = workloads.make_random((B, H, N, 64), seed=3100 + N + int(causal), dtype="bf16",
                                    device=DEV)
    check(f"D64 B{B} H{H} N{N} causal={causal}", q, k, v, causal, 0.125, "bf16",
          [(0, 0), (B // 2, 7), (B - 1, H - 1)])


@pytest.mark.parametrize("shape", [(1, 32, 1536, 128), (3, 32, 1024, 64), (1, 32, 1024, 128)])
def test_full_attention_grid_sizes(shape):
    """Full attention on grids just above and at half the CUs' worth of
    256-row tiles (whole key ranges above, split keys at or below): sampled
    heads against the oracle."""
    B, H, N, D = shape
    q, k, v = workloads.make_random((B, H, N, D), seed=5100 + N + D, dtype="bf16", device=DEV)
    check(f"full B{B} H{H} N{N} D{D}", q, k, v, False, D ** -0.5, "bf16",
          [(0, 0), (B - 1, H // 2), (B - 1, H - 1)])


@pytest.mark.parametrize("shape", [(1, 48, 2048, 128), (3, 32, 1024, 64), (1, 32, 2048, 128)])
def test_causal_grid_sizes(shape):
    """Causal attention on grids just above and at one round of the CUs'
    256-row tiles (whole key ranges above, split keys at or below): sampled
    heads against the oracle."""
    B, H, N, D = shape
    q, k, v = workloads.make_random((B, H, N, D), seed=5300 + N + D, dtype="bf16", device=DEV)
    check(f"causal B{B} H{H} N{N} D{D}", q, k, v, True, D ** -0.5, "bf16",
          [(0, 0), (B - 1, H // 2), (B - 1, H - 1)])
