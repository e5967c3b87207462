"""Seeded synthetic inputs for the attention workloads.

Shared by the tests, the smoke check and the bench. It holds no attention
arithmetic: only shapes, seeds, dtypes and the random draws. Both the HIP
path and the CPU oracle receive exactly the tensors made here.

Recipe: a CPU ``torch.Generator`` seeded with the workload's seed draws
``torch.randn`` float32 tensors of shape [B, H, N, D] in the order Q, K, V
(then dO when a backward is run); each is multiplied by the workload's
input multiplier (a power of two, so exact) and rounded to the workload's
dtype (round-to-nearest-even). The oracle upcasts those rounded values to
fp64. The pages' own verification recipe draws Q, K, V the same way with a
fixed seed ("From Self-Attention to FlashAttention", section 2).
"""

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str
    causal: bool
    seed: int
    input_mult: float = 1.0
    backward: bool = False
    scale: float = field(default=None)

    def __post_init__(self):
        if self.scale is None:
            object.__setattr__(self, "scale", 1.0 / math.sqrt(self.D))

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    def flops_fwd(self):
        """Attention forward FLOPs: two N x N x D products, halved if causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.D
        return f / 2 if self.causal else f

    def flops_bwd(self):
        """Backward FLOPs: five products of the forward's size (2.5x)."""
        return 2.5 * self.flops_fwd()

    def bytes_fwd(self):
        """Bytes the fused forward must move: read Q, K, V; write O and LSE."""
        esize = torch.empty((), dtype=self.torch_dtype).element_size()
        return 4 * self.B * self.H * self.N * self.D * esize + 4 * self.B * self.H * self.N

    def bytes_bwd(self):
        """Bytes the backward must move: read Q, K, V, O, dO, LSE; write dQ,
        dK, dV; write and read delta."""
        esize = torch.empty((), dtype=self.torch_dtype).element_size()
        bhn = self.B * self.H * self.N
        return 8 * bhn * self.D * esize + 4 * bhn + 8 * bhn


def fp32_small():
    return Workload("fp32 B1 H2 N256 D64", 1, 2, 256, 64, "fp32", False, 0)


def bf16_short():
    return Workload("bf16 B2 H8 N512 D64", 2, 8, 512, 64, "bf16", False, 42)


def fp16_causal_4k():
    return Workload("fp16 causal B1 H32 N4096 D128", 1, 32, 4096, 128, "fp16",
                    True, 1, input_mult=0.5)


SWEEP_N = (512, 1024, 2048, 4096, 8192, 16384)


def bf16_causal_sweep():
    """bf16 causal, B1 H32 D128 over the sequence lengths, plus D64 at 4096.
    The generator is re-seeded with the same seed for every shape."""
    out = [Workload(f"bf16 causal B1 H32 N{n} D128", 1, 32, n, 128, "bf16", True, 2)
           for n in SWEEP_N]
    out.append(Workload("bf16 causal B1 H32 N4096 D64", 1, 32, 4096, 64, "bf16", True, 2))
    return out


def headline():
    """bf16 causal B1 H32 N4096 D128: the forward throughput workload."""
    return Workload("bf16 causal B1 H32 N4096 D128", 1, 32, 4096, 128, "bf16", True, 2)


def bf16_training():
    return Workload("bf16 causal fwd+bwd B4 H16 N8192 D128", 4, 16, 8192, 128, "bf16",
                    True, 3, backward=True)


@dataclass(frozen=True)
class VarlenWorkload:
    """A packed batch of variable-length sequences with grouped K/V heads."""
    name: str
    lengths: tuple
    H: int
    H_kv: int
    D: int
    dtype: str
    causal: bool
    seed: int

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    @property
    def total(self):
        return sum(self.lengths)

    def cu_seqlens(self):
        cu = [0]
        for n in self.lengths:
            cu.append(cu[-1] + n)
        return cu

    def flops_fwd(self):
        """4 n^2 D per sequence and head, halved if causal."""
        f = sum(4.0 * self.H * n * n * self.D for n in self.lengths)
        return f / 2 if self.causal else f

    def flops_bwd(self):
        """Five n x n x D products per sequence and head (S, dP, dV, dQ, dK):
        2.5 times the forward's."""
        return 2.5 * self.flops_fwd()

    def bytes_fwd(self):
        esize = torch.empty((), dtype=self.torch_dtype).element_size()
        t = self.total
        return (2 * t * self.H + 2 * t * self.H_kv) * self.D * esize + 4 * t * self.H


def varlen_gqa():
    """16 causal bf16 sequences of 256..4096 tokens (seeded, uniform), 32 query
    heads over 8 K/V heads, D = 128: a prefill batch with grouped-query
    attention."""
    g = torch.Generator(device="cpu")
    g.manual_seed(4)
    lengths = tuple(int(x) for x in torch.randint(256, 4097, (16,), generator=g))
    return VarlenWorkload("bf16 causal varlen GQA 16 seqs 256..4096 H32/8 D128", lengths,
                          32, 8, 128, "bf16", True, 4)


def make_varlen_inputs(w: VarlenWorkload, device="cpu", grad=False):
    """Packed q [total, H, D], k, v [total, H_kv, D] from one generator seeded
    with w.seed (drawn in the order q, k, v), and cu_seqlens as int32. With
    grad=True an upstream gradient dO [total, H, D], drawn after v, comes
    last."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    q = torch.randn((w.total, w.H, w.D), generator=g).to(w.torch_dtype)
    k = torch.randn((w.total, w.H_kv, w.D), generator=g).to(w.torch_dtype)
    v = torch.randn((w.total, w.H_kv, w.D), generator=g).to(w.torch_dtype)
    cu = torch.tensor(w.cu_seqlens(), dtype=torch.int32)
    out = [q.to(device), k.to(device), v.to(device), cu.to(device)]
    if grad:
        out.append(torch.randn((w.total, w.H, w.D), generator=g).to(w.torch_dtype).to(device))
    return tuple(out)


@dataclass(frozen=True)
class DecodeWorkload:
    """s_q new tokens per sequence against a K/V cache of capacity cap."""
    name: str
    lengths: tuple
    cap: int
    s_q: int
    H: int
    H_kv: int
    D: int
    dtype: str
    seed: int

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    @property
    def B(self):
        return len(self.lengths)

    def bytes_moved(self):
        """K and V of every cached token read once, Q read, O and LSE written."""
        esize = torch.empty((), dtype=self.torch_dtype).element_size()
        kv = 2 * sum(self.lengths) * self.H_kv * self.D * esize
        qo = 2 * self.B * self.s_q * self.H * self.D * esize
        return kv + qo + 4 * self.B * self.H * self.s_q

    def flops(self):
        """4 D per (query row, visible key) pair."""
        f = 0
        for L in self.lengths:
            for t in range(self.s_q):
                f += 4 * self.H * self.D * max(0, min(L, L - self.s_q + t + 1))
        return float(f)


def decode_gqa():
    """Decode step of 16 sequences with cached lengths uniform in
    [1024, 16384] (seeded), one new token each, 32 query heads over 8 K/V
    heads, D = 128, bf16, cache capacity 16384."""
    g = torch.Generator(device="cpu")
    g.manual_seed(5)
    lengths = tuple(int(x) for x in torch.randint(1024, 16385, (16,), generator=g))
    return DecodeWorkload("bf16 decode 16 seqs cache 1k..16k H32/8 D128 s_q=1", lengths, 16384,
                          1, 32, 8, 128, "bf16", 5)


def make_decode_inputs(w: DecodeWorkload, device="cpu"):
    """q [B, s_q, H, D], k_cache, v_cache [B, cap, H_kv, D] from one generator
    seeded with w.seed (drawn in the order q, k, v; slots past a sequence's
    length hold draws too), and cache_seqlens int32 [B]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    q = torch.randn((w.B, w.s_q, w.H, w.D), generator=g).to(w.torch_dtype)
    k = torch.randn((w.B, w.cap, w.H_kv, w.D), generator=g).to(w.torch_dtype)
    v = torch.randn((w.B, w.cap, w.H_kv, w.D), generator=g).to(w.torch_dtype)
    lens = torch.tensor(w.lengths, dtype=torch.int32)
    return q.to(device), k.to(device), v.to(device), lens.to(device)


def all_workloads():
    return [fp32_small(), bf16_short(), fp16_causal_4k()] + bf16_causal_sweep() + [
        bf16_training()]


def make_inputs(w: Workload, with_grad_out=None, device="cpu"):
    """Draw (q, k, v[, do]) for workload w on the CPU, rounded to w's dtype,
    then move them to `device`."""
    if with_grad_out is None:
        with_grad_out = w.backward
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    shape = (w.B, w.H, w.N, w.D)
    names = ["q", "k", "v"] + (["do"] if with_grad_out else [])
    out = []
    for _ in names:
        t = torch.randn(shape, generator=g, dtype=torch.float32)
        if w.input_mult != 1.0:
            t = t * w.input_mult
        out.append(t.to(w.torch_dtype).to(device))
    return tuple(out)


def make_random(shape, seed, dtype="bf16", mult=1.0, count=3, device="cpu"):
    """`count` randn tensors of `shape` from one seeded CPU generator, for
    ad-hoc test shapes (odd N, edge cases)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    out = []
    for _ in range(count):
        t = torch.randn(shape, generator=g, dtype=torch.float32)
        if mult != 1.0:
            t = t * mult
        out.append(t.to(DTYPES[dtype]).to(device))
    return tuple(out)
