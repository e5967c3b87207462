"""CPU oracle for exact scaled dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check and the bench's
CPU-baseline leg use it. It shares no code with the HIP library.

Sources (pages cited by title and section):
  [P1] "From Self-Attention to FlashAttention: the evolution of attention
       acceleration" (wmrh.cn), sections 1 (standard vs. flash data flow)
       and 2 (online softmax, with its blockwise PyTorch sketch).
  [P2] "Flash Attention algorithm design and I/O optimisation" interview
       page (algomooc.com), sections "Positioning" and "Core mechanism".
  [P3] "FlashAttention in ops-transformer: keeping the attention matrix on
       chip" (mhpn.cn), sections "Core idea", "Online softmax" and
       "A surprise" (the backward remark).
"""

from . import rng  # noqa: F401
from .attention import (  # noqa: F401
    attention_forward,
    attention_forward_online,
    attention_forward_varlen,
    attention_backward_varlen,
    attention_decode,
    attention_forward_dropout,
    attention_backward_dropout,
    merge_partials,
    attention_backward,
    attention_probabilities,
)
