"""The parity helpers themselves (host logic, no GPU): the every-head
comparison must pass the oracle's own result rounded to the dtype, catch an
error planted in a single head or a single element, and aggregate the
relative RMS over all compared heads."""

import numpy as np
import pytest
import torch

import oracle.attention as orc
from gpu_util import compare_heads, forward_oracle, max_abs_bar

B, H, N, D = 2, 3, 40, 16
SCALE = D ** -0.5


def _inputs():
    g = torch.Generator().manual_seed(123)
    return [torch.randn(B, H, N, D, generator=g).to(torch.bfloat16) for _ in range(3)]


def _exact(q, k, v, causal):
    f = [t.to(torch.float64).numpy() for t in (q, k, v)]
    o, lse = orc.attention_forward(*f, SCALE, causal)
    return torch.from_numpy(o).to(torch.bfloat16), torch.from_numpy(lse).to(torch.float32)


def _heads():
    return [(b, h) for b in range(B) for h in range(H)]


@pytest.mark.parametrize("causal", [False, True])
def test_rounded_exact_result_passes(causal):
    q, k, v = _inputs()
    o, lse = _exact(q, k, v, causal)
    res = compare_heads("exact", (q, k, v), forward_oracle(SCALE, causal), [("O", o, 0)],
                        "bf16", _heads(), lse=(lse, 1))
    max_abs, rel_rms = res["O"]
    # Only the rounding to bf16 (at most half an ulp of values below 4).
    assert max_abs <= 2 ** -7 and rel_rms < 3e-3


def test_planted_error_in_one_head_fails():
    q, k, v = _inputs()
    o, lse = _exact(q, k, v, True)
    o[1, 2, 17, 5] += 0.05
    with pytest.raises(AssertionError, match="max_abs"):
        compare_heads("planted", (q, k, v), forward_oracle(SCALE, True), [("O", o, 0)], "bf16",
                      _heads())


def test_wrong_head_mapping_fails():
    q, k, v = _inputs()
    o, lse = _exact(q, k, v, False)
    o[0, 1], o[0, 2] = o[0, 2].clone(), o[0, 1].clone()
    with pytest.raises(AssertionError):
        compare_heads("swapped", (q, k, v), forward_oracle(SCALE, False), [("O", o, 0)],
                      "bf16", _heads())


def test_lse_error_fails():
    q, k, v = _inputs()
    o, lse = _exact(q, k, v, False)
    lse[1, 0, 3] += 1e-3
    with pytest.raises(AssertionError, match="lse"):
        compare_heads("lse", (q, k, v), forward_oracle(SCALE, False), [("O", o, 0)], "bf16",
                      _heads(), lse=(lse, 1))


def test_rel_rms_is_over_all_heads():
    """A uniform relative error of 1e-2 on every element gives a relative RMS
    of 1e-2 whatever the split into heads (and fails the 5e-3 bar)."""
    q, k, v = _inputs()
    f = [t.to(torch.float64).numpy() for t in (q, k, v)]
    o, _ = orc.attention_forward(*f, SCALE, False)
    got = torch.from_numpy(o * 1.01)
    with pytest.raises(AssertionError, match="rel_rms=1.000e-02"):
        compare_heads("scaled", (q, k, v), forward_oracle(SCALE, False), [("O", got, 0)],
                      "bf16", _heads())


def test_bar_widens_only_above_the_floor_threshold():
    assert max_abs_bar("bf16", 7.8e-3) == 2e-2
    assert max_abs_bar("bf16", 1.5625e-2) == pytest.approx(2e-2 + 3.125e-2)
    assert max_abs_bar("fp32", 1.0) == 1e-5
