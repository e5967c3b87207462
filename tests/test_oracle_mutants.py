"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them: a dropped term, a wrong sign, a wrong
index or axis, a transposed or swapped operand."""

import os
import types

import pytest

from oracle_pins import ALL_PINS

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
SRC = os.path.join(ORACLE, "attention.py")
RNG_SRC = os.path.join(ORACLE, "rng.py")

MUTANTS = {
    "mask_excludes_diagonal": ("s = np.where(kj > qi, -np.inf, s)\n    return s",
                               "s = np.where(kj >= qi, -np.inf, s)\n    return s"),
    "mask_wrong_side": ("s = np.where(kj > qi, -np.inf, s)\n    return s",
                        "s = np.where(kj < qi, -np.inf, s)\n    return s"),
    "mask_no_row_offset": ("qi = row0 + np.arange(n_rows)", "qi = np.arange(n_rows)"),
    "scale_dropped": ("s = scale * (q_rows @ k_all.T)", "s = (q_rows @ k_all.T)"),
    "lse_drops_max": ("lse[b, h, r0:r1] = m[:, 0] + np.log(l[:, 0])",
                      "lse[b, h, r0:r1] = np.log(l[:, 0])"),
    "lse_log2": ("lse[b, h, r0:r1] = m[:, 0] + np.log(l[:, 0])",
                 "lse[b, h, r0:r1] = m[:, 0] + np.log2(l[:, 0])"),
    "fwd_no_max_shift": ("                e = np.exp(s - m)\n                l = e.sum",
                         "                e = np.exp(s)\n                l = e.sum"),
    "fwd_sum_wrong_axis": ("l = e.sum(axis=1, keepdims=True)           # pass 2",
                           "l = e.sum(axis=0, keepdims=True)           # pass 2"),
    "fwd_values_reversed": ("o[b, h, r0:r1] = p @ v[b, h]",
                            "o[b, h, r0:r1] = p @ v[b, h][::-1]"),
    "fwd_values_are_keys": ("o[b, h, r0:r1] = p @ v[b, h]",
                            "o[b, h, r0:r1] = p @ k[b, h]"),
    "probs_no_normalise": ("return e / l, m[:, 0], l[:, 0]", "return e, m[:, 0], l[:, 0]"),
    "online_no_out_correction": ("acc = corr * acc + p @ v[b, h, j0:j1]",
                                 "acc = acc + p @ v[b, h, j0:j1]"),
    "online_no_sum_correction": ("run_sum = corr * run_sum +", "run_sum = run_sum +"),
    "online_corr_sign": ("np.exp(m_prev - run_max))", "np.exp(run_max - m_prev))"),
    "bwd_dv_untransposed": ("dv[b, h] += p.T @ g", "dv[b, h] += p[:, :g.shape[0]] @ g"),
    "bwd_dp_uses_keys": ("dp = g @ v[b, h].T", "dp = g @ k[b, h].T"),
    "bwd_delta_dropped": ("ds = p * (dp - delta)", "ds = p * dp"),
    "bwd_delta_sign": ("ds = p * (dp - delta)", "ds = p * (delta - dp)"),
    "bwd_delta_axis": ("delta = (p * dp).sum(axis=1, keepdims=True)",
                       "delta = (p * dp).sum(axis=1, keepdims=True) * 0 + (p * dp).mean()"),
    "bwd_dq_no_scale": ("dq[b, h, r0:r1] = scale * (ds @ k[b, h])",
                        "dq[b, h, r0:r1] = (ds @ k[b, h])"),
    "bwd_dq_uses_values": ("dq[b, h, r0:r1] = scale * (ds @ k[b, h])",
                           "dq[b, h, r0:r1] = scale * (ds @ v[b, h])"),
    "bwd_dk_uses_grad": ("dk[b, h] += scale * (ds.T @ q[b, h, r0:r1])",
                         "dk[b, h] += scale * (ds.T @ g)"),
    "varlen_head_map_mod": ("            hk = h // group\n            ob, lb",
                            "            hk = h % H_kv\n            ob, lb"),
    "varlen_sequence_shift": ("        s0, s1 = cu[b], cu[b + 1]\n        if s1 <= s0",
                              "        s0, s1 = cu[b], cu[b + 1] + (1 if b == 0 else 0)\n        if s1 <= s0"),
    "decode_causal_off_by_one": ("n = min(L, L - s_q + t + 1)", "n = min(L, L - s_q + t)"),
    "decode_ignores_length": ("n = min(L, L - s_q + t + 1)", "n = min(cap, cap - s_q + t + 1)"),
    "decode_head_map_mod": ("                hk = h // group\n                s = scale",
                            "                hk = h % H_kv\n                s = scale"),
    "merge_unweighted": ("(w[..., None] * o_parts).sum(axis=0)", "o_parts.sum(axis=0)"),
    "merge_lse_drops_max": ("safe_m + np.log(", "np.log("),
    "dropout_no_rescale": ("o[b, h, r0:r1] = (np.where(keep, prob, 0.0) @ v[b, h]) * inv_keep",
                           "o[b, h, r0:r1] = (np.where(keep, prob, 0.0) @ v[b, h])"),
    "dropout_renormalised": (
        "o[b, h, r0:r1] = (np.where(keep, prob, 0.0) @ v[b, h]) * inv_keep",
        "o[b, h, r0:r1] = (np.where(keep, prob, 0.0) / np.where(keep, prob, 0.0).sum("
        "axis=1, keepdims=True)) @ v[b, h]"),
    "dropout_bwd_dp_unmasked": ("dp = (g @ v[b, h].T) * scale_keep", "dp = (g @ v[b, h].T)"),
    "dropout_bwd_dv_unmasked": ("dv[b, h] += (prob * scale_keep).T @ g", "dv[b, h] += prob.T @ g"),
    "varlen_bwd_dk_not_summed": ("            dk[s0:s1, hk] += gk[0, 0]",
                                 "            dk[s0:s1, hk] = gk[0, 0]"),
    "varlen_bwd_dv_wrong_head": ("            dv[s0:s1, hk] += gv[0, 0]",
                                 "            dv[s0:s1, h % H_kv] += gv[0, 0]"),
    "bwd_dk_sign": ("dk[b, h] += scale * (ds.T @ q[b, h, r0:r1])",
                    "dk[b, h] -= scale * (ds.T @ q[b, h, r0:r1])"),
}


# Mistakes planted in the generator and keep-mask module; the oracle under
# test then draws its dropout bits from the mutated copy.
RNG_MUTANTS = {
    "rng_counter_swapped": ("philox4x32_10((cols >> 2)[None, :], (rows >> 2)[:, None],",
                            "philox4x32_10((rows >> 2)[:, None], (cols >> 2)[None, :],"),
    "rng_weyl_constant": ("PHILOX_W0 = 0x9E3779B9", "PHILOX_W0 = 0x9E3779B8"),
    "rng_word_of_row": ("(rows & 3)[None, :, None]", "(3 - (rows & 3))[None, :, None]"),
    "rng_threshold_truncated": ("math.floor(float(np.float32(p)) * 256.0 + 0.5)",
                                "math.floor(float(np.float32(p)) * 256.0)"),
}


def _module(name, path, old=None, new=None):
    with open(path) as f:
        src = f.read()
    if old is not None:
        assert src.count(old) >= 1, f"mutant {name}: pattern not found in {path}"
        src = src.replace(old, new, 1)
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)  # noqa: S102
    return mod


def _load_mutant(name, old, new):
    return _module(name, SRC, old, new)


def _load_rng_mutant(name, old, new):
    mod = _module(name, SRC)
    mod._rng = _module(name + "_rng", RNG_SRC, old, new)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS) + sorted(RNG_MUTANTS))
def test_mutant_is_caught(name):
    if name in MUTANTS:
        mod = _load_mutant(name, *MUTANTS[name])
    else:
        mod = _load_rng_mutant(name, *RNG_MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # any failure means the pin caught it
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches the planted mistake '{name}'"
