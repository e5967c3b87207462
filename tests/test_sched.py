"""The kernels' work orders, checked on the CPU: tests/sched_check.cpp is
compiled against the host/device scheduling functions the kernels and their
launchers use (exact_attention_113_amd/csrc/fa_sched.h) and enumerates
every workgroup of the dense, packed (empty, one-token and ragged sequences,
grouped heads), fp32, backward and decode grids: every row is produced
exactly once and every index stays inside its tensor."""

import os
import subprocess

import pytest

from exact_attention_113_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "sched_check.cpp")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("sched") / "sched_check")
    cmd = [build.hipcc_path(), "-x", "hip", f"--offload-arch={build.ARCH}", "-O2",
           "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", build.CSRC, SRC, "-o", out]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout
    return out


def test_every_row_once_and_in_bounds(checker):
    res = subprocess.run([checker], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=600)
    print(res.stdout[-3000:])
    assert res.returncode == 0, [l for l in res.stdout.splitlines() if l.startswith("FAIL")]
    last = res.stdout.strip().splitlines()[-1]
    assert last.endswith("0 failed"), last
    assert int(last.split()[0]) >= 100, last


# Plausible mistakes planted in a copy of fa_sched.h; the checker compiled
# against each copy must report a failure.
MUTANTS = {
    "xcd_slot_halved": ("return (lin & 7) * (total >> 3) + (lin >> 3);",
                        "return (lin & 7) * (total >> 3) + (lin >> 4);"),
    "fwd_pair_off": ("p = xcd * hpx + slot % hpx;", "p = xcd * hpx + slot / hpx;"),
    "fwd_pairwise_head": ("p = xcd * hpx + 2 * j + (within & 1);", "p = xcd * hpx + j + (within & 1);"),
    "fwd_pairwise_tile": ("qt = n_qtiles - 1 - within / 2;", "qt = n_qtiles - 1 - within / 4;"),
    "packed_tile_off_by_one": ("return packed ? qt - (n_qtiles - (n + bm - 1) / bm) : qt;",
                               "return packed ? qt - (n_qtiles - n / bm) : qt;"),
    "dq_tile_bound": ("return (qt < 0 || qt * bm >= n) ? -1 : qt;",
                      "return (qt < 0 || qt * bm > n) ? -1 : qt;"),
    "bwd_round_major_unit": ("unit = (blk & 7) * per_xcd + s % per_xcd;",
                             "unit = (blk & 7) * per_xcd + s / per_xcd;"),
    "seq_end_unclamped": ("const int s1 = a1 < s0 ? s0 : (a1 > total ? total : a1);",
                          "const int s1 = a1 < s0 ? s0 : a1;"),
    "decode_unit_swap": ("split = rest % n_splits;\n  b = rest / n_splits;",
                         "b = rest % n_splits;\n  split = rest / n_splits;"),
    "decode_chunk_round": ("chunk = (chunk + 127) / 128 * 128;", "chunk = chunk / 128 * 128;"),
    "decode_active_floor": ("const int n = (L + chunk - 1) / chunk;", "const int n = L / chunk;"),
    "lpt_grid_bound": ("const int64_t bound = (total + batch * (bm - 1)) / bm;",
                       "const int64_t bound = (total + bm - 1) / bm;"),
    "lpt_tile_counts": ("c[l] += nt[j] - l > 0 ? nt[j] - l : 0;",
                        "c[l] += nt[j] - l > 1 ? nt[j] - l : 0;"),
    "lpt_rank": ("const int rank = __builtin_popcountll(m2 & ((1ull << l) - 1));",
                 "const int rank = __builtin_popcountll(m2 & ((2ull << l) - 1));"),
    "compact_grid_bound": ("const int64_t bound = (total + batch * (bt - 1)) / bt;",
                           "const int64_t bound = (total + bt - 1) / bt;"),
    "compact_prefix_inclusive": ("pre[l] = sum;\n    sum += nt[l];",
                                 "sum += nt[l];\n    pre[l] = sum;"),
    "decode_order_off_by_one": ("    if (c < pre + na) {", "    if (c <= pre + na) {"),
    "split_rows": ("s.bm = 256 / s.ks;", "s.bm = 128;"),
    "f32_split_rows": ("s.bm = 32 * f32_row_groups(s.ks);", "s.bm = 32 * f32_row_groups(1);"),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_checker_catches_planted_mistake(mutant, tmp_path):
    old, new = MUTANTS[mutant]
    with open(os.path.join(build.CSRC, "fa_sched.h")) as f:
        text = f.read()
    assert text.count(old) == 1, mutant
    (tmp_path / "fa_sched.h").write_text(text.replace(old, new))
    # fa_internal.h includes "fa_sched.h" from its own directory: copy it too.
    with open(os.path.join(build.CSRC, "fa_internal.h")) as f:
        (tmp_path / "fa_internal.h").write_text(f.read())
    out = str(tmp_path / "sched_check")
    cmd = [build.hipcc_path(), "-x", "hip", f"--offload-arch={build.ARCH}", "-O1",
           "-std=c++17", "-I", str(tmp_path), "-I", os.path.join(ROOT, "include"), "-I",
           build.CSRC, SRC, "-o", out]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout
    run = subprocess.run([out], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=600)
    # A failed check, or a crash of the checker on the broken plan.
    assert run.returncode != 0, f"{mutant} not caught"
