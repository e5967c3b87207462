"""Build-time check of the decode kernel's hand-ordered loads (CPU only).

The decode kernel issues its K loads and V's transposed LDS reads as plain
instructions that the compiler does not track, and orders every use of the
loaded registers with explicit s_waitcnt statements. That is only sound if
the compiled code leaves a load's destination registers alone until the wait
that covers it. This test compiles fa_decode.hip to gfx950 assembly with the
library's own flags and checks exactly that for every kernel instantiation:
between an untracked load and the next wait of its kind, no instruction may
read or write the registers it loads, on any control-flow path (branches
are followed both ways, the key loop around its back edge).
"""

import os
import re
import subprocess

import pytest

from exact_attention_113_amd import build

CSRC = build.CSRC
KERNELS = [
    "_ZN2fa12_GLOBAL__N_113decode_kernelINS_4Bf16ELi128EEEvNS0_9DecParamsE",
    "_ZN2fa12_GLOBAL__N_113decode_kernelINS_3F16ELi128EEEvNS0_9DecParamsE",
    "_ZN2fa12_GLOBAL__N_113decode_kernelINS_4Bf16ELi64EEEvNS0_9DecParamsE",
    "_ZN2fa12_GLOBAL__N_113decode_kernelINS_3F16ELi64EEEvNS0_9DecParamsE",
]
ASYNC = ("global_load_dwordx4", "ds_read_b64_tr_b16")


def _regs(text):
    out = set()
    for m in re.finditer(r"v\[(\d+):(\d+)\]", text):
        out |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"(?<![\w\[])v(\d+)\b", text):
        out.add(int(m.group(1)))
    return out


def _dest(line):
    m = re.match(r"\S+\s+v\[(\d+):(\d+)\]", line)
    return set(range(int(m.group(1)), int(m.group(2)) + 1)) if m else set()


def _successors(body, labels, k):
    """Indices of the instructions that can run after body[k]."""
    line = body[k]
    op = line.split()[0]
    if op == "s_endpgm":
        return []
    target = None
    m = re.search(r"(\.LBB\w+)", line)
    if op.startswith("s_branch") or op.startswith("s_cbranch"):
        if m and m.group(1) in labels:
            target = labels[m.group(1)]
    if op.startswith("s_branch"):
        return [target] if target is not None else []
    nxt = [k + 1] if k + 1 < len(body) else []
    return nxt + ([target] if target is not None else [])


def violations(body):
    """(load, offending instruction) pairs for one kernel's instruction list:
    every path from an untracked load (following unconditional and both ways
    of conditional branches, loops included) is walked up to the first wait
    of its kind, and any instruction on it that reads or writes the load's
    registers is reported."""
    labels = {l[:-1]: k for k, l in enumerate(body) if l.endswith(":")}
    bad = []
    for k, line in enumerate(body):
        op = line.split()[0]
        if op not in ASYNC:
            continue
        dst = _dest(line)
        assert dst, line
        kind = "vmcnt" if op.startswith("global") else "lgkmcnt(0)"
        seen = set()
        stack = _successors(body, labels, k)
        while stack:
            i = stack.pop()
            if i in seen:
                continue
            seen.add(i)
            t = body[i]
            top = t.split()[0]
            if top == "s_waitcnt" and kind in t:
                continue
            if not top.endswith(":"):
                if top in ASYNC:
                    rest = t.split(",", 1)[1] if "," in t else ""
                    if (_dest(t) & dst) or (_regs(rest) & dst):
                        bad.append((line, t))
                elif _regs(t) & dst:
                    bad.append((line, t))
            stack.extend(_successors(body, labels, i))
    return bad


@pytest.fixture(scope="module")
def listing(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "fa_decode.s"
    flags = [f for f in build.COMMON_FLAGS if f != "-Wall"]
    cmd = [build.hipcc_path(), *flags, "--cuda-device-only", "-S",
           os.path.join(CSRC, "fa_decode.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    return out.read_text()


@pytest.mark.parametrize("kernel", KERNELS)
def test_untracked_loads_are_left_alone_until_waited(listing, kernel):
    i = listing.index(kernel + ":")
    j = listing.index(".Lfunc_end", i)
    body = [l.strip() for l in listing[i:j].split("\n")
            if l.strip() and not l.strip().startswith(";")]
    n_loads = sum(1 for l in body if l.split()[0] in ASYNC)
    assert n_loads >= 16, "expected the decode kernel's untracked loads in the listing"
    assert violations(body) == []


def test_checker_catches_a_planted_use():
    """The checker itself: a use of a loaded register before its wait is found."""
    body = ["global_load_dwordx4 v[4:7], v[0:1], off",
            "v_add_f32_e32 v8, v5, v9",
            "s_waitcnt vmcnt(0)",
            "v_add_f32_e32 v10, v4, v9"]
    assert len(violations(body)) == 1
    assert violations(body[:1] + body[2:]) == []


def test_checker_follows_branches():
    """A write in a block the load's path branches over is not a use; one in a
    block a conditional branch can reach is."""
    skipped = ["global_load_dwordx4 v[4:7], v[0:1], off",
               "s_branch .LBB0_3",
               ".LBB0_2:",
               "v_mov_b32_e32 v4, 0",
               ".LBB0_3:",
               "s_waitcnt vmcnt(0)",
               "v_add_f32_e32 v10, v4, v9",
               "s_endpgm"]
    assert violations(skipped) == []
    reached = ["global_load_dwordx4 v[4:7], v[0:1], off",
               "s_cbranch_scc1 .LBB0_2",
               "s_waitcnt vmcnt(0)",
               "s_endpgm",
               ".LBB0_2:",
               "v_mov_b32_e32 v5, 0",
               "s_endpgm"]
    assert len(violations(reached)) == 1
