"""Build-time check of the decode kernel's hand-ordered loads (CPU only).

The decode kernel issues its K loads and V's transposed LDS reads as plain
instructions that the compiler does not track, and orders every use of the
loaded registers with explicit s_waitcnt statements. That is only sound if
the compiled code leaves a load's destination registers alone until the wait
that covers it. This test compiles fa_decode.hip to gfx950 assembly with the
library's own flags and checks exactly that for every kernel instantiation:
between an untracked load and the next wait of its kind, no instruction may
read or write the registers it loads (the key loop is followed around its
back edge).
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


def violations(body):
    """(load, offending instruction) pairs for one kernel's instruction list."""
    heads = [k for k, l in enumerate(body) if "Loop Header" in l]
    loop = None
    if heads:
        start = heads[0]
        ends = [k for k, l in enumerate(body)
                if k > start and l.startswith("s_cbranch") and ".LBB" in l]
        loop = (start, max(ends))
    bad = []
    for k, line in enumerate(body):
        op = line.split()[0]
        if op not in ASYNC:
            continue
        dst = _dest(line)
        assert dst, line
        kind = "vmcnt" if op.startswith("global") else "lgkmcnt(0)"
        seq = body[k + 1:]
        if loop and loop[0] <= k <= loop[1]:
            seq = body[k + 1:loop[1] + 1] + body[loop[0]:k]
        for t in seq:
            top = t.split()[0]
            if top == "s_waitcnt" and kind in t:
                break
            if top.endswith(":"):
                continue
            if top in ASYNC:
                if _dest(t) & dst:
                    bad.append((line, t))
                rest = t.split(",", 1)[1] if "," in t else ""
                if _regs(rest) & dst:
                    bad.append((line, t))
                continue
            if _regs(t) & dst:
                bad.append((line, t))
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
