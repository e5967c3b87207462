"""Source checks of the HIP kernels (no GPU).

The HIP compiler of this toolchain evaluates __builtin_bit_cast of an
element of an ext_vector_type value (`v[e]`, constant or variable index) as
a bit_cast of element 0, on host and device alike: bit_cast(uint32_t, v[3])
gives v[0]'s bits. A copy of the element first (`const float x = v[e];` or
an explicit `(uint32_t)v[e]`) is compiled correctly. The first test shows
the behaviour on the host; the second keeps the pattern out of every
kernel source."""

import glob
import os
import re
import subprocess

from exact_attention_113_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
#include <cstdint>
#include <cstdio>
typedef float f32x4 __attribute__((ext_vector_type(4)));
__attribute__((noinline)) uint32_t direct(f32x4 v, int e) { return __builtin_bit_cast(uint32_t, v[e]); }
__attribute__((noinline)) uint32_t copied(f32x4 v, int e) { const float x = v[e]; return __builtin_bit_cast(uint32_t, x); }
int main() {
  f32x4 v = {1.0f, -2.0f, 3.0f, -4.0f};
  for (int e = 0; e < 4; ++e) printf("%08x %08x\n", direct(v, e), copied(v, e));
}
"""


def test_toolchain_vector_element_bit_cast(tmp_path):
    src = tmp_path / "probe.hip"
    src.write_text(PROBE)
    exe = str(tmp_path / "probe")
    res = subprocess.run([build.hipcc_path(), "-x", "hip", f"--offload-arch={build.ARCH}", "-O2",
                          str(src), "-o", exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True)
    assert res.returncode == 0, res.stdout
    rows = [line.split() for line in subprocess.check_output([exe], text=True).splitlines()]
    expect = ["3f800000", "c0000000", "40400000", "c0800000"]
    # The copied element is always right.
    assert [r[1] for r in rows] == expect
    # Record what the direct form gives with this toolchain (element 0 for
    # every index here); either way the sources must not use it.
    print("direct bit_cast of v[e]:", [r[0] for r in rows])


# __builtin_bit_cast(T, name[...]) with the element subscript as the whole
# operand (an explicit conversion such as (uint32_t)r[1] is a new value and
# is not matched).
PATTERN = re.compile(r"__builtin_bit_cast\(\s*[^,()]+,\s*[A-Za-z_][A-Za-z0-9_.]*\s*\[")


def test_no_bit_cast_of_a_vector_element_in_kernels():
    hits = []
    for path in sorted(glob.glob(os.path.join(build.CSRC, "*.hip")) +
                       glob.glob(os.path.join(build.CSRC, "*.h"))):
        with open(path) as f:
            for n, line in enumerate(f, 1):
                code = line.split("//")[0]
                if PATTERN.search(code):
                    hits.append(f"{os.path.basename(path)}:{n}: {line.strip()}")
    assert not hits, "bit_cast of a vector element:\n" + "\n".join(hits)


def test_pattern_matches_the_hazard():
    assert PATTERN.search("x = __builtin_bit_cast(uint32_t, p4[e]);")
    assert PATTERN.search("__builtin_bit_cast(f16x2, o[i])")
    assert not PATTERN.search("__builtin_bit_cast(float, (uint32_t)r[1])")
    assert not PATTERN.search("__builtin_bit_cast(u32x2, lo)")
