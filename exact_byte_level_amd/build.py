"""Build libtt.so (HIP for gfx950) in-tree.

    python -m exact_byte_level_amd.build

Steps: generate the Unicode class table from the ``regex`` module's tables
(csrc/gen_unicode_table.py -> csrc/_gen/unicode_table.inc), then compile the
kernels and the C-ABI host code with hipcc into exact_byte_level_amd/libtt.so.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
GEN = os.path.join(CSRC, "_gen")
LIB = os.path.join(HERE, "libtt.so")
ARCH = os.environ.get("TT_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "--offload-arch=" + ARCH, "-std=c++17", "-fPIC", "-shared",
    # packed-FP32 instructions off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose=False):
    os.makedirs(GEN, exist_ok=True)
    inc = os.path.join(GEN, "unicode_table.inc")
    subprocess.check_call([sys.executable, os.path.join(CSRC, "gen_unicode_table.py"), inc])
    tmp = LIB + ".tmp"
    cmd = ["hipcc"] + HIPCC_FLAGS + [
        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", GEN,
        os.path.join(CSRC, "tt_kernels.hip"), os.path.join(CSRC, "tt_api.cpp"),
        "-o", tmp,
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
