"""CPU test of the launch planner (glu_api.cpp) with a recording stub in
place of the kernel launch: tiling, 32-bit kernel index ranges and pointer
offsets for shapes from one element to beyond 2^33 elements."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mlp_gated_activation_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                                reason="needs g++ and the ROCm headers")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("plan") / "plan_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", f"-I{CSRC}",
                    "-I/opt/rocm/include", os.path.join(ROOT, "tests", "plan_check.cpp"),
                    os.path.join(CSRC, "glu_api.cpp"), "-o", exe], check=True)
    return exe


BIG = (1 << 33) + (1 << 20) + 3
CASES = [
    # direction layout dtype rows cols ld_in ld_out misalign
    ("fwd", 0, 2, 4096, 14336, 14336, 14336, 0),      # headline
    ("bwd", 0, 2, 4096, 14336, 14336, 14336, 0),
    ("fwd", 0, 2, 4096, 11008, 11008, 11008, 0),
    ("fwd", 1, 2, 4096, 14336, 28672, 14336, 0),      # [gate | up]
    ("bwd", 1, 2, 4096, 14336, 28672, 14336, 0),
    ("fwd", 1, 1, 8191, 18944, 37888, 18944, 0),      # odd rows
    ("bwd", 1, 1, 8191, 18944, 37888, 18944, 0),
    ("fwd", 0, 0, 64, 1024, 1024, 1024, 0),
    ("fwd", 0, 2, 1, BIG, BIG, BIG, 0),               # merged row beyond 2^33: column chunks
    ("bwd", 0, 2, 1, BIG, BIG, BIG, 0),
    ("fwd", 0, 2, 3, (1 << 32) + 5, (1 << 32) + 8, (1 << 32) + 8, 0),   # strided rows wider than 2^31
    ("fwd", 1, 2, (1 << 17) + 3, 1 << 16, 1 << 17, 1 << 16, 0),         # row chunks past 2^30 units
    ("bwd", 1, 2, (1 << 17) + 3, 1 << 16, 1 << 17, 1 << 16, 0),
    ("fwd", 0, 2, (1 << 17) + 3, 1 << 16, 1 << 16, 1 << 16, 1),         # element path, merged, 2^33
    ("fwd", 0, 1, 5, 3, 3, 3, 0), ("fwd", 0, 1, 1, 1, 1, 1, 0), ("fwd", 0, 0, 7, 9, 13, 11, 0),
    ("fwd", 1, 2, 3, 17, 40, 17, 0), ("bwd", 0, 2, 37, 1000, 3024, 1000, 1),
    ("fwd", 0, 2, 2, (1 << 31) + 1, (1 << 31) + 1, (1 << 31) + 1, 1),   # element path, long rows
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-L{c[1]}-D{c[2]}-{c[3]}x{c[4]}-m{c[7]}" for c in CASES])
def test_plan(checker, case):
    out = subprocess.run([checker, *map(str, case)], capture_output=True, text=True)
    assert out.stdout.startswith("ok"), out.stdout + out.stderr


def test_exact_inplace_alias_accepted(checker):
    # the alias check rejects partial overlaps (test_abi.py) but must let the
    # exact in-place cases through to the launch
    out = subprocess.run([checker, "inplace"], capture_output=True, text=True)
    assert out.stdout.startswith("ok 2"), out.stdout + out.stderr
