"""CPU test of the strided-operand planner (glu_fwd_strided / glu_bwd_strided
in glu_api.cpp) with recording stubs in place of the kernel launches: which
path each layout takes, full tile coverage with per-launch grid limits, and
the stride / alias rules, all before any HIP call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mlp_gated_activation_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                                reason="needs g++ and the ROCm headers")

OK, SHAPE, STRIDE, ALIAS = 0, 2, 3, 5


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("strided") / "strided_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", f"-I{CSRC}",
                    "-I/opt/rocm/include", os.path.join(ROOT, "tests", "strided_check.cpp"),
                    os.path.join(CSRC, "glu_api.cpp"), "-o", exe], check=True)
    return exe


R, C = 4096, 14336
RM = (C, 1)        # row-major (R, C)
CM = (1, R)        # column-major (R, C), i.e. a transposed (C, R) tensor
T20 = 1 << 20
CASES = {
    # name: (direction, dtype, rows, cols, [(rs, cs) per operand], extra specs, status, path)
    "all row-major": ("fwd", 2, R, C, [RM, RM, RM], [], OK, "rows"),
    "all column-major": ("fwd", 2, R, C, [CM, CM, CM], [], OK, "cols"),
    "column-major bwd": ("bwd", 1, R, C, [CM] * 5, [], OK, "cols"),
    "padded rows": ("fwd", 0, 37, 1000, [(1024, 1), (1000, 1), (3000, 1)], [], OK, "rows"),
    "transposed b": ("fwd", 2, R, C, [RM, CM, RM], [], OK, "tiles"),
    "transposed y": ("fwd", 2, R, C, [RM, RM, CM], [], OK, "tiles"),
    "transposed dy": ("bwd", 2, R, C, [RM, RM, CM, RM, RM], [], OK, "tiles"),
    "broadcast row of b": ("fwd", 2, 300, 512, [(512, 1), (0, 1), (512, 1)], [], OK, "tiles"),
    "per-row scalar b": ("fwd", 2, 300, 512, [(512, 1), (1, 0), (512, 1)], [], OK, "tiles"),
    "scalar b": ("fwd", 1, 65, 128, [(128, 1), (0, 0), (128, 1)], [], OK, "tiles"),
    "column slice stride 2": ("fwd", 2, 100, 304, [(608, 2), (304, 1), (304, 1)], [], OK, "tiles"),
    "ragged tiles": ("bwd", 0, 65, 127, [(128, 1), (1, 68), (128, 1), (1, 68), (128, 1)], [], OK, "tiles"),
    "unaligned strides": ("fwd", 2, 65, 127, [(127, 1), (1, 65), (127, 1)], [], OK, "tiles"),
    "gate_up halves in place": ("bwd", 2, 100, 200, [(400, 1), (400, 1), (200, 1), (400, 1), (400, 1)],
                                ["o0=i0", "i1+200", "o1+200"], OK, "rows"),
    "gate_up halves transposed dy": ("bwd", 2, 100, 200, [(400, 1), (400, 1), (1, 100), (400, 1), (400, 1)],
                                     ["o0=i0", "i1+200", "o1+200"], OK, "tiles"),
    "y over a, transposed": ("fwd", 2, 128, 200, [(1, 128), (200, 1), (1, 128)], ["o0=i0"], OK, "tiles"),
    "many tile launches": ("fwd", 2, T20, T20, [(T20, 1), (1, T20), (T20, 1)], [], OK, "tiles"),
    "empty": ("fwd", 2, 0, 5, [RM, RM, RM], [], OK, "none"),
    # rejects
    "negative stride": ("fwd", 2, 10, 10, [(10, 1), (-10, 1), (10, 1)], [], STRIDE, "none"),
    "y rows overlap": ("fwd", 2, 100, 200, [(200, 1), (200, 1), (100, 1)], [], STRIDE, "none"),
    "y broadcast": ("fwd", 2, 100, 200, [(200, 1), (200, 1), (0, 1)], [], STRIDE, "none"),
    "y shifted over a": ("fwd", 2, 100, 200, [(200, 1), (200, 1), (200, 1)], ["o0+1"], ALIAS, "none"),
    "y over a with other strides": ("fwd", 2, 100, 200, [(200, 1), (200, 1), (1, 100)], ["o0=i0"], ALIAS,
                                    "none"),
    "da overlaps db": ("bwd", 2, 100, 200, [(200, 1), (200, 1), (200, 1), (400, 1), (400, 1)],
                       ["o1+1", "o0+0"], ALIAS, "none"),
    "too many tiles": ("fwd", 2, 1 << 23, 1 << 23, [(1 << 23, 1), (1, 1 << 23), (1 << 23, 1)], [], SHAPE,
                       "none"),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_strided_plan(checker, name):
    d, dt, rows, cols, ops, extra, status, path = CASES[name]
    args = [checker, d, str(dt), str(rows), str(cols)]
    for rs, cs in ops:
        args += [str(rs), str(cs)]
    out = subprocess.run(args + extra, capture_output=True, text=True)
    assert not out.stdout.startswith("FAIL"), out.stdout + out.stderr
    got = out.stdout.split()
    assert int(got[0]) == status and got[1] == path, (name, out.stdout)
    if name == "many tile launches":
        assert int(got[2]) == (T20 // 64) ** 2 // (1 << 22)
    if name in MODES:
        assert got[3:] == MODES[name], (name, out.stdout)


# orientation and per-operand access modes (D: 16-byte chunks along the
# computed rows, T: 16-byte chunks turned around in LDS, G: element gather)
MODES = {
    "transposed b": ["keep", "DTD"],
    "transposed y": ["keep", "DDT"],
    "transposed dy": ["keep", "DDTDD"],
    "broadcast row of b": ["keep", "DDD"],          # stride-0 rows: chunks re-read from cache
    "per-row scalar b": ["keep", "DTD"],            # (1, 0) strides: chunks down the column
    "scalar b": ["keep", "DGD"],
    "column slice stride 2": ["keep", "GDD"],
    "ragged tiles": ["keep", "DTDTD"],
    "unaligned strides": ["keep", "GGG"],
    "y over a, transposed": ["flip", "DTD"],
}
