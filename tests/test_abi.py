"""CPU tests of the C-ABI boundary: the library loads, exports exactly what
include/glu.h declares, and rejects every invalid argument combination on
the host before any HIP call (nothing here launches a kernel)."""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "glu.h")
CSRC = os.path.join(ROOT, "mlp_gated_activation_amd", "csrc")

from conftest import ensure_built

ensure_built()
from mlp_gated_activation_amd import glu  # noqa: E402
lib = glu._lib

OK, NULL, SHAPE, STRIDE, ENUM, ALIAS, INPLACE, HIP, ARG = range(9)
P = 0x7f0000000000          # fake device addresses: validation never dereferences them
S, GU = 0, 1
F32, F16, BF16 = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"GLU_API\s+[\w\s\*]+?\b(glu_\w+)\s*\(", text)


def test_header_declarations_are_exported():
    names = declared_functions()
    assert set(names) == {"glu_fwd", "glu_bwd", "glu_fwd_strided", "glu_bwd_strided", "glu_gemm_fwd",
                          "glu_add_rmsnorm_fwd", "glu_status_string", "glu_version"}
    nm = subprocess.run(["nm", "-D", "--defined-only", glu.library_path()],
                        capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in nm.splitlines() if " T " in l}
    assert exported == set(names), exported


def test_reference_library_exports_its_header():
    """libglu_ref.so (the benchmark's data-movement reference kernels) exports
    exactly what include/glu_ref.h declares, and rejects bad arguments on the
    host before any launch."""
    import ctypes
    from mlp_gated_activation_amd import build
    text = open(os.path.join(ROOT, "include", "glu_ref.h")).read()
    names = set(re.findall(r"GLU_REF_API\s+int\s+(glu_ref_\w+)\s*\(", text))
    assert names == {"glu_ref_fwd_mix", "glu_ref_bwd_mix", "glu_ref_rms_mix", "glu_ref_copy", "glu_ref_tile_bwd_mix",
                     "glu_ref_tile_fwd_mix"}
    nm = subprocess.run(["nm", "-D", "--defined-only", build.REF_LIB], capture_output=True, text=True,
                        check=True).stdout
    assert {l.split()[-1] for l in nm.splitlines() if " T " in l} == names
    ref = ctypes.CDLL(build.REF_LIB)
    p, u64 = ctypes.c_void_p, ctypes.c_uint64
    ref.glu_ref_copy.argtypes = [p, p, u64, p]
    ref.glu_ref_fwd_mix.argtypes = [p, p, p, u64, p]
    assert ref.glu_ref_copy(None, P, 16, None) == -1          # NULL
    assert ref.glu_ref_copy(P + 8, P, 16, None) == -1         # unaligned
    assert ref.glu_ref_fwd_mix(P, P, P, 24, None) == -1       # not a multiple of 16 bytes
    ref.glu_ref_tile_fwd_mix.argtypes = [p, p, p, ctypes.c_int64, ctypes.c_int64, p]
    assert ref.glu_ref_tile_fwd_mix(P, P, P, 64, 100, None) == -1     # cols not a multiple of 64
    assert ref.glu_ref_tile_fwd_mix(P, P, P, 0, 64, None) == -1       # empty


def test_version_and_status_strings():
    assert glu.version() >> 16 == 1
    for s in range(9):
        assert len(glu.status_string(s)) > 5
    assert glu.status_string(99) == "unknown status"


def fwd(kind=0, layout=S, dtype=BF16, rows=4, cols=64, a=P, lda=64, b=P + (1 << 20), ldb=64,
        y=P + (2 << 20), ldy=64, inplace=0):
    return lib.glu_fwd(kind, layout, dtype, rows, cols, a, lda, b, ldb, y, ldy, inplace, None)


def bwd(kind=0, layout=S, dtype=BF16, rows=4, cols=64, a=P, lda=64, b=P + (1 << 20), ldb=64,
        dy=P + (2 << 20), lddy=64, da=P + (3 << 20), ldda=64, db=P + (4 << 20), lddb=64, inplace=0):
    return lib.glu_bwd(kind, layout, dtype, rows, cols, a, lda, b, ldb, dy, lddy, da, ldda, db, lddb,
                       inplace, None)


@pytest.mark.parametrize("args,want", [
    (dict(kind=4), ENUM), (dict(kind=-1), ENUM), (dict(layout=2), ENUM), (dict(dtype=3), ENUM),
    (dict(inplace=2), INPLACE), (dict(inplace=-1), INPLACE),
    (dict(rows=-1), SHAPE), (dict(cols=-5), SHAPE), (dict(rows=1 << 31), SHAPE),
    (dict(rows=0, a=None, b=None, y=None), OK), (dict(cols=0, a=None, b=None, y=None), OK),
    (dict(a=None), NULL), (dict(b=None), NULL), (dict(y=None), NULL),
    (dict(layout=GU, b=P + (1 << 20), lda=128), NULL),          # gate_up takes no b
    (dict(lda=63), STRIDE), (dict(ldb=10), STRIDE), (dict(ldy=0), STRIDE),
    (dict(layout=GU, b=None, lda=127), STRIDE),                  # x needs 2*cols
    (dict(inplace=1), INPLACE),                                  # y given with inplace
    (dict(inplace=1, y=None, b=P + 2), ALIAS),                   # y := b one element past a
    (dict(inplace=1, y=None, b=P + 2 * 63), ALIAS),              # y := b over a's last element
    (dict(inplace=1, y=None, b=P - 2 * 63 - 2 * 64 * 3), ALIAS),  # b's last row ends inside a's first
    (dict(inplace=1, y=None, b=P, ldb=128), ALIAS),              # same start, other stride
    (dict(rows=1 << 30, lda=1 << 40), SHAPE),                    # extent overflows int64
    (dict(cols=1 << 62, lda=1 << 62, ldb=1 << 62, ldy=1 << 62, rows=2), SHAPE),
    (dict(y=P + 2 * 2), ALIAS),                                  # y straddles a's rows
    (dict(y=P + (1 << 20) + 2 * 63), ALIAS),                     # y overlaps b's tail
    (dict(y=P, ldy=128), ALIAS),                                 # same start, other stride
    (dict(layout=GU, b=None, lda=128, y=P + 2 * 64 - 2, ldy=128), ALIAS),  # off by one element
    (dict(layout=GU, b=None, lda=128, y=P + 2 * 64, ldy=256, rows=2), ALIAS),
])
def test_fwd_rejects(args, want):
    assert fwd(**args) == want


@pytest.mark.parametrize("args,want", [
    (dict(kind=7), ENUM), (dict(inplace=3), INPLACE), (dict(rows=-2), SHAPE),
    (dict(rows=0, a=None, b=None, dy=None, da=None, db=None), OK),
    (dict(dy=None), NULL), (dict(da=None), NULL), (dict(db=None), NULL), (dict(a=None), NULL),
    (dict(lddy=1), STRIDE), (dict(ldda=3), STRIDE), (dict(lddb=63), STRIDE),
    (dict(inplace=1), INPLACE), (dict(inplace=1, da=None), INPLACE), (dict(inplace=1, db=None), INPLACE),
    (dict(db=P + (3 << 20)), ALIAS),                              # da == db exactly: two writers
    (dict(db=P + (3 << 20) + 2), ALIAS),                          # da, db overlap
    (dict(da=P + 2), ALIAS),                                      # da straddles a
    (dict(db=P + (2 << 20) + 64), ALIAS),                         # db overlaps dy partially
    (dict(layout=GU, b=None, lda=128, ldda=128), NULL),           # gate_up dx: db must be NULL
    (dict(layout=GU, b=None, lda=128, db=None, ldda=127), STRIDE),
    (dict(layout=GU, b=None, lda=128, db=None, da=P + 2, ldda=128), ALIAS),
    (dict(inplace=1, da=None, db=None, dy=P + 2), ALIAS),         # dy overlaps a, not exactly
])
def test_bwd_rejects(args, want):
    assert bwd(**args) == want


def sfwd(kind=0, dtype=BF16, rows=4, cols=64, a=P, ars=64, acs=1, b=P + (1 << 20), brs=64, bcs=1,
         y=P + (2 << 20), yrs=64, ycs=1):
    return lib.glu_fwd_strided(kind, dtype, rows, cols, a, ars, acs, b, brs, bcs, y, yrs, ycs, None)


def sbwd(kind=0, dtype=BF16, rows=4, cols=64, a=P, ars=64, acs=1, b=P + (1 << 20), brs=64, bcs=1,
         dy=P + (2 << 20), dyrs=64, dycs=1, da=P + (3 << 20), dars=64, dacs=1, db=P + (4 << 20), dbrs=64,
         dbcs=1):
    return lib.glu_bwd_strided(kind, dtype, rows, cols, a, ars, acs, b, brs, bcs, dy, dyrs, dycs,
                               da, dars, dacs, db, dbrs, dbcs, None)


@pytest.mark.parametrize("args,want", [
    (dict(kind=4), ENUM), (dict(dtype=-1), ENUM), (dict(rows=-1), SHAPE), (dict(cols=-1), SHAPE),
    (dict(rows=0, a=None, b=None, y=None), OK),
    (dict(a=None), NULL), (dict(b=None), NULL), (dict(y=None), NULL),
    (dict(ars=-64), STRIDE), (dict(bcs=-1), STRIDE), (dict(ycs=-1), STRIDE),
    (dict(yrs=32), STRIDE),                                    # rows of y overlap
    (dict(yrs=0), STRIDE), (dict(ycs=0), STRIDE),              # y broadcast
    (dict(yrs=1, ycs=1), STRIDE),
    (dict(a=P + 1), ARG), (dict(dtype=F32, y=P + (2 << 20) + 2), ARG),   # not element aligned
    (dict(rows=1 << 40, ars=1 << 30), SHAPE),                  # extent overflows
    (dict(y=P + 2), ALIAS),                                    # y one element past a
    (dict(y=P, yrs=1, ycs=4), ALIAS),                          # a's memory, other strides
    (dict(b=P + 64 * 2, y=P + 64 * 2 + 2, yrs=128, ars=128, brs=128), ALIAS),
    (dict(rows=1 << 23, cols=1 << 23, ars=1 << 23, brs=1, bcs=1 << 23, yrs=1 << 23, b=P + (1 << 48),
          y=P + (2 << 48)), SHAPE),                            # more than 2^32 tiles
])
def test_fwd_strided_rejects(args, want):
    # only rejected or empty calls here: an accepted call would launch a
    # kernel on the fake addresses (accepted layouts are covered by the
    # planner test with recording stubs)
    assert sfwd(**args) == want


@pytest.mark.parametrize("args,want", [
    (dict(kind=9), ENUM), (dict(dy=None), NULL), (dict(da=None), NULL), (dict(db=None), NULL),
    (dict(dyrs=-1), STRIDE), (dict(dars=0), STRIDE), (dict(dbrs=1, dbcs=1), STRIDE),
    (dict(db=P + (3 << 20)), ALIAS),                            # da == db
    (dict(da=P + (2 << 20) + 2), ALIAS),                        # da straddles dy
    (dict(da=P, dars=1, dacs=4), ALIAS),
    (dict(a=P, b=P + 128, ars=128, brs=128, da=P, dars=128, db=P + 126, dbrs=128), ALIAS),
    (dict(dy=P + (2 << 20) + 1), ARG),
])
def test_bwd_strided_rejects(args, want):
    assert sbwd(**args) == want


def gemm(kind=0, dtype=BF16, M=4, N=16, K=64, x=P, ldx=64, wg=P + (1 << 20), ldwg=64, wu=P + (2 << 20),
         ldwu=64, h=P + (3 << 20), ldh=16, gu=None, ldgu=0):
    return lib.glu_gemm_fwd(kind, dtype, M, N, K, x, ldx, wg, ldwg, wu, ldwu, h, ldh, gu, ldgu, None)


@pytest.mark.parametrize("args,want", [
    (dict(kind=4), ENUM), (dict(dtype=F32), ENUM), (dict(dtype=3), ENUM),
    (dict(M=-1), SHAPE), (dict(N=-1), SHAPE), (dict(K=-8), SHAPE), (dict(M=1 << 31), SHAPE),
    (dict(M=0, x=None, wg=None, wu=None, h=None), OK), (dict(N=0, h=None), OK),
    (dict(h=None), NULL), (dict(x=None), NULL), (dict(wg=None), NULL), (dict(wu=None), NULL),
    (dict(ldx=56), STRIDE), (dict(ldwg=8), STRIDE), (dict(ldh=15), STRIDE),
    (dict(gu=P + (4 << 20), ldgu=31), STRIDE),
    (dict(K=60, ldx=64), ARG),                              # K not a multiple of 8
    (dict(ldx=68), ARG), (dict(ldwu=72 + 4), ARG),          # row strides not 16-byte multiples
    (dict(x=P + 8), ARG), (dict(wg=P + (1 << 20) + 2), ARG),
    (dict(h=P + (3 << 20) + 1), ARG),
    (dict(M=1 << 20, N=1 << 20, ldh=1 << 20), SHAPE),      # more than 2^24 workgroup tiles
    (dict(h=P + 64), ALIAS),                                # h inside x
    (dict(h=P + (2 << 20) - 16), ALIAS),                    # h runs into w_up
    (dict(gu=P + (1 << 20), ldgu=32), ALIAS),               # gu over w_gate
    (dict(gu=P + (3 << 20) + 8, ldgu=32), ALIAS),           # gu over h
])
def test_gemm_rejects(args, want):
    # rejected or empty calls only: an accepted call would launch a kernel
    assert gemm(**args) == want


def rms(dtype=BF16, rows=4, hidden=64, x=P, ldx=64, r=P + (1 << 20), ldr=64, g=P + (2 << 20),
        h=P + (3 << 20), ldh=64, y=P + (4 << 20), ldy=64, rstd=P + (5 << 20), eps=1e-6):
    return lib.glu_add_rmsnorm_fwd(dtype, rows, hidden, x, ldx, r, ldr, g, h, ldh, y, ldy, rstd, eps, None)


@pytest.mark.parametrize("args,want", [
    (dict(dtype=3), ENUM), (dict(rows=-1), SHAPE), (dict(hidden=-1), SHAPE),
    (dict(eps=0.0), ARG), (dict(eps=-1e-6), ARG), (dict(eps=float("inf")), ARG), (dict(eps=float("nan")), ARG),
    (dict(rows=0, x=None, r=None, g=None, h=None, y=None), OK),
    (dict(rows=1 << 31), SHAPE), (dict(hidden=(1 << 31) + 1, ldx=1 << 32, ldr=1 << 32, ldh=1 << 32, ldy=1 << 32), SHAPE),
    (dict(x=None), NULL), (dict(r=None), NULL), (dict(g=None), NULL), (dict(h=None), NULL), (dict(y=None), NULL),
    (dict(ldx=63), STRIDE), (dict(ldr=1), STRIDE), (dict(ldh=0), STRIDE), (dict(ldy=60), STRIDE),
    (dict(h=P + 2), ALIAS),                              # h straddles x
    (dict(y=P + (1 << 20) + 64), ALIAS),                 # y overlaps residual partially
    (dict(h=P + (4 << 20)), ALIAS),                      # h == y: two outputs
    (dict(y=P + (2 << 20) - 64), ALIAS),                 # y runs into gamma
    (dict(rstd=P + 64), ALIAS),                          # rstd inside x
    (dict(rstd=P + (4 << 20) + 4), ALIAS),               # rstd inside y
    (dict(hidden=70000, ldx=70000, ldr=70000, ldh=70000, ldy=70000, h=P), ALIAS),  # two-pass: h over x
])
def test_add_rmsnorm_rejects(args, want):
    assert rms(**args) == want


def _compile_host(src: str, tmp: str) -> str:
    exe = os.path.join(tmp, "t")
    subprocess.run(["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{CSRC}",
                    "-I/opt/rocm/include", "-x", "c++", "-", "-o", exe], input=src, text=True, check=True)
    return exe


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_row_divider_is_exact():
    """The kernels divide unit indices by units-per-row with a multiply-high;
    check the host-computed constants against plain division for every
    divisor shape that matters and numerators up to 2^31."""
    src = r'''
#include "glu_internal.h"
#include <cstdio>
#include <random>
int main() {
  std::mt19937_64 rng(1);
  const uint32_t ds[] = {1, 2, 3, 5, 7, 8, 9, 128, 1376, 1792, 2368, 1000003, 65535, 65536, 65537,
                         (1u << 30) - 1, 1u << 30, 2147483647u};
  long bad = 0;
  for (uint32_t d : ds) {
    glu::Divider v = glu::make_divider(d);
    auto q = [&](uint32_t n) { return (uint32_t)((((uint64_t)n * v.magic) >> 32) + n) >> v.shift; };
    for (uint32_t n = 0; n < 200000; ++n) bad += q(n) != n / d;
    for (int i = 0; i < 2000000; ++i) { uint32_t n = rng() & 0x7fffffffu; bad += q(n) != n / d; }
    for (uint32_t k = 0; k < 4096; ++k) { uint64_t n = (uint64_t)d * k; if (n < (1ull << 31)) {
      bad += q((uint32_t)n) != k; if (n) bad += q((uint32_t)n - 1) != k - 1; } }
    bad += q(0x7fffffffu) != 0x7fffffffu / d;
  }
  printf("%ld\n", bad);
  return 0;
}'''
    with tempfile.TemporaryDirectory() as tmp:
        out = subprocess.run([_compile_host(src, tmp)], capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "0"


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_gemm_tile_order_is_a_bijection():
    """xcd_remap followed by grouped_coord (the GEMM's workgroup -> tile map)
    visits every (row tile, column tile) exactly once, for grids that do and
    do not divide by the 8 XCDs or the group height."""
    src = r"""
#include "glu_internal.h"
#include "gemm_internal.h"
#include <cstdio>
#include <vector>
int main() {
    int bad = 0;
    const unsigned shapes[][2] = {{16, 112}, {1, 1}, {1, 7}, {3, 5}, {5, 3}, {17, 9}, {33, 113}, {4, 8}, {7, 1},
                                  {2, 1000}, {1000, 2}, {13, 13}};
    for (auto &sh : shapes) {
        const unsigned tm = sh[0], tn = sh[1], n = tm * tn;
        std::vector<int> seen(n, 0);
        for (unsigned b = 0; b < n; ++b) {
            const unsigned l = glu::xcd_remap(b, n);
            if (l >= n) { ++bad; continue; }
            const glu::TileCoord c = glu::grouped_coord(l, tm, tn, glu::kGemmGroup);
            if (c.r >= tm || c.c >= tn) { ++bad; continue; }
            seen[c.r * tn + c.c]++;
        }
        for (int v : seen) bad += v != 1;
    }
    std::printf("%d\n", bad);
}
"""
    with tempfile.TemporaryDirectory() as tmp:
        out = subprocess.run([_compile_host(src, tmp)], capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "0"


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_kernel_isa():
    """The compiled gfx950 kernels: no MFMA and no packed fp32 ops anywhere,
    no fp64 in the bf16/fp16 kernels, and every vector kernel moves each of
    its streams with 16-byte loads/stores (GLU_UNROLL per thread)."""
    from mlp_gated_activation_amd import build as b
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [b.HIPCC, *[f for f in b.FLAGS if f not in ("-shared",)], f"-I{b.INCLUDE}", f"-I{b.CSRC}",
               "--save-temps", "-c", b.SOURCES[0], "-o", os.path.join(tmp, "k.o")]
        subprocess.run(cmd, cwd=tmp, check=True, capture_output=True)
        asm = open(os.path.join(tmp, "glu_kernels-hip-amdgcn-amd-amdhsa-gfx950.s")).read()
    unroll = int(re.search(r"#define GLU_UNROLL (\d+)", open(os.path.join(CSRC, "glu_internal.h")).read()).group(1))
    starts = [(m.start(), m.group(1)) for m in re.finditer(r"^(_Z\w*glu_kernel\w*):", asm, re.M)]
    # 3 dtypes x 4 kinds x vector/element x flat/strided, forward at one
    # block size and backward at two
    assert len(starts) == 144
    assert set(re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)) == {"0"}, "a kernel uses scratch"
    # every kernel of the library: no MFMA, no packed fp32
    for name in re.findall(r"^(_Z\w+):", asm, re.M):
        pos = asm.find(name + ":")
        body = asm[pos:asm.find("s_endpgm", pos)]
        assert "mfma" not in body and not re.search(r"v_pk_(add|mul|fma)_f32", body), name
    for pos, name in starts:
        body = asm[pos:asm.find("s_endpgm", pos)]
        assert "mfma" not in body, name
        assert not re.search(r"v_pk_(add|mul|fma)_f32", body), name
        m = re.search(r"glu_kernelINS0_(\w+?)ELi(\d)ELb(\d)ELb(\d)ELb(\d)E", name)
        storage, bwd, vec = m.group(1), m.group(3) == "1", m.group(4) == "1"
        if storage != "4SF32":
            assert not re.search(r"^\s+v_\w+_f64", body, re.M), name
        if vec:
            assert len(re.findall("global_load_dwordx4", body)) == unroll * (3 if bwd else 2), name
            assert len(re.findall("global_store_dwordx4", body)) == unroll * (2 if bwd else 1), name


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_tile_kernel_isa():
    """The LDS-tiled strided kernels: 24 instances (3 dtypes x 4 kinds x
    fwd/bwd), no scratch, no MFMA or packed fp32, and LDS sized at launch
    (no static LDS; the host asks for at most 3 slots of 64 x 65 floats)."""
    from mlp_gated_activation_amd import build as b
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [b.HIPCC, *[f for f in b.FLAGS if f not in ("-shared",)], f"-I{b.INCLUDE}", f"-I{b.CSRC}",
               "--save-temps", "-c", b.SOURCES[0], "-o", os.path.join(tmp, "k.o")]
        subprocess.run(cmd, cwd=tmp, check=True, capture_output=True)
        asm = open(os.path.join(tmp, "glu_kernels-hip-amdgcn-amd-amdhsa-gfx950.s")).read()
    names = re.findall(r"^(_Z\w*glu_tile_kernel\w*):", asm, re.M)
    assert len(names) == 24
    for name in names:
        pos = asm.find(name + ":")
        body = asm[pos:asm.find("s_endpgm", pos)]
        assert "mfma" not in body and not re.search(r"v_pk_(add|mul|fma)_f32", body), name
        assert "ds_write" in body and "ds_read" in body, name
    meta = asm[asm.find("amdhsa.kernels"):]
    for block in re.split(r"\n  - ", meta):
        if "glu_tile_kernel" in block:
            lds = int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", block).group(1))
            scratch = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))
            assert lds == 0 and scratch == 0, block[:200]


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_gemm_kernel_isa():
    """The gate/up GEMM kernels: 16 instances (bf16/fp16 x 4 kinds x the
    large and small tile configurations), MFMA in the k loop, no scratch, no
    packed fp32, LDS within the 160 KiB of a CU."""
    from mlp_gated_activation_amd import build as b
    src = [s for s in b.SOURCES if s.endswith("gemm_kernels.hip")][0]
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [b.HIPCC, *[f for f in b.FLAGS if f not in ("-shared",)], f"-I{b.INCLUDE}", f"-I{b.CSRC}",
               "--save-temps", "-c", src, "-o", os.path.join(tmp, "k.o")]
        subprocess.run(cmd, cwd=tmp, check=True, capture_output=True)
        asm = open(os.path.join(tmp, "gemm_kernels-hip-amdgcn-amd-amdhsa-gfx950.s")).read()
    names = re.findall(r"^(_Z\w*gemm_glu_kernel\w*):", asm, re.M)
    assert len(names) == 16
    for name in names:
        pos = asm.find(name + ":")
        body = asm[pos:asm.find("s_endpgm", pos)]
        assert re.search(r"v_mfma_f32_32x32x16_(bf16|f16)", body), name
        assert not re.search(r"v_pk_(add|mul|fma)_f32", body), name
    meta = asm[asm.find("amdhsa.kernels"):]
    for block in re.split(r"\n  - ", meta):
        if "gemm_glu_kernel" in block:
            lds = int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", block).group(1))
            scratch = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))
            assert 0 < lds <= 160 * 1024 and scratch == 0, block[:200]


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_rmsnorm_kernel_isa():
    """The add+RMSNorm kernels: no MFMA or packed fp32, no fp64 outside the
    fp32-data instances, 16-byte vector I/O on the aligned path."""
    from mlp_gated_activation_amd import build as b
    src = [s for s in b.SOURCES if s.endswith("rmsnorm_kernels.hip")][0]
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [b.HIPCC, *[f for f in b.FLAGS if f not in ("-shared",)], f"-I{b.INCLUDE}", f"-I{b.CSRC}",
               "--save-temps", "-c", src, "-o", os.path.join(tmp, "k.o")]
        subprocess.run(cmd, cwd=tmp, check=True, capture_output=True)
        asm = open(os.path.join(tmp, "rmsnorm_kernels-hip-amdgcn-amd-amdhsa-gfx950.s")).read()
    names = re.findall(r"^(_Z\w*rmsnorm\w*kernel\w*):", asm, re.M)
    # per dtype: 15 one-row shapes and the two-pass kernel, vector and element
    # paths, and 5 pipelined multi-row shapes (vector path only); for bf16 and
    # fp16 also the 64 x 8 shape with gamma loaded early
    assert len(names) == 3 * (2 * 16 + 5) + 2
    # the rows per CU the launcher assumes for the 64 x 8 shape: five waves
    # per SIMD (<= 96 VGPRs) with gamma late, four (97 .. 128) with it early
    meta = {m.group(1): int(m.group(2)) for m in
            re.finditer(r"\.name:\s+(_Z\w+)\s*\n(?:\s+\.[^\n]*\n)*?\s+\.vgpr_count:\s+(\d+)", asm)}
    for st in ("RBf16", "RF16"):
        late = [v for n, v in meta.items() if re.search(rf"add_rmsnorm_kernelINS0_{len(st)}{st}ELi64ELi8ELb1ELb0E", n)]
        early = [v for n, v in meta.items() if re.search(rf"add_rmsnorm_kernelINS0_{len(st)}{st}ELi64ELi8ELb1ELb1E", n)]
        assert len(late) == 1 and len(early) == 1, (st, late, early)
        assert late[0] <= 96 and 96 < early[0] <= 128, (st, late, early)
    # register arrays must stay in registers: no private (scratch) memory
    assert re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm) and \
        set(re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)) == {"0"}
    for name in names:
        pos = asm.find(name + ":")
        body = asm[pos:asm.find("s_endpgm", pos)]
        assert "mfma" not in body and not re.search(r"v_pk_(add|mul|fma)_f32", body), name
        if "RF32" not in name:
            assert not re.search(r"^\s+v_\w+_f64", body, re.M), name
        if (re.search(r"add_rmsnorm_kernelI\w+?ELi\d+ELi\d+ELb1ELb[01]E", name) or "rows_kernel" in name
                or re.search(r"loop_kernelI\w+?ELb1EEEvNS_7RmsArgsE", name)):   # VEC instances
            assert "global_load_dwordx4" in body and "global_store_dwordx4" in body, name
