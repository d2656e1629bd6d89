"""The C-ABI library on the host: it loads, exports every symbol include/*.h declares, and
rejects bad arguments before anything reaches the GPU (no compute calls here)."""

import ctypes
import glob
import os
import re
import subprocess

import pytest

import grouped_nvfp4_w4a16_amd as pkg
from grouped_nvfp4_w4a16_amd import build as builder

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkg.LIB_PATH):
        builder.build()
    return pkg.load()


def _declared_functions():
    names = []
    for path in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M):
            names.append(m.group(1))
    return sorted(set(names))


def test_header_declares_the_four_calls_and_helpers():
    names = _declared_functions()
    for want in ("moe_align", "moe_w4a16_grouped_gemm", "swiglu_clamp", "moe_combine"):
        assert want in names
    assert sorted(pkg.EXPORTS) == names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", pkg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_library_was_built_from_these_sources(lib):
    """The source hash compiled into the library is the hash of the sources on disk, and
    load() refuses a library whose hash differs."""
    assert lib.moe_w4a16_source_sha256().decode() == builder.source_sha256()
    assert builder.built_source_sha256() == builder.source_sha256()
    assert len(builder.source_sha256()) == 64
    names = [os.path.relpath(p, ROOT) for p in builder.hashed_files()]
    assert "include/moe_w4a16.h" in names
    assert "grouped_nvfp4_w4a16_amd/csrc/grouped_gemm.hip" in names


def test_status_strings(lib):
    assert lib.moe_w4a16_status_string(0) == b"ok"
    assert lib.moe_w4a16_status_string(1) == b"invalid argument"
    assert lib.moe_w4a16_status_string(99) == b"unknown status"


def _bad(ptr=0x1000):
    return ctypes.c_void_p(ptr)


def test_invalid_arguments_are_rejected_on_the_host(lib):
    n = None
    # moe_align: negative rows, zero experts, too many experts, NULL offsets
    assert lib.moe_align(n, -1, 8, 16, n, n, _bad(), n, n, n, n) == 1
    assert lib.moe_align(n, 4, 8, 0, n, n, _bad(), n, n, n, n) == 1
    assert lib.moe_align(n, 4, 8, 4096, n, n, _bad(), n, n, n, n) == 1
    assert lib.moe_align(n, 4, 8, 16, n, n, n, n, n, n, n) == 1
    assert b"expert_offsets" in lib.moe_w4a16_last_error()
    # grouped GEMM: k not a multiple of 256, n not a multiple of 16, misaligned a, NULL table
    args = dict(a=_bad(), lda=512, a_rows=8, g=n, pp=_bad(), sp=_bad(), s2=_bad(), off=_bad(),
                e=4, c=_bad(), ldc=64, rows=8, nn=64, k=512)

    def gemm(**kw):
        a = {**args, **kw}
        return lib.moe_w4a16_grouped_gemm(a["a"], a["lda"], a["a_rows"], a["g"], a["pp"], a["sp"],
                                          a["s2"], a["off"], a["e"], n, n, a["c"], a["ldc"],
                                          a["rows"], a["nn"], a["k"], n)
    assert gemm(k=500) == 1
    assert gemm(nn=40) == 1
    assert gemm(a=_bad(0x1008)) == 1
    assert gemm(pp=n) == 1
    assert gemm(lda=256) == 1
    assert gemm(rows=0) == 0  # nothing to do: returns without a launch
    # swiglu: n not a multiple of 8, non-positive limit
    assert lib.swiglu_clamp(_bad(), _bad(), 16, _bad(), 16, 4, 12, 7.0, n) == 1
    assert lib.swiglu_clamp(_bad(), _bad(), 16, _bad(), 16, 4, 16, 0.0, n) == 1
    assert lib.swiglu_clamp(n, n, 16, n, 16, 0, 16, 7.0, n) == 0  # empty
    # combine: hidden not a multiple of 8, zero top_k
    assert lib.moe_combine(_bad(), 16, 4, _bad(), _bad(), n, 0, _bad(), 16, 4, 12, 2, n) == 1
    assert lib.moe_combine(_bad(), 16, 4, _bad(), _bad(), n, 0, _bad(), 16, 4, 16, 0, n) == 1
    # dequant: k not a multiple of 32
    assert lib.moe_w4a16_dequant_bf16(_bad(), _bad(), 1.0, _bad(), 4, 48, n) == 1
    # dense split-K: a workspace below the size query (capacity), one not 256-byte aligned
    need = lib.moe_dense_workspace_bytes(64, 128, 1024, 0)
    assert lib.moe_dense_gemm_bf16(_bad(), 1024, _bad(), 1024, _bad(), 128, 64, 128, 1024,
                                   _bad(), need - 1, n) == 2
    assert lib.moe_dense_gemm_bf16(_bad(), 1024, _bad(), 1024, _bad(), 128, 64, 128, 1024,
                                   _bad(0x1010), need, n) == 1
    # no-allocation dense GEMM: partials beyond the library's scratch (capacity), bad n
    big = lib.moe_dense_workspace_bytes(1024, 8320, 4096, 0)
    assert big > (32 << 20)
    assert lib.moe_dense_gemm_bf16_noalloc(_bad(), 4096, _bad(), 4096, _bad(), 8320, 1024, 8320,
                                           4096, n) == 2
    assert b"scratch" in lib.moe_w4a16_last_error()
    assert lib.moe_dense_gemm_bf16_noalloc(_bad(), 1024, _bad(), 1024, _bad(), 128, 64, 120,
                                           1024, n) == 1
    # HBM read probe: NULL buffer, bytes not a multiple of 16, misaligned, bad unroll
    assert lib.moe_hbm_read_probe(n, 1024, _bad(), 8, 8, n) == 1
    assert lib.moe_hbm_read_probe(_bad(), 1000, _bad(), 8, 8, n) == 1
    assert lib.moe_hbm_read_probe(_bad(0x1008), 1024, _bad(), 8, 8, n) == 1
    assert lib.moe_hbm_read_probe(_bad(), 1024, _bad(), 8, 5, n) == 1
    assert b"unroll" in lib.moe_w4a16_last_error()


def _splitk_bytes(m, n, k, swiglu):
    """The split-K workspace size from its definition: 128 x 128 FP32 per tile of 128 rows
    x 128 weight rows (64 output columns in the gate/up form) and K split; K splits 4 or
    2 ways (the most with every split at least 8 steps of 64 k per 128-row tile, the steps
    dividing evenly and at most 8 ways per row tile group: ways * ceil(m / 128) <= 8),
    else 1."""
    steps = k // 64
    row_tiles = -(-m // 128)
    ways = next((s for s in (4, 2)
                 if s * row_tiles <= 8 and steps % s == 0 and steps // s >= 8 * row_tiles), 1)
    tiles = row_tiles * -(-n // (64 if swiglu else 128))
    return tiles * ways * 128 * 128 * 4


@pytest.mark.parametrize("m,n,k,swiglu", [
    (256, 2048, 6144, 1), (256, 6144, 2048, 0), (1, 16, 64, 0), (130, 272, 1024, 0),
    (300, 4096, 512, 1), (8, 48, 0, 0), (4096, 16, 2560, 1), (40, 96, 320, 0),
    (70, 160, 704, 0)])
def test_dense_workspace_size_query(lib, m, n, k, swiglu):
    assert lib.moe_dense_workspace_bytes(m, n, k, swiglu) == _splitk_bytes(m, n, k, swiglu)
    assert lib.moe_dense_workspace_bytes(0, n, k, swiglu) == 0
