"""CPU tier of the C ABI: the library loads, exports every entry point its
header declares, and rejects bad arguments on the host (status codes) before
any HIP call. No compute call is made here (there is no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qwg.h")


@pytest.fixture(scope="module")
def L():
    from quantized_weight_decode_gemv_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        from quantized_weight_decode_gemv_amd import build
        build.build()
    return _binding.lib()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qwg_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for want in ("qwg_dequant_q4k", "qwg_dequant_iq3", "qwg_gemv_q4k", "qwg_gemv_iq3",
                 "qwg_gemm_q4k", "qwg_strerror", "qwg_row_bytes", "qwg_version",
                 "qwg_plan_splits", "qwg_gemm_q4k_ex", "qwg_gemv_iq3_ex", "qwg_group_create_q4k",
                 "qwg_group_create_iq3", "qwg_group_run", "qwg_group_workgroups",
                 "qwg_group_destroy", "qwg_tiled_bytes", "qwg_pack_q4k_tiles",
                 "qwg_gemv_q4k_tiled", "qwg_group_create_q4k_tiled", "qwg_pack_iq3_tiles",
                 "qwg_gemv_iq3_tiled", "qwg_group_create_iq3_tiled", "qwg_dequant_iq3_xxs",
                 "qwg_gemv_iq3_xxs", "qwg_pack_iq3_xxs_tiles", "qwg_dequant_iq3s",
                 "qwg_dequant_iq4xs", "qwg_pack_iq3s_tiles", "qwg_pack_iq4xs_tiles",
                 "qwg_gemv_iq3s_tiled", "qwg_gemv_iq4xs_tiled", "qwg_group_create_iq3s_tiled",
                 "qwg_gemv_iq3s", "qwg_gemv_iq4xs", "qwg_group_create_iq3s",
                 "qwg_group_create_iq4xs",
                 "qwg_group_create_iq4xs_tiled", "qwg_encode_iq3",
                 "qwg_group_create_q4k_batched", "qwg_group_create_q4k_batched_tiled",
                 "qwg_gemm_q4k_tiled", "qwg_gemm_q4k_noalloc", "qwg_workspace_reserve",
                 "qwg_chain_create_q4k", "qwg_chain_run", "qwg_chain_status", "qwg_chain_phases",
                 "qwg_chain_destroy", "qwg_chain_tagged",
                 "qwg_workspace_release"):
        assert want in names


def test_library_exports_every_declared_symbol(L):
    from quantized_weight_decode_gemv_amd import _binding
    out = subprocess.run(["nm", "-D", "--defined-only", _binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qwg_[a-z0-9_]+)$", out, flags=re.M))
    for name in declared_symbols():
        assert name in exported, name
        assert hasattr(L, name)


def test_version_and_strerror(L):
    assert L.qwg_version() >= 100
    for st in range(0, 11):
        assert len(L.qwg_strerror(st)) > 0


def test_row_bytes(L):
    assert L.qwg_row_bytes(0, 2048) == 8 * 144 == 1152
    assert L.qwg_row_bytes(0, 5632) == 3168
    assert L.qwg_row_bytes(1, 2048) == 784
    assert L.qwg_row_bytes(1, 5632) == 2156
    assert L.qwg_row_bytes(0, 300) == -2
    assert L.qwg_row_bytes(2, 2048) == 784       # IQ3_XXS: the same 98-byte blocks
    assert L.qwg_row_bytes(2, 5632) == 2156
    assert L.qwg_row_bytes(3, 2048) == 880         # IQ3_S
    assert L.qwg_row_bytes(4, 5632) == 22 * 136    # IQ4_XS
    assert L.qwg_row_bytes(5, 256) == -6
    assert L.qwg_row_bytes(7, 256) == -6


def test_tiled_bytes(L):
    assert L.qwg_tiled_bytes(0, 2048, 2048) == 2048 * 1152
    assert L.qwg_tiled_bytes(0, 2048, 65) == 128 * 1152      # rows rounded up to whole tiles
    assert L.qwg_tiled_bytes(0, 5632, 1) == 64 * 3168
    assert L.qwg_tiled_bytes(1, 2048, 64) == 64 * 8 * 102     # IQ3: the implied signs written out
    assert L.qwg_tiled_bytes(1, 2048, 65) == 128 * 8 * 102
    assert L.qwg_tiled_bytes(2, 2048, 65) == 128 * 8 * 102
    assert L.qwg_tiled_bytes(3, 2048, 65) == 128 * 8 * 110
    assert L.qwg_tiled_bytes(4, 512, 1) == 64 * 2 * 136
    assert L.qwg_tiled_bytes(5, 2048, 64) == -6
    assert L.qwg_tiled_bytes(0, 300, 64) == -2


def test_plan_splits(L):
    # small row counts split the n_in sum; large ones do not; splits <= blocks per row
    assert L.qwg_plan_splits(0, 2048, 256) == 8
    assert L.qwg_plan_splits(0, 2048, 2048) == 8
    assert 1 <= L.qwg_plan_splits(0, 2048, 32000) <= 8
    assert L.qwg_plan_splits(0, 256, 1 << 20) == 1
    assert L.qwg_plan_splits(0, 257, 64) == -2
    assert L.qwg_plan_splits(0, 65536 + 256, 64) == -2
    assert L.qwg_plan_splits(5, 256, 64) == -6


FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("call,status", [
    # NULL pointers -> 1
    (lambda L: L.qwg_gemv_q4k(None, FAKE, FAKE, 256, 1, None), 1),
    (lambda L: L.qwg_gemv_q4k(FAKE, None, FAKE, 256, 1, None), 1),
    (lambda L: L.qwg_gemv_q4k(FAKE, FAKE, None, 256, 1, None), 1),
    (lambda L: L.qwg_gemv_iq3(FAKE, FAKE, FAKE, None, 256, 1, None), 1),
    (lambda L: L.qwg_gemm_q4k(None, FAKE, FAKE, 256, 1, 2, None), 1),
    (lambda L: L.qwg_dequant_q4k(None, FAKE, 256, None), 1),
    (lambda L: L.qwg_dequant_iq3(FAKE, None, FAKE, 256, None), 1),
    # shapes -> 2
    (lambda L: L.qwg_gemv_q4k(FAKE, FAKE, FAKE, 300, 1, None), 2),
    (lambda L: L.qwg_gemv_q4k(FAKE, FAKE, FAKE, 0, 1, None), 2),
    (lambda L: L.qwg_gemv_q4k(FAKE, FAKE, FAKE, 256, 0, None), 2),
    (lambda L: L.qwg_gemv_q4k(FAKE, FAKE, FAKE, 65536 + 256, 1, None), 2),
    (lambda L: L.qwg_gemv_q4k(FAKE, FAKE, FAKE, 256, (1 << 24) + 1, None), 2),
    (lambda L: L.qwg_gemv_iq3(FAKE, FAKE, FAKE, FAKE, 128, 4, None), 2),
    (lambda L: L.qwg_dequant_q4k(FAKE, FAKE, 255, None), 2),
    (lambda L: L.qwg_dequant_iq3(FAKE, FAKE, FAKE, -256, None), 2),
    (lambda L: L.qwg_gemm_q4k_ex(None, FAKE, FAKE, 256, 1, 1, 4, 1, None), 1),
    (lambda L: L.qwg_gemm_q4k_ex(FAKE, FAKE, FAKE, 200, 1, 1, 4, 1, None), 2),
    (lambda L: L.qwg_gemm_q4k_ex(FAKE, FAKE, FAKE, 256, 1, 9, 4, 1, None), 4),
    (lambda L: L.qwg_gemm_q4k_ex(FAKE, FAKE + 4, FAKE, 256, 1, 1, 4, 1, None), 3),
    # matrix-core engine (waves = 1) needs batch >= 2; other wave counts are invalid
    (lambda L: L.qwg_gemm_q4k_ex(FAKE, FAKE, FAKE, 256, 1, 1, 1, 1, None), 2),
    (lambda L: L.qwg_gemm_q4k_ex(FAKE, FAKE, FAKE, 256, 1, 2, 5, 1, None), 2),
    (lambda L: L.qwg_gemm_q4k_ex(FAKE, FAKE, FAKE, 256, 1, 1, 3, 1, None), 2),   # stream: batch >= 2
    (lambda L: L.qwg_gemm_q4k_ex(FAKE, FAKE, FAKE, 512, 1, 2, 3, 3, None), 2),
    (lambda L: L.qwg_gemm_q4k_ex(FAKE, FAKE, FAKE, 512, 1, 2, 1, 3, None), 2),
    (lambda L: L.qwg_gemm_q4k_ex(FAKE, FAKE, FAKE, 256, 1, 1, 2, 1, None), 2),
    (lambda L: L.qwg_gemm_q4k_ex(FAKE, FAKE, FAKE, 512, 1, 2, 2, 3, None), 2),
    # batch -> 4
    (lambda L: L.qwg_gemm_q4k(FAKE, FAKE, FAKE, 256, 1, 0, None), 4),
    (lambda L: L.qwg_gemm_q4k(FAKE, FAKE, FAKE, 256, 1, 9, None), 4),
    # alignment -> 3
    (lambda L: L.qwg_gemv_q4k(FAKE, FAKE, FAKE + 8, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_q4k(FAKE, FAKE + 4, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_q4k(FAKE + 2, FAKE, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq3(FAKE, FAKE, FAKE + 1, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq3(FAKE, FAKE, FAKE, FAKE + 4, 256, 1, None), 3),
    (lambda L: L.qwg_dequant_q4k(FAKE + 4, FAKE, 256, None), 3),
    (lambda L: L.qwg_dequant_q4k(FAKE, FAKE + 4, 256, None), 3),
    (lambda L: L.qwg_dequant_iq3(FAKE + 1, FAKE, FAKE, 256, None), 3),
    # tile layout
    (lambda L: L.qwg_pack_q4k_tiles(None, FAKE, 256, 1, None), 1),
    (lambda L: L.qwg_pack_q4k_tiles(FAKE, FAKE, 300, 1, None), 2),
    (lambda L: L.qwg_pack_q4k_tiles(FAKE + 8, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_pack_q4k_tiles(FAKE, FAKE + 4, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_q4k_tiled(FAKE, FAKE, None, 256, 1, None), 1),
    (lambda L: L.qwg_gemv_q4k_tiled(FAKE, FAKE, FAKE, 256, 0, None), 2),
    (lambda L: L.qwg_gemv_q4k_tiled(FAKE, FAKE, FAKE + 8, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_q4k_tiled(FAKE, FAKE + 4, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_pack_iq3_tiles(FAKE, None, 256, 1, None), 1),
    (lambda L: L.qwg_pack_iq3_tiles(FAKE, FAKE, 256, 0, None), 2),
    (lambda L: L.qwg_pack_iq3_tiles(FAKE + 2, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_pack_iq3_tiles(FAKE, FAKE + 1, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq3_tiled(FAKE, FAKE, FAKE, None, 256, 1, None), 1),
    (lambda L: L.qwg_gemv_iq3_tiled(FAKE, FAKE, FAKE, FAKE, 100, 1, None), 2),
    (lambda L: L.qwg_gemv_iq3_tiled(FAKE, FAKE, FAKE + 2, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq3_tiled(FAKE, FAKE, FAKE, FAKE + 8, 256, 1, None), 3),
    # IQ3_XXS (llama.cpp byte order): the same rules as the container entry points
    (lambda L: L.qwg_dequant_iq3_xxs(None, FAKE, FAKE, 256, None), 1),
    (lambda L: L.qwg_dequant_iq3_xxs(FAKE, None, FAKE, 256, None), 1),
    (lambda L: L.qwg_dequant_iq3_xxs(FAKE, FAKE, FAKE, 100, None), 2),
    (lambda L: L.qwg_dequant_iq3_xxs(FAKE + 1, FAKE, FAKE, 256, None), 3),
    (lambda L: L.qwg_dequant_iq3_xxs(FAKE, FAKE + 4, FAKE, 256, None), 3),
    (lambda L: L.qwg_dequant_iq3_xxs(FAKE, FAKE, FAKE + 4, 256, None), 3),
    (lambda L: L.qwg_gemv_iq3_xxs(FAKE, FAKE, FAKE, None, 256, 1, None), 1),
    (lambda L: L.qwg_gemv_iq3_xxs(None, FAKE, FAKE, FAKE, 256, 1, None), 1),
    (lambda L: L.qwg_gemv_iq3_xxs(FAKE, FAKE, FAKE, FAKE, 384, 1, None), 2),
    (lambda L: L.qwg_gemv_iq3_xxs(FAKE, FAKE, FAKE, FAKE, 256, 0, None), 2),
    (lambda L: L.qwg_gemv_iq3_xxs(FAKE, FAKE, FAKE + 1, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq3_xxs(FAKE, FAKE + 4, FAKE, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq3_xxs(FAKE, FAKE, FAKE, FAKE + 4, 256, 1, None), 3),
    (lambda L: L.qwg_pack_iq3_xxs_tiles(None, FAKE, 256, 1, None), 1),
    (lambda L: L.qwg_pack_iq3_xxs_tiles(FAKE, FAKE, 0, 1, None), 2),
    (lambda L: L.qwg_pack_iq3_xxs_tiles(FAKE + 4, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_pack_iq3_xxs_tiles(FAKE, FAKE + 1, 256, 1, None), 3),
    # the allocation-free GEMM: the same validation as qwg_gemm_q4k
    (lambda L: L.qwg_gemm_q4k_noalloc(None, FAKE, FAKE, 256, 1, 1, None), 1),
    (lambda L: L.qwg_gemm_q4k_noalloc(FAKE, FAKE, FAKE, 300, 1, 1, None), 2),
    (lambda L: L.qwg_gemm_q4k_noalloc(FAKE, FAKE, FAKE, 256, 0, 1, None), 2),
    (lambda L: L.qwg_gemm_q4k_noalloc(FAKE, FAKE, FAKE, 256, 1, 0, None), 4),
    (lambda L: L.qwg_gemm_q4k_noalloc(FAKE, FAKE, FAKE, 256, 1, 9, None), 4),
    (lambda L: L.qwg_gemm_q4k_noalloc(FAKE, FAKE + 4, FAKE, 256, 1, 1, None), 3),
    (lambda L: L.qwg_gemm_q4k_noalloc(FAKE, FAKE, FAKE + 8, 256, 1, 1, None), 3),
    # IQ3 encoder
    (lambda L: L.qwg_encode_iq3(None, FAKE, FAKE, 1, 256, None), 1),
    (lambda L: L.qwg_encode_iq3(FAKE, None, FAKE, 1, 256, None), 1),
    (lambda L: L.qwg_encode_iq3(FAKE, FAKE, None, 1, 256, None), 1),
    (lambda L: L.qwg_encode_iq3(FAKE, FAKE, FAKE, 0, 256, None), 2),
    (lambda L: L.qwg_encode_iq3(FAKE, FAKE, FAKE, 1, 300, None), 2),
    (lambda L: L.qwg_encode_iq3(FAKE, FAKE + 2, FAKE, 1, 256, None), 3),
    (lambda L: L.qwg_encode_iq3(FAKE, FAKE, FAKE + 4, 1, 256, None), 3),
    # IQ3_S / IQ4_XS
    (lambda L: L.qwg_dequant_iq3s(None, FAKE, FAKE, 256, None), 1),
    (lambda L: L.qwg_dequant_iq3s(FAKE, FAKE, FAKE, 257, None), 2),
    (lambda L: L.qwg_dequant_iq3s(FAKE + 1, FAKE, FAKE, 256, None), 3),
    (lambda L: L.qwg_dequant_iq3s(FAKE, FAKE + 4, FAKE, 256, None), 3),
    (lambda L: L.qwg_dequant_iq4xs(FAKE, None, FAKE, 256, None), 1),
    (lambda L: L.qwg_dequant_iq4xs(FAKE + 2, FAKE, FAKE, 256, None), 3),
    (lambda L: L.qwg_dequant_iq4xs(FAKE, FAKE, FAKE + 8, 256, None), 3),
    (lambda L: L.qwg_pack_iq3s_tiles(None, FAKE, 256, 1, None), 1),
    (lambda L: L.qwg_pack_iq3s_tiles(FAKE, FAKE, 300, 1, None), 2),
    (lambda L: L.qwg_pack_iq3s_tiles(FAKE + 8, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_pack_iq4xs_tiles(FAKE, FAKE + 1, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq3s_tiled(FAKE, FAKE, FAKE, None, 256, 1, None), 1),
    (lambda L: L.qwg_gemv_iq3s_tiled(FAKE, FAKE, FAKE, FAKE, 256, 0, None), 2),
    (lambda L: L.qwg_gemv_iq3s_tiled(FAKE, FAKE, FAKE + 2, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq4xs_tiled(FAKE, FAKE + 4, FAKE, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq4xs_tiled(FAKE, FAKE, FAKE, FAKE + 4, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq4xs_tiled(None, FAKE, FAKE, FAKE, 256, 1, None), 1),
    # row-major IQ3_S / IQ4_XS: weights 16-byte aligned like the tile layout
    (lambda L: L.qwg_gemv_iq3s(FAKE, FAKE, FAKE, None, 256, 1, None), 1),
    (lambda L: L.qwg_gemv_iq3s(FAKE, FAKE, None, FAKE, 256, 1, None), 1),
    (lambda L: L.qwg_gemv_iq3s(FAKE, FAKE, FAKE, FAKE, 384, 1, None), 2),
    (lambda L: L.qwg_gemv_iq3s(FAKE, FAKE, FAKE, FAKE, 256, 0, None), 2),
    (lambda L: L.qwg_gemv_iq3s(FAKE, FAKE, FAKE + 2, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq3s(FAKE, FAKE + 4, FAKE, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq3s(FAKE + 2, FAKE, FAKE, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq4xs(FAKE, FAKE, FAKE + 8, FAKE, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq4xs(FAKE, FAKE, FAKE, FAKE + 4, 256, 1, None), 3),
    (lambda L: L.qwg_gemv_iq4xs(None, FAKE, FAKE, FAKE, 256, 1, None), 1),
    # IQ3 with an explicit decomposition
    (lambda L: L.qwg_gemv_iq3_ex(FAKE, FAKE, FAKE, None, 256, 1, 4, 1, None), 1),
    (lambda L: L.qwg_gemv_iq3_ex(FAKE, FAKE, FAKE, FAKE, 384, 1, 4, 1, None), 2),
    (lambda L: L.qwg_gemv_iq3_ex(FAKE, FAKE, FAKE, FAKE, 256, 1, 2, 1, None), 2),
    (lambda L: L.qwg_gemv_iq3_ex(FAKE, FAKE, FAKE, FAKE, 256, 1, 32, 1, None), 2),
    (lambda L: L.qwg_gemv_iq3_ex(FAKE, FAKE, FAKE, FAKE, 512, 1, 4, 3, None), 2),
    (lambda L: L.qwg_gemv_iq3_ex(FAKE, FAKE, FAKE, FAKE, 512, 1, 4, -1, None), 2),
    (lambda L: L.qwg_gemv_iq3_ex(FAKE, FAKE, FAKE + 3, FAKE, 256, 1, 4, 1, None), 3),
    (lambda L: L.qwg_gemv_iq3_ex(FAKE, FAKE + 8, FAKE, FAKE, 256, 1, 4, 1, None), 3),
    (lambda L: L.qwg_gemv_iq3_ex(FAKE, FAKE, FAKE, FAKE + 8, 256, 1, 4, 1, None), 3),
])
def test_validation_errors(L, call, status):
    assert call(L) == status


class _Desc(ctypes.Structure):
    _fields_ = [("y", ctypes.c_void_p), ("x", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("n_in", ctypes.c_int64), ("n_out", ctypes.c_int64)]


@pytest.mark.parametrize("desc,status", [
    ((0, FAKE, FAKE, 256, 1), 1),
    ((FAKE, FAKE, FAKE, 300, 1), 2),
    ((FAKE, FAKE, FAKE, 256, 0), 2),
    ((FAKE, FAKE + 4, FAKE, 256, 1), 3),
    ((FAKE, FAKE, FAKE + 8, 256, 1), 3),
    ((FAKE + 2, FAKE, FAKE, 256, 1), 3),
])
def test_group_validation_errors(L, desc, status):
    arr = (_Desc * 2)(_Desc(FAKE, FAKE, FAKE, 256, 64), _Desc(*desc))
    out = ctypes.c_void_p(123)
    assert L.qwg_group_create_q4k(arr, 2, ctypes.byref(out)) == status
    assert out.value is None  # nothing allocated, handle cleared


@pytest.mark.parametrize("desc,status", [
    ((0, FAKE, FAKE, 256, 1), 1),
    ((FAKE, FAKE, FAKE, 300, 1), 2),
    ((FAKE, FAKE + 4, FAKE, 256, 1), 3),
    ((FAKE, FAKE, FAKE + 1, 256, 1), 3),   # IQ3 weights need only 2-byte alignment
    ((FAKE + 2, FAKE, FAKE, 256, 1), 3),
])
def test_iq3_group_validation_errors(L, desc, status):
    arr = (_Desc * 2)(_Desc(FAKE, FAKE, FAKE + 2, 256, 64), _Desc(*desc))
    out = ctypes.c_void_p(123)
    assert L.qwg_group_create_iq3(arr, 2, FAKE, ctypes.byref(out)) == status
    assert out.value is None
    ok = (_Desc * 1)(_Desc(FAKE, FAKE, FAKE + 2, 256, 64))
    assert L.qwg_group_create_iq3(ok, 1, None, ctypes.byref(out)) == 1
    assert L.qwg_group_create_iq3(ok, 1, FAKE + 4, ctypes.byref(out)) == 3
    assert L.qwg_group_create_iq3(ok, 0, FAKE, ctypes.byref(out)) == 2


def test_tiled_group_validation_errors(L):
    arr = (_Desc * 2)(_Desc(FAKE, FAKE, FAKE, 256, 64), _Desc(FAKE, FAKE, FAKE + 8, 256, 1))
    out = ctypes.c_void_p(123)
    assert L.qwg_group_create_q4k_tiled(arr, 2, ctypes.byref(out)) == 3
    assert out.value is None
    # IQ3 tile layout: 16-byte aligned weights (row-major IQ3 accepts 2-byte)
    arr3 = (_Desc * 1)(_Desc(FAKE, FAKE, FAKE + 2, 256, 1))
    assert L.qwg_group_create_iq3_tiled(arr3, 1, FAKE, ctypes.byref(out)) == 3
    assert L.qwg_group_create_iq3_tiled(arr3, 1, None, ctypes.byref(out)) == 1
    assert L.qwg_group_create_q4k_tiled(None, 1, ctypes.byref(out)) == 1
    assert L.qwg_group_create_q4k_tiled(arr, 0, ctypes.byref(out)) == 2
    # IQ3_S / IQ4_XS tiled groups: the same member rules, plus the grid/table
    for create in (L.qwg_group_create_iq3s_tiled, L.qwg_group_create_iq4xs_tiled,
                   L.qwg_group_create_iq3s, L.qwg_group_create_iq4xs):
        assert create(arr3, 1, FAKE, ctypes.byref(out)) == 3
        assert create(arr3, 1, None, ctypes.byref(out)) == 1
        assert create(arr, 2, FAKE + 4, ctypes.byref(out)) == 3
        assert create(arr, 0, FAKE, ctypes.byref(out)) == 2
        assert out.value is None


def test_gemm_tiled_validation_errors(L):
    f = L.qwg_gemm_q4k_tiled
    assert f(None, FAKE, FAKE, 256, 1, 2, None) == 1
    assert f(FAKE, FAKE, FAKE, 300, 1, 2, None) == 2
    assert f(FAKE, FAKE, FAKE, 256, 0, 2, None) == 2
    for batch in (0, 9):
        assert f(FAKE, FAKE, FAKE, 256, 1, batch, None) == 4
    assert f(FAKE, FAKE + 4, FAKE, 256, 1, 2, None) == 3
    assert f(FAKE, FAKE, FAKE + 8, 256, 1, 2, None) == 3
    out = ctypes.c_void_p(123)
    ok = (_Desc * 1)(_Desc(FAKE, FAKE, FAKE, 256, 64))
    for batch in (1, 9):
        assert L.qwg_group_create_q4k_batched_tiled(ok, 1, batch, ctypes.byref(out)) == 4
    bad = (_Desc * 1)(_Desc(FAKE, FAKE, FAKE + 8, 256, 64))
    assert L.qwg_group_create_q4k_batched_tiled(bad, 1, 4, ctypes.byref(out)) == 3
    assert out.value is None


def test_batched_group_validation_errors(L):
    out = ctypes.c_void_p(123)
    ok = (_Desc * 1)(_Desc(FAKE, FAKE, FAKE, 256, 64))
    assert L.qwg_group_create_q4k_batched(None, 1, 4, ctypes.byref(out)) == 1
    assert L.qwg_group_create_q4k_batched(ok, 1, 4, None) == 1
    assert L.qwg_group_create_q4k_batched(ok, 0, 4, ctypes.byref(out)) == 2
    for batch in (-1, 0, 1, 9):
        assert L.qwg_group_create_q4k_batched(ok, 1, batch, ctypes.byref(out)) == 4
    for desc, status in [((0, FAKE, FAKE, 256, 1), 1), ((FAKE, FAKE, FAKE, 300, 1), 2),
                         ((FAKE, FAKE + 4, FAKE, 256, 1), 3), ((FAKE, FAKE, FAKE + 8, 256, 1), 3)]:
        arr = (_Desc * 2)(_Desc(FAKE, FAKE, FAKE, 256, 64), _Desc(*desc))
        assert L.qwg_group_create_q4k_batched(arr, 2, 8, ctypes.byref(out)) == status
        assert out.value is None


def test_group_null_and_count_errors(L):
    out = ctypes.c_void_p()
    arr = (_Desc * 1)(_Desc(FAKE, FAKE, FAKE, 256, 64))
    assert L.qwg_group_create_q4k(None, 1, ctypes.byref(out)) == 1
    assert L.qwg_group_create_q4k(arr, 1, None) == 1
    assert L.qwg_group_create_q4k(arr, 0, ctypes.byref(out)) == 2
    assert L.qwg_group_create_q4k(arr, 65537, ctypes.byref(out)) == 2
    assert L.qwg_group_run(None, None) == 1
    assert L.qwg_group_workgroups(None) == -1
    assert L.qwg_group_destroy(None) == 0


def test_python_binding_rejects_cpu_tensors():
    import torch
    import quantized_weight_decode_gemv_amd as qwg
    w = torch.zeros(144, dtype=torch.uint8)
    x = torch.zeros(256)
    with pytest.raises(ValueError):
        qwg.gemv_q4k(w, x)
    with pytest.raises(ValueError):
        qwg.dequant_q4k(w)


def test_binding_has_no_fallback(monkeypatch, tmp_path):
    from quantized_weight_decode_gemv_amd import _binding
    monkeypatch.setattr(_binding, "_lib", None)
    monkeypatch.setattr(_binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        _binding.lib()


def test_chain_validation_errors(L):
    # Rejected on the host before any HIP call: NULL pointers, phase sizes that
    # do not add up, bad shapes or alignment, and an input that overlaps an
    # output of the same phase.
    out = ctypes.c_void_p()
    one = (ctypes.c_int * 1)(1)
    good = _Desc(FAKE, FAKE + 4096, FAKE + 8192, 256, 64)
    assert L.qwg_chain_create_q4k(None, 1, one, 1, ctypes.byref(out)) == 1
    assert L.qwg_chain_create_q4k((_Desc * 1)(good), 1, None, 1, ctypes.byref(out)) == 1
    assert L.qwg_chain_create_q4k((_Desc * 1)(good), 1, one, 1, None) == 1
    assert L.qwg_chain_create_q4k((_Desc * 1)(good), 0, one, 1, ctypes.byref(out)) == 2
    assert L.qwg_chain_create_q4k((_Desc * 1)(good), 1, (ctypes.c_int * 1)(2), 1, ctypes.byref(out)) == 2
    assert L.qwg_chain_create_q4k((_Desc * 2)(good, good), 2, one, 1, ctypes.byref(out)) == 2
    assert L.qwg_chain_create_q4k((_Desc * 1)(_Desc(FAKE, FAKE + 4096, FAKE + 8192, 300, 64)), 1, one,
                                  1, ctypes.byref(out)) == 2
    assert L.qwg_chain_create_q4k((_Desc * 1)(_Desc(FAKE, FAKE + 4100, FAKE + 8192, 256, 64)), 1, one,
                                  1, ctypes.byref(out)) == 3
    assert L.qwg_chain_create_q4k((_Desc * 1)(_Desc(FAKE, FAKE + 4096, FAKE + 8200, 256, 64)), 1, one,
                                  1, ctypes.byref(out)) == 3
    # x of the second member is the y of the first, both in one phase
    a = _Desc(FAKE, FAKE + 4096, FAKE + 8192, 256, 256)
    b = _Desc(FAKE + 65536, FAKE, FAKE + 8192, 256, 64)
    assert L.qwg_chain_create_q4k((_Desc * 2)(a, b), 2, (ctypes.c_int * 1)(2), 1, ctypes.byref(out)) == 2
    assert L.qwg_chain_run(None, None) == 1
    assert L.qwg_chain_status(None) == 1
    assert L.qwg_chain_phases(None) == -1
    assert L.qwg_chain_tagged(None) == -1
    assert L.qwg_chain_destroy(None) == 0
