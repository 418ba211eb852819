"""ctypes binding of libqwg (include/qwg.h). Argument marshalling only: every
step of the computation runs in the library's HIP kernels. Tensors must be on a
HIP device; calls enqueue on torch's current stream."""
from __future__ import annotations

import ctypes
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqwg.so")

QWG_FMT_Q4K = 0
QWG_FMT_IQ3 = 1
QWG_FMT_IQ3_XXS = 2   # IQ3 blocks in llama.cpp's byte order (d, indices, words)
QWG_FMT_IQ3_S = 3
QWG_FMT_IQ4_XS = 4
IQ3S_BYTES = 110
IQ4XS_BYTES = 136
# table argument shape and row-major source alignment of the codebook formats
_CB = {QWG_FMT_IQ3_S: ("iq3s", (512, 4), IQ3S_BYTES, 2), QWG_FMT_IQ4_XS: ("iq4xs", (16,), IQ4XS_BYTES, 4)}
QK = 256
Q4K_BYTES = 144
IQ3_BYTES = 98
MAX_BATCH = 8

_lib = None


class QwgError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({lib().qwg_strerror(status).decode()})")


def lib() -> ctypes.CDLL:
    """Load libqwg.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m quantized_weight_decode_gemv_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.qwg_version.restype = I
        L.qwg_strerror.argtypes = [I]
        L.qwg_strerror.restype = ctypes.c_char_p
        L.qwg_row_bytes.argtypes = [I, I64]
        L.qwg_row_bytes.restype = I64
        L.qwg_plan_splits.argtypes = [I, I64, I64]
        L.qwg_plan_splits.restype = I
        L.qwg_dequant_q4k.argtypes = [P, P, I64, P]
        L.qwg_dequant_iq3.argtypes = [P, P, P, I64, P]
        L.qwg_dequant_iq3_xxs.argtypes = [P, P, P, I64, P]
        L.qwg_gemv_iq3_xxs.argtypes = [P, P, P, P, I64, I64, P]
        L.qwg_pack_iq3_xxs_tiles.argtypes = [P, P, I64, I64, P]
        L.qwg_encode_iq3.argtypes = [P, P, P, I64, I64, P]
        for name in ("iq3s", "iq4xs"):
            getattr(L, f"qwg_dequant_{name}").argtypes = [P, P, P, I64, P]
            getattr(L, f"qwg_pack_{name}_tiles").argtypes = [P, P, I64, I64, P]
            getattr(L, f"qwg_gemv_{name}").argtypes = [P, P, P, P, I64, I64, P]
            getattr(L, f"qwg_gemv_{name}_tiled").argtypes = [P, P, P, P, I64, I64, P]
            getattr(L, f"qwg_group_create_{name}").argtypes = [P, I, P, ctypes.POINTER(P)]
            getattr(L, f"qwg_group_create_{name}_tiled").argtypes = [P, I, P, ctypes.POINTER(P)]
        L.qwg_gemv_q4k.argtypes = [P, P, P, I64, I64, P]
        L.qwg_gemv_iq3.argtypes = [P, P, P, P, I64, I64, P]
        L.qwg_gemm_q4k.argtypes = [P, P, P, I64, I64, I, P]
        L.qwg_gemm_q4k_ex.argtypes = [P, P, P, I64, I64, I, I, I, P]
        L.qwg_gemm_q4k_noalloc.argtypes = [P, P, P, I64, I64, I, P]
        L.qwg_chain_create_q4k.argtypes = [P, I, P, I, ctypes.POINTER(P)]
        L.qwg_chain_run.argtypes = [P, P]
        L.qwg_chain_status.argtypes = [P]
        L.qwg_chain_phases.argtypes = [P]
        L.qwg_chain_tagged.argtypes = [P]
        L.qwg_chain_destroy.argtypes = [P]
        L.qwg_workspace_reserve.argtypes = [P]
        L.qwg_workspace_release.argtypes = [P]
        L.qwg_gemv_iq3_ex.argtypes = [P, P, P, P, I64, I64, I, I, P]
        L.qwg_group_create_q4k.argtypes = [P, I, ctypes.POINTER(P)]
        L.qwg_group_create_q4k_tiled.argtypes = [P, I, ctypes.POINTER(P)]
        L.qwg_group_create_q4k_batched.argtypes = [P, I, I, ctypes.POINTER(P)]
        L.qwg_group_create_q4k_batched_tiled.argtypes = [P, I, I, ctypes.POINTER(P)]
        L.qwg_gemm_q4k_tiled.argtypes = [P, P, P, I64, I64, I, P]
        L.qwg_tiled_bytes.argtypes = [I, I64, I64]
        L.qwg_tiled_bytes.restype = I64
        L.qwg_pack_q4k_tiles.argtypes = [P, P, I64, I64, P]
        L.qwg_gemv_q4k_tiled.argtypes = [P, P, P, I64, I64, P]
        L.qwg_pack_iq3_tiles.argtypes = [P, P, I64, I64, P]
        L.qwg_gemv_iq3_tiled.argtypes = [P, P, P, P, I64, I64, P]
        L.qwg_group_create_iq3_tiled.argtypes = [P, I, P, ctypes.POINTER(P)]
        L.qwg_group_create_iq3.argtypes = [P, I, P, ctypes.POINTER(P)]
        L.qwg_group_run.argtypes = [P, P]
        L.qwg_group_workgroups.argtypes = [P]
        L.qwg_group_destroy.argtypes = [P]
        for f in ("qwg_dequant_q4k", "qwg_dequant_iq3", "qwg_gemv_q4k", "qwg_gemv_iq3",
                  "qwg_gemv_iq3_ex", "qwg_gemm_q4k", "qwg_gemm_q4k_ex", "qwg_group_create_q4k",
                  "qwg_group_create_q4k_tiled", "qwg_pack_q4k_tiles", "qwg_gemv_q4k_tiled",
                  "qwg_pack_iq3_tiles", "qwg_gemv_iq3_tiled", "qwg_group_create_iq3_tiled",
                  "qwg_group_create_iq3", "qwg_group_run", "qwg_group_workgroups",
                  "qwg_group_destroy", "qwg_group_create_q4k_batched",
                  "qwg_group_create_q4k_batched_tiled", "qwg_gemm_q4k_tiled",
                  "qwg_gemm_q4k_noalloc", "qwg_workspace_reserve", "qwg_workspace_release",
                  "qwg_chain_create_q4k", "qwg_chain_run", "qwg_chain_status", "qwg_chain_phases",
                  "qwg_chain_destroy"):
            getattr(L, f).restype = I
        _lib = L
    return _lib


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a tensor on a HIP device")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise QwgError(rc, what)


def row_bytes(fmt: int, n_in: int) -> int:
    v = lib().qwg_row_bytes(fmt, n_in)
    if v < 0:
        raise ValueError(f"invalid n_in {n_in} for format {fmt}")
    return v


def plan_splits(fmt: int, n_in: int, n_out: int) -> int:
    """Workgroups sharing each 64-row tile for this GEMV shape (1 = no split)."""
    v = lib().qwg_plan_splits(fmt, n_in, n_out)
    if v < 0:
        raise ValueError(f"invalid shape n_in={n_in} n_out={n_out}")
    return v


def _weights(w: torch.Tensor, n_in: int, block_bytes: int) -> int:
    _dev(w, "w", torch.uint8)
    if n_in <= 0 or n_in % QK:
        raise ValueError(f"n_in must be a positive multiple of {QK}, got {n_in}")
    rb = (n_in // QK) * block_bytes
    if w.numel() % rb:
        raise ValueError(f"w has {w.numel()} bytes, not a whole number of {rb}-byte rows")
    return w.numel() // rb


def dequant_q4k(w: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Packed Q4_K blocks (uint8, 144 bytes per 256 weights) -> fp32 weights."""
    _dev(w, "w", torch.uint8)
    if w.numel() % Q4K_BYTES:
        raise ValueError("byte count is not a multiple of 144")
    n = w.numel() // Q4K_BYTES * QK
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=w.device)
    _dev(out, "out", torch.float32)
    if out.numel() != n:
        raise ValueError("out has the wrong size")
    _check(lib().qwg_dequant_q4k(w.data_ptr(), out.data_ptr(), n, _stream(w)), "qwg_dequant_q4k")
    return out


def dequant_iq3(w: torch.Tensor, grid: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Packed IQ3 blocks (uint8, 98 bytes per 256 weights) + fp32 grid [256, 4] -> fp32."""
    return _dequant_iq3(w, grid, out, "qwg_dequant_iq3")


def dequant_iq3_xxs(w: torch.Tensor, grid: torch.Tensor,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """IQ3_XXS blocks in llama.cpp's byte order + its grid (fp32 [256, 4]) -> fp32."""
    return _dequant_iq3(w, grid, out, "qwg_dequant_iq3_xxs")


def _dequant_iq3(w, grid, out, fn: str) -> torch.Tensor:
    _dev(w, "w", torch.uint8)
    _dev(grid, "grid", torch.float32)
    if grid.shape != (256, 4):
        raise ValueError("grid must be [256, 4]")
    if w.numel() % IQ3_BYTES:
        raise ValueError("byte count is not a multiple of 98")
    n = w.numel() // IQ3_BYTES * QK
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=w.device)
    _dev(out, "out", torch.float32)
    if out.numel() != n:
        raise ValueError("out has the wrong size")
    _check(getattr(lib(), fn)(w.data_ptr(), grid.data_ptr(), out.data_ptr(), n, _stream(w)), fn)
    return out


def gemv_q4k(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x; w uint8 [n_out, row_bytes] (or flat), x fp32 [n_in]."""
    _dev(x, "x", torch.float32)
    n_in = x.numel()
    n_out = _weights(w, n_in, Q4K_BYTES)
    if out is None:
        out = torch.empty(n_out, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if out.numel() != n_out:
        raise ValueError("out has the wrong size")
    _check(lib().qwg_gemv_q4k(out.data_ptr(), x.data_ptr(), w.data_ptr(), n_in, n_out, _stream(x)),
           "qwg_gemv_q4k")
    return out


def tiled_bytes(n_in: int, n_out: int, fmt: int = QWG_FMT_Q4K) -> int:
    v = lib().qwg_tiled_bytes(fmt, n_in, n_out)
    if v < 0:
        raise ValueError(f"invalid shape n_in={n_in} n_out={n_out}")
    return v


def pack_q4k_tiles(w: torch.Tensor, n_in: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Row-major Q4_K weights (uint8, n_out rows) -> the tile layout (uint8,
    tiled_bytes(n_in, n_out) bytes) that gemv_q4k_tiled and tiled groups take."""
    n_out = _weights(w, n_in, Q4K_BYTES)
    nbytes = tiled_bytes(n_in, n_out)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _dev(out, "out", torch.uint8)
    if out.numel() != nbytes:
        raise ValueError("out has the wrong size")
    _check(lib().qwg_pack_q4k_tiles(out.data_ptr(), w.data_ptr(), n_in, n_out, _stream(w)),
           "qwg_pack_q4k_tiles")
    return out


def gemv_q4k_tiled(w: torch.Tensor, x: torch.Tensor, n_out: int,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x for weights in the tile layout (pack_q4k_tiles)."""
    _dev(w, "w", torch.uint8)
    _dev(x, "x", torch.float32)
    n_in = x.numel()
    if w.numel() != tiled_bytes(n_in, n_out):
        raise ValueError("w is not a tile-layout matrix of this shape")
    if out is None:
        out = torch.empty(n_out, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if out.numel() != n_out:
        raise ValueError("out has the wrong size")
    _check(lib().qwg_gemv_q4k_tiled(out.data_ptr(), x.data_ptr(), w.data_ptr(), n_in, n_out,
                                    _stream(x)), "qwg_gemv_q4k_tiled")
    return out


def pack_iq3_tiles(w: torch.Tensor, n_in: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Row-major IQ3 weights (uint8, n_out rows) -> the IQ3 tile layout that
    gemv_iq3_tiled and tiled IQ3 groups take."""
    return _pack_iq3(w, n_in, out, "qwg_pack_iq3_tiles")


def pack_iq3_xxs_tiles(w: torch.Tensor, n_in: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Row-major IQ3_XXS weights in llama.cpp's byte order -> the same IQ3 tile
    layout (gemv_iq3_tiled and tiled IQ3 groups take it, with llama.cpp's grid)."""
    return _pack_iq3(w, n_in, out, "qwg_pack_iq3_xxs_tiles")


def _pack_iq3(w, n_in, out, fn: str) -> torch.Tensor:
    n_out = _weights(w, n_in, IQ3_BYTES)
    nbytes = tiled_bytes(n_in, n_out, QWG_FMT_IQ3)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _dev(out, "out", torch.uint8)
    if out.numel() != nbytes:
        raise ValueError("out has the wrong size")
    _check(getattr(lib(), fn)(out.data_ptr(), w.data_ptr(), n_in, n_out, _stream(w)), fn)
    return out


def gemv_iq3_tiled(w: torch.Tensor, x: torch.Tensor, grid: torch.Tensor, n_out: int,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x for IQ3 weights in the tile layout (pack_iq3_tiles)."""
    _dev(w, "w", torch.uint8)
    _dev(x, "x", torch.float32)
    _grid(grid)
    n_in = x.numel()
    if w.numel() != tiled_bytes(n_in, n_out, QWG_FMT_IQ3):
        raise ValueError("w is not an IQ3 tile-layout matrix of this shape")
    if out is None:
        out = torch.empty(n_out, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if out.numel() != n_out:
        raise ValueError("out has the wrong size")
    _check(lib().qwg_gemv_iq3_tiled(out.data_ptr(), x.data_ptr(), w.data_ptr(), grid.data_ptr(),
                                    n_in, n_out, _stream(x)), "qwg_gemv_iq3_tiled")
    return out


def _grid(grid: torch.Tensor) -> None:
    _dev(grid, "grid", torch.float32)
    if grid.shape != (256, 4):
        raise ValueError("grid must be [256, 4]")


def gemv_iq3(w: torch.Tensor, x: torch.Tensor, grid: torch.Tensor,
             out: torch.Tensor | None = None, waves: int = 0, splits: int = 0) -> torch.Tensor:
    """y = W x for IQ3 weights; w uint8 [n_out, row_bytes] (or flat), x fp32 [n_in],
    grid fp32 [256, 4]. waves/splits force the work decomposition (0 = automatic)."""
    _dev(x, "x", torch.float32)
    _grid(grid)
    n_in = x.numel()
    n_out = _weights(w, n_in, IQ3_BYTES)
    if out is None:
        out = torch.empty(n_out, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if out.numel() != n_out:
        raise ValueError("out has the wrong size")
    if waves or splits:
        _check(lib().qwg_gemv_iq3_ex(out.data_ptr(), x.data_ptr(), w.data_ptr(), grid.data_ptr(),
                                     n_in, n_out, waves, splits, _stream(x)), "qwg_gemv_iq3_ex")
    else:
        _check(lib().qwg_gemv_iq3(out.data_ptr(), x.data_ptr(), w.data_ptr(), grid.data_ptr(), n_in,
                                  n_out, _stream(x)), "qwg_gemv_iq3")
    return out


def gemv_iq3_xxs(w: torch.Tensor, x: torch.Tensor, grid: torch.Tensor,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x for IQ3_XXS weights in llama.cpp's byte order; w uint8 [n_out,
    row_bytes] (or flat), x fp32 [n_in], grid fp32 [256, 4] (llama.cpp's table)."""
    _dev(x, "x", torch.float32)
    _grid(grid)
    n_in = x.numel()
    n_out = _weights(w, n_in, IQ3_BYTES)
    if out is None:
        out = torch.empty(n_out, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if out.numel() != n_out:
        raise ValueError("out has the wrong size")
    _check(lib().qwg_gemv_iq3_xxs(out.data_ptr(), x.data_ptr(), w.data_ptr(), grid.data_ptr(),
                                  n_in, n_out, _stream(x)), "qwg_gemv_iq3_xxs")
    return out


def encode_iq3(x: torch.Tensor, grid: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 weights x [n_rows, n_in] (n_in % 256 == 0) -> uint8 [n_rows, n_in/256*98]
    IQ3 container blocks (iq3_pack.py page, encode()); grid fp32 [256, 4] in weight units."""
    _dev(x, "x", torch.float32)
    _grid(grid)
    if x.dim() != 2 or x.shape[1] % QK:
        raise ValueError("x must be [n_rows, n_in] with n_in a multiple of 256")
    n_rows, n_in = x.shape
    if out is None:
        out = torch.empty(n_rows, n_in // QK * IQ3_BYTES, dtype=torch.uint8, device=x.device)
    _dev(out, "out", torch.uint8)
    if out.numel() != n_rows * (n_in // QK) * IQ3_BYTES:
        raise ValueError("out has the wrong size")
    _check(lib().qwg_encode_iq3(out.data_ptr(), x.data_ptr(), grid.data_ptr(), n_rows, n_in,
                                _stream(x)), "qwg_encode_iq3")
    return out


def _cb_table(fmt: int, tab: torch.Tensor) -> None:
    _dev(tab, "grid" if fmt == QWG_FMT_IQ3_S else "table", torch.float32)
    if tuple(tab.shape) != _CB[fmt][1]:
        raise ValueError(f"{_CB[fmt][0]} needs a table of shape {list(_CB[fmt][1])}")


def _cb_dequant(fmt, w, tab, out):
    name, _, nbytes, _ = _CB[fmt]
    _dev(w, "w", torch.uint8)
    _cb_table(fmt, tab)
    if w.numel() % nbytes:
        raise ValueError(f"byte count is not a multiple of {nbytes}")
    n = w.numel() // nbytes * QK
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=w.device)
    _dev(out, "out", torch.float32)
    if out.numel() != n:
        raise ValueError("out has the wrong size")
    _check(getattr(lib(), f"qwg_dequant_{name}")(w.data_ptr(), tab.data_ptr(), out.data_ptr(), n,
                                                  _stream(w)), f"qwg_dequant_{name}")
    return out


def _cb_pack(fmt, w, n_in, out):
    name, _, nbytes, _ = _CB[fmt]
    n_out = _weights(w, n_in, nbytes)
    size = tiled_bytes(n_in, n_out, fmt)
    if out is None:
        out = torch.empty(size, dtype=torch.uint8, device=w.device)
    _dev(out, "out", torch.uint8)
    if out.numel() != size:
        raise ValueError("out has the wrong size")
    _check(getattr(lib(), f"qwg_pack_{name}_tiles")(out.data_ptr(), w.data_ptr(), n_in, n_out,
                                                     _stream(w)), f"qwg_pack_{name}_tiles")
    return out


def _cb_gemv(fmt, w, x, tab, out):
    name, _, nbytes, _ = _CB[fmt]
    _dev(x, "x", torch.float32)
    _cb_table(fmt, tab)
    n_in = x.numel()
    n_out = _weights(w, n_in, nbytes)
    if out is None:
        out = torch.empty(n_out, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if out.numel() != n_out:
        raise ValueError("out has the wrong size")
    _check(getattr(lib(), f"qwg_gemv_{name}")(out.data_ptr(), x.data_ptr(), w.data_ptr(),
                                               tab.data_ptr(), n_in, n_out, _stream(x)),
           f"qwg_gemv_{name}")
    return out


def _cb_gemv_tiled(fmt, w, x, tab, n_out, out):
    name = _CB[fmt][0]
    _dev(w, "w", torch.uint8)
    _dev(x, "x", torch.float32)
    _cb_table(fmt, tab)
    n_in = x.numel()
    if w.numel() != tiled_bytes(n_in, n_out, fmt):
        raise ValueError(f"w is not a {name} tile-layout matrix of this shape")
    if out is None:
        out = torch.empty(n_out, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if out.numel() != n_out:
        raise ValueError("out has the wrong size")
    _check(getattr(lib(), f"qwg_gemv_{name}_tiled")(out.data_ptr(), x.data_ptr(), w.data_ptr(),
                                                     tab.data_ptr(), n_in, n_out, _stream(x)),
           f"qwg_gemv_{name}_tiled")
    return out


def dequant_iq3s(w: torch.Tensor, grid: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """IQ3_S blocks (uint8, 110 bytes per 256 weights) + fp32 grid [512, 4] -> fp32."""
    return _cb_dequant(QWG_FMT_IQ3_S, w, grid, out)


def dequant_iq4xs(w: torch.Tensor, table: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """IQ4_XS blocks (uint8, 136 bytes per 256 weights) + fp32 table [16] -> fp32."""
    return _cb_dequant(QWG_FMT_IQ4_XS, w, table, out)


def pack_iq3s_tiles(w: torch.Tensor, n_in: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Row-major IQ3_S weights -> the IQ3_S tile layout that gemv_iq3s_tiled takes."""
    return _cb_pack(QWG_FMT_IQ3_S, w, n_in, out)


def pack_iq4xs_tiles(w: torch.Tensor, n_in: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Row-major IQ4_XS weights -> the IQ4_XS tile layout that gemv_iq4xs_tiled takes."""
    return _cb_pack(QWG_FMT_IQ4_XS, w, n_in, out)


def gemv_iq3s(w: torch.Tensor, x: torch.Tensor, grid: torch.Tensor,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x for row-major IQ3_S weights; w uint8 [n_out, row_bytes] (or flat,
    16-byte aligned), x fp32 [n_in], grid fp32 [512, 4]."""
    return _cb_gemv(QWG_FMT_IQ3_S, w, x, grid, out)


def gemv_iq4xs(w: torch.Tensor, x: torch.Tensor, table: torch.Tensor,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x for row-major IQ4_XS weights; w uint8 [n_out, row_bytes] (or flat,
    16-byte aligned), x fp32 [n_in], table fp32 [16]."""
    return _cb_gemv(QWG_FMT_IQ4_XS, w, x, table, out)


def gemv_iq3s_tiled(w: torch.Tensor, x: torch.Tensor, grid: torch.Tensor, n_out: int,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x for IQ3_S weights in the tile layout (pack_iq3s_tiles)."""
    return _cb_gemv_tiled(QWG_FMT_IQ3_S, w, x, grid, n_out, out)


def gemv_iq4xs_tiled(w: torch.Tensor, x: torch.Tensor, table: torch.Tensor, n_out: int,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x for IQ4_XS weights in the tile layout (pack_iq4xs_tiles)."""
    return _cb_gemv_tiled(QWG_FMT_IQ4_XS, w, x, table, n_out, out)


def gemm_q4k_tiled(w: torch.Tensor, x: torch.Tensor, n_out: int,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X W^T for tile-layout Q4_K weights (pack_q4k_tiles) and X fp32
    [batch, n_in] (1 <= batch <= 8) -> [batch, n_out]."""
    _dev(x, "x", torch.float32)
    _dev(w, "w", torch.uint8)
    if x.dim() != 2 or not 1 <= x.shape[0] <= MAX_BATCH:
        raise ValueError("x must be [batch, n_in] with 1 <= batch <= 8")
    batch, n_in = x.shape
    if w.numel() != tiled_bytes(n_in, n_out):
        raise ValueError("w is not a tile-layout matrix of this shape")
    if out is None:
        out = torch.empty(batch, n_out, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if out.shape != (batch, n_out):
        raise ValueError("out has the wrong shape")
    _check(lib().qwg_gemm_q4k_tiled(out.data_ptr(), x.data_ptr(), w.data_ptr(), n_in, n_out, batch,
                                    _stream(x)), "qwg_gemm_q4k_tiled")
    return out


def gemm_q4k(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None,
             waves: int = 0, splits: int = 0) -> torch.Tensor:
    """Y = X W^T for X fp32 [batch, n_in] (1 <= batch <= 8) -> [batch, n_out].
    waves/splits force the work decomposition (0 = automatic)."""
    _dev(x, "x", torch.float32)
    if x.dim() != 2 or not 1 <= x.shape[0] <= MAX_BATCH:
        raise ValueError("x must be [batch, n_in] with 1 <= batch <= 8")
    batch, n_in = x.shape
    n_out = _weights(w, n_in, Q4K_BYTES)
    if out is None:
        out = torch.empty(batch, n_out, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if out.shape != (batch, n_out):
        raise ValueError("out has the wrong shape")
    if waves or splits:
        _check(lib().qwg_gemm_q4k_ex(out.data_ptr(), x.data_ptr(), w.data_ptr(), n_in, n_out, batch,
                                     waves, splits, _stream(x)), "qwg_gemm_q4k_ex")
    else:
        _check(lib().qwg_gemm_q4k(out.data_ptr(), x.data_ptr(), w.data_ptr(), n_in, n_out, batch,
                                  _stream(x)), "qwg_gemm_q4k")
    return out


def gemm_q4k_noalloc(w: torch.Tensor, x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """gemm_q4k through qwg_gemm_q4k_noalloc (split sums in the library's static
    scratch: the call allocates nothing). x fp32 [batch, n_in]; `out` is
    [batch, n_out] (allocated here if None, before the call)."""
    _dev(x, "x", torch.float32)
    if x.dim() != 2 or not 1 <= x.shape[0] <= MAX_BATCH:
        raise ValueError("x must be [batch, n_in] with 1 <= batch <= 8")
    batch, n_in = x.shape
    n_out = _weights(w, n_in, Q4K_BYTES)
    if out is None:
        out = torch.empty(batch, n_out, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32)
    if out.shape != (batch, n_out):
        raise ValueError("out has the wrong shape")
    _check(lib().qwg_gemm_q4k_noalloc(out.data_ptr(), x.data_ptr(), w.data_ptr(), n_in, n_out,
                                      batch, _stream(x)), "qwg_gemm_q4k_noalloc")
    return out


def workspace_reserve(stream: torch.cuda.Stream) -> None:
    """Create the split-sum workspace of `stream` now (not under capture)."""
    with torch.cuda.device(stream.device):
        _check(lib().qwg_workspace_reserve(ctypes.c_void_p(stream.cuda_stream)),
               "qwg_workspace_reserve")


def workspace_release(stream: torch.cuda.Stream) -> None:
    """Free the split-sum workspace of `stream` (waits for the device)."""
    with torch.cuda.device(stream.device):
        _check(lib().qwg_workspace_release(ctypes.c_void_p(stream.cuda_stream)),
               "qwg_workspace_release")


class GemvDesc(ctypes.Structure):
    """qwg_gemv_desc: one member of a grouped launch."""
    _fields_ = [("y", ctypes.c_void_p), ("x", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("n_in", ctypes.c_int64), ("n_out", ctypes.c_int64)]


class Group:
    """Many independent GEMVs y_i = W_i x_i of one format run by one launch.

    members: sequence of (w, x, y) device tensors (uint8 weights, fp32 x [n_in],
    fp32 y [n_out]); fmt QWG_FMT_Q4K, QWG_FMT_IQ3 (then `grid`, fp32 [256, 4], is
    shared by every member), QWG_FMT_IQ3_S (grid [512, 4]) or QWG_FMT_IQ4_XS
    (`grid` is the 16-value table). The tensors are referenced by the plan (kept
    alive here) and must stay in place; run() recomputes every y_i from the
    current x_i.
    """

    def __init__(self, members, fmt: int = QWG_FMT_Q4K, grid: torch.Tensor | None = None,
                 tiled: bool = False):
        members = list(members)
        if not members:
            raise ValueError("a group needs at least one member")
        if fmt not in (QWG_FMT_Q4K, QWG_FMT_IQ3, QWG_FMT_IQ3_S, QWG_FMT_IQ4_XS):
            raise ValueError(f"unknown format {fmt}")
        if fmt in _CB:
            if grid is None:
                raise ValueError("the group needs its grid or table")
            _cb_table(fmt, grid)
        elif fmt == QWG_FMT_IQ3:
            if grid is None:
                raise ValueError("an IQ3 group needs the grid")
            _grid(grid)
        block_bytes = {QWG_FMT_Q4K: Q4K_BYTES, QWG_FMT_IQ3: IQ3_BYTES}.get(fmt) or _CB[fmt][2]
        descs = (GemvDesc * len(members))()
        for i, (w, x, y) in enumerate(members):
            _dev(x, "x", torch.float32)
            _dev(y, "y", torch.float32)
            n_in = x.numel()
            if tiled:
                _dev(w, "w", torch.uint8)
                n_out = y.numel()
                if w.numel() != tiled_bytes(n_in, n_out, fmt):
                    raise ValueError(f"member {i}: w is not a tile-layout matrix of this shape")
            else:
                n_out = _weights(w, n_in, block_bytes)
            if y.numel() != n_out:
                raise ValueError(f"member {i}: y has {y.numel()} elements, expected {n_out}")
            descs[i] = GemvDesc(y.data_ptr(), x.data_ptr(), w.data_ptr(), n_in, n_out)
        self._members = members
        self._grid = grid
        self._device = members[0][1].device
        handle = ctypes.c_void_p()
        if fmt in _CB:
            fn = f"qwg_group_create_{_CB[fmt][0]}" + ("_tiled" if tiled else "")
            _check(getattr(lib(), fn)(descs, len(members), grid.data_ptr(), ctypes.byref(handle)), fn)
        elif fmt == QWG_FMT_Q4K and tiled:
            _check(lib().qwg_group_create_q4k_tiled(descs, len(members), ctypes.byref(handle)),
                   "qwg_group_create_q4k_tiled")
        elif fmt == QWG_FMT_Q4K:
            _check(lib().qwg_group_create_q4k(descs, len(members), ctypes.byref(handle)),
                   "qwg_group_create_q4k")
        elif tiled:
            _check(lib().qwg_group_create_iq3_tiled(descs, len(members), grid.data_ptr(),
                                                    ctypes.byref(handle)),
                   "qwg_group_create_iq3_tiled")
        else:
            _check(lib().qwg_group_create_iq3(descs, len(members), grid.data_ptr(),
                                              ctypes.byref(handle)), "qwg_group_create_iq3")
        self._handle = handle

    @property
    def workgroups(self) -> int:
        return lib().qwg_group_workgroups(self._handle)

    def run(self, stream=None) -> None:
        if self._handle is None:
            raise RuntimeError("group destroyed")
        s = stream if stream is not None else torch.cuda.current_stream(self._device)
        _check(lib().qwg_group_run(self._handle, ctypes.c_void_p(s.cuda_stream)), "qwg_group_run")

    def close(self) -> None:
        if self._handle is not None:
            torch.cuda.synchronize(self._device)
            _check(lib().qwg_group_destroy(self._handle), "qwg_group_destroy")
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Q4kGroup(Group):
    """Group of Q4_K GEMVs (members as for Group; tiled: weights in the tile
    layout, y giving each member's n_out)."""

    def __init__(self, members, tiled: bool = False):
        super().__init__(members, QWG_FMT_Q4K, tiled=tiled)


class Q4kBatchedGroup(Group):
    """Group of batched Q4_K products Y_i = X_i W_i^T run by one launch on the
    matrix cores: members (w, x, y) with Q4_K weights w (row-major, or the tile
    layout with tiled=True), x fp32 [batch, n_in] and y fp32 [batch, n_out],
    every member with the same batch (2..8). run() recomputes every Y_i from
    the current X_i."""

    def __init__(self, members, tiled: bool = False):
        members = list(members)
        if not members:
            raise ValueError("a group needs at least one member")
        batch = None
        descs = (GemvDesc * len(members))()
        for i, (w, x, y) in enumerate(members):
            _dev(x, "x", torch.float32)
            _dev(y, "y", torch.float32)
            if x.dim() != 2 or y.dim() != 2:
                raise ValueError(f"member {i}: x and y must be [batch, n]")
            if batch is None:
                batch = x.shape[0]
                if not 2 <= batch <= MAX_BATCH:
                    raise ValueError("batch must be 2..8")
            if x.shape[0] != batch or y.shape[0] != batch:
                raise ValueError(f"member {i}: every member needs the same batch ({batch})")
            n_in = x.shape[1]
            if tiled:
                _dev(w, "w", torch.uint8)
                n_out = y.shape[1]
                if w.numel() != tiled_bytes(n_in, n_out):
                    raise ValueError(f"member {i}: w is not a tile-layout matrix of this shape")
            else:
                n_out = _weights(w, n_in, Q4K_BYTES)
            if y.shape[1] != n_out:
                raise ValueError(f"member {i}: y has {y.shape[1]} columns, expected {n_out}")
            descs[i] = GemvDesc(y.data_ptr(), x.data_ptr(), w.data_ptr(), n_in, n_out)
        self._members = members
        self._grid = None
        self._device = members[0][1].device
        self.batch = batch
        handle = ctypes.c_void_p()
        fn = "qwg_group_create_q4k_batched_tiled" if tiled else "qwg_group_create_q4k_batched"
        _check(getattr(lib(), fn)(descs, len(members), batch, ctypes.byref(handle)), fn)
        self._handle = handle


class Iq3Group(Group):
    """Group of IQ3 GEMVs sharing one grid (members as for Group; tiled: weights
    in the IQ3 tile layout, y giving each member's n_out)."""

    def __init__(self, members, grid: torch.Tensor, tiled: bool = False):
        super().__init__(members, QWG_FMT_IQ3, grid, tiled=tiled)


class Iq3sGroup(Group):
    """Group of IQ3_S GEMVs sharing one [512, 4] grid (tiled: weights in the
    IQ3_S tile layout; otherwise row-major, each w 16-byte aligned)."""

    def __init__(self, members, grid: torch.Tensor, tiled: bool = True):
        super().__init__(members, QWG_FMT_IQ3_S, grid, tiled=tiled)


class Iq4xsGroup(Group):
    """Group of IQ4_XS GEMVs sharing one 16-value table (tiled: weights in the
    IQ4_XS tile layout; otherwise row-major, each w 16-byte aligned)."""

    def __init__(self, members, table: torch.Tensor, tiled: bool = True):
        super().__init__(members, QWG_FMT_IQ4_XS, table, tiled=tiled)


class Q4kChain:
    """A decoder's weight stream as one launch whose phases run in order: phase
    p+1's products read their activations only after every member of phase p
    has stored its output (qwg_chain_create_q4k).

    phases: sequence of phases, each a sequence of members (w, x, y): Q4_K
    weights in the tile layout (pack_q4k_tiles), fp32 x [n_in], fp32 y [n_out].
    A member's x may be the y tensor of a member of an earlier phase. The
    tensors are referenced by the plan (kept alive here) and must stay in place.
    """

    def __init__(self, phases):
        phases = [list(ph) for ph in phases]
        if not phases or any(not ph for ph in phases):
            raise ValueError("a chain needs at least one phase, each with at least one member")
        members = [m for ph in phases for m in ph]
        descs = (GemvDesc * len(members))()
        for i, (w, x, y) in enumerate(members):
            _dev(x, "x", torch.float32)
            _dev(y, "y", torch.float32)
            _dev(w, "w", torch.uint8)
            n_in, n_out = x.numel(), y.numel()
            if w.numel() != tiled_bytes(n_in, n_out):
                raise ValueError(f"member {i}: w is not a tile-layout matrix of this shape")
            descs[i] = GemvDesc(y.data_ptr(), x.data_ptr(), w.data_ptr(), n_in, n_out)
        sizes = (ctypes.c_int * len(phases))(*[len(ph) for ph in phases])
        self._members = members
        self._device = members[0][1].device
        handle = ctypes.c_void_p()
        _check(lib().qwg_chain_create_q4k(descs, len(members), sizes, len(phases),
                                          ctypes.byref(handle)), "qwg_chain_create_q4k")
        self._handle = handle

    @property
    def launch_phases(self) -> int:
        return lib().qwg_chain_phases(self._handle)

    @property
    def tagged(self) -> bool:
        """True if the phases wait on tagged done words (see qwg_chain_create_q4k),
        False if on a flag barrier per phase."""
        return lib().qwg_chain_tagged(self._handle) == 1

    def run(self, stream=None) -> None:
        if self._handle is None:
            raise RuntimeError("chain destroyed")
        s = stream if stream is not None else torch.cuda.current_stream(self._device)
        _check(lib().qwg_chain_run(self._handle, ctypes.c_void_p(s.cuda_stream)), "qwg_chain_run")

    def status(self) -> None:
        """Wait for the device; raise QwgError if a wait of an earlier run gave up."""
        _check(lib().qwg_chain_status(self._handle), "qwg_chain_status")

    def close(self) -> None:
        if self._handle is not None:
            torch.cuda.synchronize(self._device)
            _check(lib().qwg_chain_destroy(self._handle), "qwg_chain_destroy")
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
