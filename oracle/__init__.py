"""qwg oracle: plain, slow CPU reference (ctypes over qwg_oracle.c).

TEST INFRASTRUCTURE ONLY. Only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP library and
its Python binding never import it, and it imports nothing from them.

What it computes, and where the pages define it:

* Q4_K dequant: "用 Python 重写 picoLM" page, ``dequantize_q4_K`` listing.
* IQ3 ("fmt=5") dequant: iq3_pack.py page, module docstring and ``decode()``.
* IQ3_XXS in llama.cpp's byte order: codebook.py page, the format table of its
  docstring, ``get_d``, ``get_s``, ``eff_np`` and ``dequant``.
* IQ3_S and IQ4_XS: the same page (format table, ``get_s``, ``eff_np``,
  ``dequant``; the IQ3_S branch of ``encode`` for its code bytes).
* IQ3 encoder: iq3_pack.py page, ``encode()`` (float32, numpy's evaluation
  order; see ``orc_encode_iq3``).
* GEMV / GEMM: ``y = W @ x`` over the fp32 dequantized rows, accumulated in fp64
  with k ascending, plus ``s = sum |w * x|`` for the per-row error bound
  (argument order of picoLM's ``matmul(out, x, W, n_in, n_out, type)`` call in
  the same page's ``model_forward`` listing).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qwg_oracle.c")
LIB = os.path.join(HERE, "liborc.so")

QK = 256
Q4K_BYTES = 144
IQ3_BYTES = 98
IQ3S_BYTES = 110
IQ4XS_BYTES = 136

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, no FP contraction, no fast-math, OpenMP)."""
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_encode_iq3.argtypes = [P, P, I64, I64, P]
        L.orc_q4k_unpack_scales.argtypes = [P, P, P]
        L.orc_q4k_pack_scales.argtypes = [P, P, P]
        L.orc_dequant_q4k.argtypes = [P, I64, P]
        L.orc_dequant_iq3.argtypes = [P, P, I64, P]
        L.orc_dequant_iq3_xxs.argtypes = [P, P, I64, P]
        L.orc_gemv_iq3_xxs.argtypes = [P, P, P, I64, I64, P, P]
        L.orc_gemv_iq3_xxs_rows.argtypes = [P, P, P, I64, P, I64, P, P]
        for f in ("iq3s", "iq4xs"):
            getattr(L, f"orc_dequant_{f}").argtypes = [P, P, I64, P]
            getattr(L, f"orc_gemv_{f}").argtypes = [P, P, P, I64, I64, P, P]
            getattr(L, f"orc_gemv_{f}_rows").argtypes = [P, P, P, I64, P, I64, P, P]
        L.orc_gemv_q4k.argtypes = [P, P, I64, I64, P, P]
        L.orc_gemv_iq3.argtypes = [P, P, P, I64, I64, P, P]
        L.orc_gemm_q4k.argtypes = [P, P, I64, I64, ctypes.c_int, P, P]
        L.orc_gemv_q4k_rows.argtypes = [P, P, I64, P, I64, P, P]
        L.orc_gemv_iq3_rows.argtypes = [P, P, P, I64, P, I64, P, P]
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_get_threads.restype = ctypes.c_int
        for name in ("orc_dequant_q4k", "orc_dequant_iq3", "orc_gemv_q4k", "orc_gemv_iq3",
                     "orc_gemm_q4k", "orc_gemv_q4k_rows", "orc_gemv_iq3_rows",
                     "orc_dequant_iq3_xxs", "orc_gemv_iq3_xxs", "orc_gemv_iq3_xxs_rows",
                     "orc_dequant_iq3s", "orc_gemv_iq3s", "orc_gemv_iq3s_rows",
                     "orc_dequant_iq4xs", "orc_gemv_iq4xs", "orc_gemv_iq4xs_rows",
                     "orc_encode_iq3"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint8:
        raise ValueError("packed blocks must be uint8")
    return a


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def set_threads(n: int) -> None:
    lib().orc_set_threads(int(n))


def get_threads() -> int:
    return int(lib().orc_get_threads())


def f16_to_f32(bits: int) -> float:
    return float(lib().orc_f16_to_f32(int(bits) & 0xFFFF))


def unpack_q4k_scales(p) -> tuple[np.ndarray, np.ndarray]:
    p = _u8(p)
    if p.size != 12:
        raise ValueError("need 12 packed bytes")
    sc = np.zeros(8, np.uint8)
    mn = np.zeros(8, np.uint8)
    lib().orc_q4k_unpack_scales(_ptr(p), _ptr(sc), _ptr(mn))
    return sc, mn


def pack_q4k_scales(sc, mn) -> np.ndarray:
    sc = np.ascontiguousarray(sc, dtype=np.uint8)
    mn = np.ascontiguousarray(mn, dtype=np.uint8)
    if sc.size != 8 or mn.size != 8 or sc.max() > 63 or mn.max() > 63:
        raise ValueError("need eight 6-bit scales and eight 6-bit mins")
    p = np.zeros(12, np.uint8)
    lib().orc_q4k_pack_scales(_ptr(sc), _ptr(mn), _ptr(p))
    return p


def dequant_q4k(blocks, n: int) -> np.ndarray:
    blocks = _u8(blocks)
    if blocks.size * QK != n * Q4K_BYTES:
        raise ValueError("byte count does not match n")
    out = np.empty(n, np.float32)
    _check(lib().orc_dequant_q4k(_ptr(blocks), n, _ptr(out)), "dequant_q4k")
    return out


def dequant_iq3(blocks, grid, n: int) -> np.ndarray:
    blocks = _u8(blocks)
    grid = _f32(grid)
    if grid.shape != (256, 4):
        raise ValueError("grid must be [256, 4]")
    if blocks.size * QK != n * IQ3_BYTES:
        raise ValueError("byte count does not match n")
    out = np.empty(n, np.float32)
    _check(lib().orc_dequant_iq3(_ptr(blocks), _ptr(grid), n, _ptr(out)), "dequant_iq3")
    return out


def dequant_iq3_xxs(blocks, grid, n: int) -> np.ndarray:
    """IQ3_XXS blocks in llama.cpp's byte order (codebook.py page)."""
    blocks = _u8(blocks)
    grid = _f32(grid)
    if grid.shape != (256, 4):
        raise ValueError("grid must be [256, 4]")
    if blocks.size * QK != n * IQ3_BYTES:
        raise ValueError("byte count does not match n")
    out = np.empty(n, np.float32)
    _check(lib().orc_dequant_iq3_xxs(_ptr(blocks), _ptr(grid), n, _ptr(out)), "dequant_iq3_xxs")
    return out


# codebook formats with a table argument: (block bytes, table shape)
_TABLED = {"iq3s": (IQ3S_BYTES, (512, 4)), "iq4xs": (IQ4XS_BYTES, (16,))}


def _tabled_dequant(fmt, blocks, table, n):
    nbytes, tshape = _TABLED[fmt]
    blocks = _u8(blocks)
    table = _f32(table)
    if table.shape != tshape:
        raise ValueError(f"table must be {list(tshape)}")
    if blocks.size * QK != n * nbytes:
        raise ValueError("byte count does not match n")
    out = np.empty(n, np.float32)
    _check(getattr(lib(), f"orc_dequant_{fmt}")(_ptr(blocks), _ptr(table), n, _ptr(out)),
           f"dequant_{fmt}")
    return out


def _tabled_gemv(fmt, w, table, x, n_in, n_out):
    nbytes, tshape = _TABLED[fmt]
    w = _u8(w)
    x = _f32(x)
    table = _f32(table)
    if w.size != n_out * (n_in // QK) * nbytes or x.size != n_in or table.shape != tshape:
        raise ValueError("shape mismatch")
    y = np.empty(n_out, np.float64)
    s = np.empty(n_out, np.float64)
    _check(getattr(lib(), f"orc_gemv_{fmt}")(_ptr(w), _ptr(table), _ptr(x), n_in, n_out, _ptr(y),
                                              _ptr(s)), f"gemv_{fmt}")
    return y, s


def _tabled_rows(fmt, w, table, x, n_in, rows):
    nbytes, tshape = _TABLED[fmt]
    w = _u8(w)
    x = _f32(x)
    table = _f32(table)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    row_bytes = (n_in // QK) * nbytes
    if rows.size == 0 or rows.min() < 0 or (rows.max() + 1) * row_bytes > w.size:
        raise ValueError("rows out of range")
    if table.shape != tshape:
        raise ValueError(f"table must be {list(tshape)}")
    y = np.empty(rows.size, np.float64)
    s = np.empty(rows.size, np.float64)
    _check(getattr(lib(), f"orc_gemv_{fmt}_rows")(_ptr(w), _ptr(table), _ptr(x), n_in, _ptr(rows),
                                                   rows.size, _ptr(y), _ptr(s)), f"gemv_{fmt}_rows")
    return y, s


def dequant_iq3s(blocks, grid, n: int) -> np.ndarray:
    """IQ3_S blocks (110 bytes) with a [512, 4] grid (codebook.py page)."""
    return _tabled_dequant("iq3s", blocks, grid, n)


def dequant_iq4xs(blocks, table, n: int) -> np.ndarray:
    """IQ4_XS blocks (136 bytes) with a 16-value table (codebook.py page)."""
    return _tabled_dequant("iq4xs", blocks, table, n)


def gemv_iq3s(w, grid, x, n_in: int, n_out: int):
    return _tabled_gemv("iq3s", w, grid, x, n_in, n_out)


def gemv_iq4xs(w, table, x, n_in: int, n_out: int):
    return _tabled_gemv("iq4xs", w, table, x, n_in, n_out)


def gemv_iq3s_rows(w, grid, x, n_in: int, rows):
    return _tabled_rows("iq3s", w, grid, x, n_in, rows)


def gemv_iq4xs_rows(w, table, x, n_in: int, rows):
    return _tabled_rows("iq4xs", w, table, x, n_in, rows)


def f32_to_f16(v: float) -> int:
    """binary16 bits of the float32 value v, rounded to nearest even."""
    return int(lib().orc_f32_to_f16(float(np.float32(v))))


def encode_iq3(x, grid) -> np.ndarray:
    """fp32 x [n_rows, n_in] (n_in % 256 == 0, finite) -> uint8 [n_rows, n_in/256*98]
    98-byte IQ3 blocks (iq3_pack.py page, encode()), grid [256, 4] in weight units."""
    x = _f32(x)
    if x.ndim != 2 or x.shape[1] % QK:
        raise ValueError("x must be [n_rows, n_in] with n_in % 256 == 0")
    grid = _f32(grid)
    if grid.shape != (256, 4):
        raise ValueError("grid must be [256, 4]")
    out = np.empty((x.shape[0], x.shape[1] // QK * IQ3_BYTES), np.uint8)
    _check(lib().orc_encode_iq3(_ptr(x), _ptr(grid), x.shape[0], x.shape[1], _ptr(out)),
           "encode_iq3")
    return out


def gemv_q4k(w, x, n_in: int, n_out: int) -> tuple[np.ndarray, np.ndarray]:
    """(y, s) in fp64, each [n_out]."""
    w = _u8(w)
    x = _f32(x)
    if w.size != n_out * (n_in // QK) * Q4K_BYTES or x.size != n_in:
        raise ValueError("shape mismatch")
    y = np.empty(n_out, np.float64)
    s = np.empty(n_out, np.float64)
    _check(lib().orc_gemv_q4k(_ptr(w), _ptr(x), n_in, n_out, _ptr(y), _ptr(s)), "gemv_q4k")
    return y, s


def gemv_iq3(w, grid, x, n_in: int, n_out: int) -> tuple[np.ndarray, np.ndarray]:
    w = _u8(w)
    x = _f32(x)
    grid = _f32(grid)
    if w.size != n_out * (n_in // QK) * IQ3_BYTES or x.size != n_in or grid.shape != (256, 4):
        raise ValueError("shape mismatch")
    y = np.empty(n_out, np.float64)
    s = np.empty(n_out, np.float64)
    _check(lib().orc_gemv_iq3(_ptr(w), _ptr(grid), _ptr(x), n_in, n_out, _ptr(y), _ptr(s)),
           "gemv_iq3")
    return y, s


def gemv_iq3_xxs(w, grid, x, n_in: int, n_out: int) -> tuple[np.ndarray, np.ndarray]:
    w = _u8(w)
    x = _f32(x)
    grid = _f32(grid)
    if w.size != n_out * (n_in // QK) * IQ3_BYTES or x.size != n_in or grid.shape != (256, 4):
        raise ValueError("shape mismatch")
    y = np.empty(n_out, np.float64)
    s = np.empty(n_out, np.float64)
    _check(lib().orc_gemv_iq3_xxs(_ptr(w), _ptr(grid), _ptr(x), n_in, n_out, _ptr(y), _ptr(s)),
           "gemv_iq3_xxs")
    return y, s


def gemm_q4k(w, x, n_in: int, n_out: int) -> tuple[np.ndarray, np.ndarray]:
    """x [batch, n_in] -> (Y, S) fp64 [batch, n_out]."""
    w = _u8(w)
    x = _f32(x)
    if x.ndim != 2 or x.shape[1] != n_in:
        raise ValueError("x must be [batch, n_in]")
    batch = x.shape[0]
    if w.size != n_out * (n_in // QK) * Q4K_BYTES:
        raise ValueError("shape mismatch")
    y = np.empty((batch, n_out), np.float64)
    s = np.empty((batch, n_out), np.float64)
    _check(lib().orc_gemm_q4k(_ptr(w), _ptr(x), n_in, n_out, batch, _ptr(y), _ptr(s)),
           "gemm_q4k")
    return y, s


def gemv_q4k_rows(w, x, n_in: int, rows) -> tuple[np.ndarray, np.ndarray]:
    """Only the listed rows of the GEMV (w is the whole matrix)."""
    w = _u8(w)
    x = _f32(x)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    row_bytes = (n_in // QK) * Q4K_BYTES
    if rows.size == 0 or rows.min() < 0 or (rows.max() + 1) * row_bytes > w.size:
        raise ValueError("rows out of range")
    y = np.empty(rows.size, np.float64)
    s = np.empty(rows.size, np.float64)
    _check(lib().orc_gemv_q4k_rows(_ptr(w), _ptr(x), n_in, _ptr(rows), rows.size, _ptr(y),
                                   _ptr(s)), "gemv_q4k_rows")
    return y, s


def gemv_iq3_rows(w, grid, x, n_in: int, rows) -> tuple[np.ndarray, np.ndarray]:
    w = _u8(w)
    x = _f32(x)
    grid = _f32(grid)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    row_bytes = (n_in // QK) * IQ3_BYTES
    if rows.size == 0 or rows.min() < 0 or (rows.max() + 1) * row_bytes > w.size:
        raise ValueError("rows out of range")
    y = np.empty(rows.size, np.float64)
    s = np.empty(rows.size, np.float64)
    _check(lib().orc_gemv_iq3_rows(_ptr(w), _ptr(grid), _ptr(x), n_in, _ptr(rows), rows.size,
                                   _ptr(y), _ptr(s)), "gemv_iq3_rows")
    return y, s


def gemv_iq3_xxs_rows(w, grid, x, n_in: int, rows) -> tuple[np.ndarray, np.ndarray]:
    w = _u8(w)
    x = _f32(x)
    grid = _f32(grid)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    row_bytes = (n_in // QK) * IQ3_BYTES
    if rows.size == 0 or rows.min() < 0 or (rows.max() + 1) * row_bytes > w.size:
        raise ValueError("rows out of range")
    y = np.empty(rows.size, np.float64)
    s = np.empty(rows.size, np.float64)
    _check(lib().orc_gemv_iq3_xxs_rows(_ptr(w), _ptr(grid), _ptr(x), n_in, _ptr(rows),
                                       rows.size, _ptr(y), _ptr(s)), "gemv_iq3_xxs_rows")
    return y, s


# ---------------------------------------------------------------- block builders (tests)

def q4k_block(d_bits: int, dmin_bits: int, sc, mn, q) -> np.ndarray:
    """One 144-byte Q4_K block from its fields, q being the 256 quants in weight
    order. Places q by the nibble layout of the dequantize_q4_K listing: weight i
    lives in quant byte 32*(i//64) + i%32, low nibble when (i//32) is even."""
    q = np.asarray(q, dtype=np.int64).reshape(256)
    if q.min() < 0 or q.max() > 15:
        raise ValueError("quants are 4-bit")
    b = np.zeros(Q4K_BYTES, np.uint8)
    b[0], b[1] = d_bits & 0xFF, (d_bits >> 8) & 0xFF
    b[2], b[3] = dmin_bits & 0xFF, (dmin_bits >> 8) & 0xFF
    b[4:16] = pack_q4k_scales(sc, mn)
    qs = np.zeros(128, np.int64)
    for i in range(256):
        j, c = i // 32, i // 64
        pos = 32 * c + i % 32
        qs[pos] |= q[i] if j % 2 == 0 else (q[i] << 4)
    b[16:] = qs.astype(np.uint8)
    return b


def iq3_block(idx, words, d_bits: int) -> np.ndarray:
    """One 98-byte IQ3 block: 64 grid indices, 8 uint32 words (little-endian), fp16 d."""
    idx = np.asarray(idx, dtype=np.int64).reshape(64)
    words = np.asarray(words, dtype=np.uint64).reshape(8)
    b = np.zeros(IQ3_BYTES, np.uint8)
    b[:64] = idx.astype(np.uint8)
    for ib in range(8):
        w = int(words[ib])
        for k in range(4):
            b[64 + 4 * ib + k] = (w >> (8 * k)) & 0xFF
    b[96], b[97] = d_bits & 0xFF, (d_bits >> 8) & 0xFF
    return b


def iq3_xxs_block(idx, words, d_bits: int) -> np.ndarray:
    """One 98-byte IQ3_XXS block in llama.cpp's order: fp16 d, 64 grid indices,
    8 uint32 words (little-endian)."""
    idx = np.asarray(idx, dtype=np.int64).reshape(64)
    words = np.asarray(words, dtype=np.uint64).reshape(8)
    b = np.zeros(IQ3_BYTES, np.uint8)
    b[0], b[1] = d_bits & 0xFF, (d_bits >> 8) & 0xFF
    b[2:66] = idx.astype(np.uint8)
    for ib in range(8):
        w = int(words[ib])
        for k in range(4):
            b[66 + 4 * ib + k] = (w >> (8 * k)) & 0xFF
    return b


def iq3s_block(idx, neg, s, d_bits: int) -> np.ndarray:
    """One 110-byte IQ3_S block from 64 nine-bit grid indices, 256 sign flags
    (True = negative) and 8 four-bit sub-scales, placed as the codebook.py
    page's encode writes them (packbits little-endian for the ninth bits and
    the signs, sub-scales as nibbles, low nibble first)."""
    idx = np.asarray(idx, dtype=np.int64).reshape(64)
    neg = np.asarray(neg, dtype=bool).reshape(256)
    s = np.asarray(s, dtype=np.int64).reshape(8)
    if idx.min() < 0 or idx.max() > 511 or s.min() < 0 or s.max() > 15:
        raise ValueError("field out of range")
    b = np.zeros(IQ3S_BYTES, np.uint8)
    b[0], b[1] = d_bits & 0xFF, (d_bits >> 8) & 0xFF
    b[2:66] = (idx & 0xFF).astype(np.uint8)
    b[66:74] = np.packbits(((idx >> 8) & 1).astype(np.uint8), bitorder="little")
    b[74:106] = np.packbits(neg.astype(np.uint8), bitorder="little")
    b[106:110] = (s[0::2] | (s[1::2] << 4)).astype(np.uint8)
    return b


def iq4xs_block(q, s, d_bits: int) -> np.ndarray:
    """One 136-byte IQ4_XS block from 256 four-bit codes (weight order) and 8
    six-bit sub-scales: s split as the codebook.py page's set_s writes it (low
    four bits as nibbles at bytes 4-7, top two bits at bits 2ib of the uint16 at
    bytes 2-3), codes in the IQ4_NL nibble order of that page's encode, per
    32-weight sub-block at bytes 8 + 16 ib."""
    q = np.asarray(q, dtype=np.int64).reshape(8, 32)
    s = np.asarray(s, dtype=np.int64).reshape(8)
    if q.min() < 0 or q.max() > 15 or s.min() < 0 or s.max() > 63:
        raise ValueError("field out of range")
    b = np.zeros(IQ4XS_BYTES, np.uint8)
    b[0], b[1] = d_bits & 0xFF, (d_bits >> 8) & 0xFF
    hi = int(sum(((int(s[ib]) >> 4) & 3) << (2 * ib) for ib in range(8)))
    b[2], b[3] = hi & 0xFF, (hi >> 8) & 0xFF
    lo = s & 15
    b[4:8] = (lo[0::2] | (lo[1::2] << 4)).astype(np.uint8)
    b[8:] = (q[:, :16] | (q[:, 16:] << 4)).reshape(128).astype(np.uint8)
    return b
