"""CPU oracle for sliced r-bit qgemm over nested bit-plane weights.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the library.  It wraps the
plain C oracle in ``nbw_oracle.c`` (fp64, one step per definition, see the
header of that file for the definitions and the passages they follow) and adds
nothing to the arithmetic: this module only marshals numpy arrays.

bf16 tensors travel as ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nbw_oracle.c")
_LIB = os.path.join(_HERE, "libnbw_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/libnbw_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fopenmp", "-shared", "-fPIC",
             _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _configure(lib):
    """Declare the C signatures on a loaded oracle library and return it."""
    i64, i32, vp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
    lib.nbwo_plane_bytes.argtypes = [i64, i64]
    lib.nbwo_plane_bytes.restype = i64
    lib.nbwo_pack.argtypes = [vp, i64, i64, vp]
    lib.nbwo_pack.restype = None
    lib.nbwo_unpack.argtypes = [vp, i64, i64, i32, vp]
    lib.nbwo_unpack.restype = None
    lib.nbwo_dequant_value.argtypes = [dp, i32, i32]
    lib.nbwo_dequant_value.restype = dp
    lib.nbwo_dequant.argtypes = [vp, vp, i64, i64, i32, vp]
    lib.nbwo_dequant.restype = None
    lib.nbwo_qgemm.argtypes = [vp, i64, vp, vp, i64, i64, i32, vp]
    lib.nbwo_qgemm.restype = i32
    lib.nbwo_qgemm_rows.argtypes = [vp, i64, vp, vp, i64, i64, i32, vp, i64, vp]
    lib.nbwo_qgemm_rows.restype = i32
    lib.nbwo_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.nbwo_bf16_to_double.restype = dp
    lib.nbwo_dequant_value_asym.argtypes = [dp, dp, i32, i32]
    lib.nbwo_dequant_value_asym.restype = dp
    lib.nbwo_qgemm_asym_rows.argtypes = [vp, i64, vp, vp, vp, i64, i64, i32, vp, i64, vp]
    lib.nbwo_qgemm_asym_rows.restype = i32
    lib.nbwo_choose_codes.argtypes = [vp, i64, i64, vp, vp, vp, i32, vp]
    lib.nbwo_choose_codes.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check_shape(n: int, k: int) -> None:
    if n < 1 or k < 128 or k % 128:
        raise ValueError(f"oracle needs n >= 1 and k a positive multiple of 128 (n={n}, k={k})")


def plane_bytes(n: int, k: int) -> int:
    _check_shape(n, k)
    return int(_load().nbwo_plane_bytes(n, k))


def pack(codes: np.ndarray) -> np.ndarray:
    """uint8 codes [n][k] -> uint8 planes [8 * plane_bytes(n, k)]."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    n, k = codes.shape
    _check_shape(n, k)
    out = np.empty(8 * plane_bytes(n, k), dtype=np.uint8)
    _load().nbwo_pack(_ptr(codes), n, k, _ptr(out))
    return out


def _check_planes(planes: np.ndarray, n: int, k: int, r: int) -> np.ndarray:
    _check_shape(n, k)
    if not 1 <= r <= 8:
        raise ValueError(f"r must be in 1..8, got {r}")
    planes = np.ascontiguousarray(planes, dtype=np.uint8).reshape(-1)
    if planes.size < r * plane_bytes(n, k):
        raise ValueError("plane buffer shorter than r planes")
    return planes


def unpack(planes: np.ndarray, n: int, k: int, r: int) -> np.ndarray:
    """Codes of the r-bit child, read from planes 0..r-1 only -> uint8 [n][k]."""
    planes = _check_planes(planes, n, k, r)
    out = np.empty((n, k), dtype=np.uint8)
    _load().nbwo_unpack(_ptr(planes), n, k, r, _ptr(out))
    return out


def dequant_value(s: float, q: int, r: int) -> float:
    return float(_load().nbwo_dequant_value(float(s), int(q), int(r)))


def _check_scales(scales: np.ndarray, n: int, k: int) -> np.ndarray:
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    if scales.shape != (n, k // 128):
        raise ValueError(f"scales must be [n][k/128] = {(n, k // 128)}, got {scales.shape}")
    return scales


def dequant(planes: np.ndarray, scales_bf16: np.ndarray, n: int, k: int, r: int) -> np.ndarray:
    """fp64 weights [n][k] of the r-bit child."""
    planes = _check_planes(planes, n, k, r)
    scales = _check_scales(scales_bf16, n, k)
    out = np.empty((n, k), dtype=np.float64)
    _load().nbwo_dequant(_ptr(planes), _ptr(scales), n, k, r, _ptr(out))
    return out


def qgemm(x_bf16: np.ndarray, planes: np.ndarray, scales_bf16: np.ndarray, n: int, k: int,
          r: int) -> np.ndarray:
    """fp64 Y [batch][n] = X . dequant_r(W)^T."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    if x.ndim != 2 or x.shape[1] != k or x.shape[0] < 1:
        raise ValueError(f"x must be [batch][{k}], got {x.shape}")
    planes = _check_planes(planes, n, k, r)
    scales = _check_scales(scales_bf16, n, k)
    out = np.empty((x.shape[0], n), dtype=np.float64)
    rc = _load().nbwo_qgemm(_ptr(x), x.shape[0], _ptr(planes), _ptr(scales), n, k, r, _ptr(out))
    if rc != 0:
        raise MemoryError("oracle qgemm: allocation failed")
    return out


def qgemm_rows(x_bf16: np.ndarray, planes: np.ndarray, scales_bf16: np.ndarray, n: int, k: int,
               r: int, rows) -> np.ndarray:
    """fp64 Y[:, rows] ([batch][len(rows)]) for the selected output rows only."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    if x.ndim != 2 or x.shape[1] != k or x.shape[0] < 1:
        raise ValueError(f"x must be [batch][{k}], got {x.shape}")
    planes = _check_planes(planes, n, k, r)
    scales = _check_scales(scales_bf16, n, k)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    if rows.size and (rows.min() < 0 or rows.max() >= n):
        raise ValueError("row index out of range")
    out = np.empty((x.shape[0], rows.size), dtype=np.float64)
    rc = _load().nbwo_qgemm_rows(_ptr(x), x.shape[0], _ptr(planes), _ptr(scales), n, k, r,
                                 _ptr(rows), rows.size, _ptr(out))
    if rc != 0:
        raise MemoryError("oracle qgemm_rows: allocation failed")
    return out


def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def dequant_value_asym(s: float, z: float, q: int, r: int) -> float:
    """Asymmetric child value s * (2^(8-r) * (q + 1/2) - 1/2 - z)."""
    return float(_load().nbwo_dequant_value_asym(float(s), float(z), int(q), int(r)))


def qgemm_asym(x_bf16: np.ndarray, planes: np.ndarray, scales_bf16: np.ndarray,
               zeros_bf16: np.ndarray, n: int, k: int, r: int, rows=None) -> np.ndarray:
    """fp64 Y [batch][len(rows)] of the asymmetric child (all rows by default)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    if x.ndim != 2 or x.shape[1] != k or x.shape[0] < 1:
        raise ValueError(f"x must be [batch][{k}], got {x.shape}")
    planes = _check_planes(planes, n, k, r)
    scales = _check_scales(scales_bf16, n, k)
    zeros = _check_scales(zeros_bf16, n, k)
    rows = np.arange(n, dtype=np.int64) if rows is None else \
        np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    if rows.size and (rows.min() < 0 or rows.max() >= n):
        raise ValueError("row index out of range")
    out = np.empty((x.shape[0], rows.size), dtype=np.float64)
    rc = _load().nbwo_qgemm_asym_rows(_ptr(x), x.shape[0], _ptr(planes), _ptr(scales),
                                      _ptr(zeros), n, k, r, _ptr(rows), rows.size, _ptr(out))
    if rc != 0:
        raise MemoryError("oracle qgemm_asym: allocation failed")
    return out


def choose_codes(w_f32: np.ndarray, scales_bf16: np.ndarray, widths, lambdas) -> np.ndarray:
    """Parent codes uint8 [n][k] minimising the lambda-weighted child errors (brute force)."""
    w = np.ascontiguousarray(w_f32, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be [n][k]")
    n, k = w.shape
    _check_shape(n, k)
    scales = _check_scales(scales_bf16, n, k)
    widths = np.ascontiguousarray(widths, dtype=np.int32).reshape(-1)
    lambdas = np.ascontiguousarray(lambdas, dtype=np.float64).reshape(-1)
    if widths.size != lambdas.size or widths.size < 1 or widths.min() < 1 or widths.max() > 8:
        raise ValueError("widths (1..8) and lambdas must be non-empty and of equal length")
    out = np.empty((n, k), dtype=np.uint8)
    _load().nbwo_choose_codes(_ptr(w), n, k, _ptr(scales), _ptr(widths), _ptr(lambdas),
                              int(widths.size), _ptr(out))
    return out
