"""ctypes wrapper of the CPU oracle (liboracle.so, built from bd_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library.  Arrays are numpy;
bf16 and fp16 values travel as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "bd_oracle.c")

F32, BF16, F16 = 0, 1, 2
MATRIX, GROUP, ROW, COL = 0, 1, 2, 3


def build(verbose: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C11, -O2, no fast-math, OpenMP)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           SRC, "-lm", "-o", LIB]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        vp, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_f64_to_f16.argtypes = [dbl]
        L.orc_f64_to_f16.restype = ctypes.c_uint16
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = dbl
        L.orc_delta.argtypes = [vp, vp, i32, i64, vp]
        L.orc_delta.restype = None
        L.orc_count_nonfinite.argtypes = [vp, i64]
        L.orc_count_nonfinite.restype = i64
        L.orc_clip_stats.argtypes = [vp, i64, dbl, vp]
        L.orc_clip_stats.restype = None
        L.orc_clamp.argtypes = [vp, i64, i32, dbl, dbl, vp]
        L.orc_clamp.restype = None
        L.orc_words_per_row.argtypes = [i64]
        L.orc_words_per_row.restype = i64
        L.orc_pack_signs.argtypes = [vp, i64, i64, vp]
        L.orc_pack_signs.restype = None
        L.orc_scales_count.argtypes = [i32, i64, i64, i64]
        L.orc_scales_count.restype = i64
        L.orc_absmean_scales.argtypes = [vp, i64, i64, i32, i64, i32, vp]
        L.orc_absmean_scales.restype = None
        L.orc_compress.argtypes = [vp, vp, i32, i64, i64, i32, i64, dbl, i32, vp, vp, vp]
        L.orc_compress.restype = i64
        L.orc_select_axis.argtypes = [vp, vp, i32, i64, i64, dbl, vp]
        L.orc_select_axis.restype = i64
        L.orc_quantize_rows.argtypes = [vp, i32, i64, i64, vp, vp]
        L.orc_quantize_rows.restype = None
        L.orc_apply_q8.argtypes = [vp, i32, i64, i64, vp, vp, i64, vp, vp, i32, i64, i32, i32,
                                   vp, vp, vp, vp]
        L.orc_apply_q8.restype = None
        L.orc_reconstruct.argtypes = [vp, vp, i32, i64, i32, i64, i64, vp, i32, vp]
        L.orc_reconstruct.restype = None
        L.orc_apply.argtypes = [vp, i32, i64, i64, vp, i32, i64, vp, vp, i32, i64, i32, i32, vp,
                                vp, vp, vp]
        L.orc_apply.restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _dtype_of(a: np.ndarray, dtype=None) -> int:
    if dtype is not None:
        return dtype
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"unsupported array dtype {a.dtype}")


def num_threads() -> int:
    return int(lib().orc_num_threads())


def f64_to_f16(x: float) -> int:
    return int(lib().orc_f64_to_f16(float(x)))


def f16_to_f64(h: int) -> float:
    return float(lib().orc_f16_to_f64(int(h)))


def delta(wf: np.ndarray, wb, dtype=None) -> np.ndarray:
    wf = np.ascontiguousarray(wf)
    out = np.empty(wf.shape, dtype=np.float32)
    wbc = None if wb is None else np.ascontiguousarray(wb)
    lib().orc_delta(_p(wf), _p(wbc), _dtype_of(wf, dtype), wf.size, _p(out))
    return out


def clip_stats(d: np.ndarray, k: float):
    d = np.ascontiguousarray(d, dtype=np.float32)
    out = np.zeros(4, dtype=np.float64)
    lib().orc_clip_stats(_p(d), d.size, float(k), _p(out))
    return tuple(float(v) for v in out)


def clamp(d: np.ndarray, clip: bool, lo: float, hi: float) -> np.ndarray:
    d = np.ascontiguousarray(d, dtype=np.float32)
    out = np.empty(d.shape, dtype=np.float64)
    lib().orc_clamp(_p(d), d.size, int(bool(clip)), float(lo), float(hi), _p(out))
    return out


def pack_signs(dc: np.ndarray) -> np.ndarray:
    dc = np.ascontiguousarray(dc, dtype=np.float64)
    d_out, d_in = dc.shape
    wpr = int(lib().orc_words_per_row(d_in))
    out = np.zeros((d_out, wpr), dtype=np.uint64)
    lib().orc_pack_signs(_p(dc), d_out, d_in, _p(out))
    return out


def scales_count(mode: int, d_out: int, d_in: int, g: int = 128) -> int:
    return int(lib().orc_scales_count(mode, d_out, d_in, g))


def _scale_np(sdtype):
    return np.uint16 if sdtype == F16 else np.float32


def absmean_scales(dc: np.ndarray, mode: int, g: int = 128, sdtype: int = F32) -> np.ndarray:
    dc = np.ascontiguousarray(dc, dtype=np.float64)
    d_out, d_in = dc.shape
    out = np.zeros(scales_count(mode, d_out, d_in, g), dtype=_scale_np(sdtype))
    lib().orc_absmean_scales(_p(dc), d_out, d_in, mode, g, sdtype, _p(out))
    return out


def compress(wf: np.ndarray, wb, mode: int, g: int = 128, clip_k: float = 0.0,
             sdtype: int = F32, dtype=None):
    """Returns (words uint64[d_out][wpr], scales, stats(mu, sigma, lo, hi), n_nonfinite)."""
    wf = np.ascontiguousarray(wf)
    d_out, d_in = wf.shape
    wbc = None if wb is None else np.ascontiguousarray(wb)
    words = np.zeros((d_out, int(lib().orc_words_per_row(d_in))), dtype=np.uint64)
    scales = np.zeros(scales_count(mode, d_out, d_in, g), dtype=_scale_np(sdtype))
    stats = np.zeros(4, dtype=np.float64)
    bad = lib().orc_compress(_p(wf), _p(wbc), _dtype_of(wf, dtype), d_out, d_in, mode, g,
                             float(clip_k), sdtype, _p(words), _p(scales), _p(stats))
    if bad < 0:
        raise MemoryError("oracle compress: allocation failed")
    return words, scales, tuple(float(v) for v in stats), int(bad)


def quantize_rows(w: np.ndarray, dtype=None):
    """INT8 base weights, symmetric per output row (the reading of the pages' INT8
    base): returns (q int8 [d_out][d_in], s float32 [d_out])."""
    w = np.ascontiguousarray(w)
    d_out, d_in = w.shape
    q = np.zeros((d_out, d_in), dtype=np.int8)
    s = np.zeros(d_out, dtype=np.float32)
    lib().orc_quantize_rows(_p(w), _dtype_of(w, dtype), d_out, d_in, _p(q), _p(s))
    return q, s


def apply_q8(x: np.ndarray, q: np.ndarray, s: np.ndarray, words_bank: np.ndarray,
             scales_bank: np.ndarray, mode: int, user_ids: np.ndarray, g: int = 128,
             sdtype: int = F32, xdtype=None):
    """apply() with the base weight given as INT8 rows and their scales."""
    x = np.ascontiguousarray(x)
    q = np.ascontiguousarray(q, dtype=np.int8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    words_bank = np.ascontiguousarray(words_bank, dtype=np.uint64)
    scales_bank = np.ascontiguousarray(scales_bank)
    ids = np.ascontiguousarray(user_ids, dtype=np.int32)
    T, d_in = x.shape
    n_rows = q.shape[0]
    U = words_bank.shape[0]
    y = np.empty((T, n_rows), dtype=np.float64)
    yb = np.empty_like(y)
    yd = np.empty_like(y)
    lib().orc_apply_q8(_p(x), _dtype_of(x, xdtype), T, d_in, _p(q), _p(s), n_rows, _p(words_bank),
                       _p(scales_bank), mode, g, sdtype, U, _p(ids), _p(y), _p(yb), _p(yd))
    return y, yb, yd


def select_axis(wf: np.ndarray, wb, clip_k: float = 0.0, dtype=None):
    """Per-layer choice between ROW and COL absmean scales ([P5] "Key Contributions" 2,
    read without data: the axis whose reconstruction is closer to the delta).
    Returns (err_row, err_col, axis, n_nonfinite)."""
    wf = np.ascontiguousarray(wf)
    d_out, d_in = wf.shape
    wbc = None if wb is None else np.ascontiguousarray(wb)
    out = np.zeros(3, dtype=np.float64)
    bad = lib().orc_select_axis(_p(wf), _p(wbc), _dtype_of(wf, dtype), d_out, d_in,
                                float(clip_k), _p(out))
    if bad < 0:
        raise MemoryError("oracle select_axis: allocation failed")
    return float(out[0]), float(out[1]), int(out[2]), int(bad)


def reconstruct(words: np.ndarray, scales: np.ndarray, mode: int, d_out: int, d_in: int,
                g: int = 128, sdtype: int = F32, wb=None, wdtype=None) -> np.ndarray:
    words = np.ascontiguousarray(words, dtype=np.uint64)
    scales = np.ascontiguousarray(scales)
    out = np.empty((d_out, d_in), dtype=np.float64)
    wbc = None if wb is None else np.ascontiguousarray(wb)
    wd = 0 if wbc is None else _dtype_of(wbc, wdtype)
    lib().orc_reconstruct(_p(words), _p(scales), mode, g, sdtype, d_out, d_in, _p(wbc), wd, _p(out))
    return out


def apply(x: np.ndarray, wb_rows: np.ndarray, words_bank: np.ndarray, scales_bank: np.ndarray,
          mode: int, user_ids: np.ndarray, g: int = 128, sdtype: int = F32, xdtype=None,
          wdtype=None):
    """Plain-definition apply over the given output rows.

    x [T][d_in]; wb_rows [n_rows][d_in]; words_bank [U][n_rows][wpr];
    scales_bank [U][per-user count for n_rows rows].  Returns (y, y_base,
    y_delta), each float64 [T][n_rows]."""
    x = np.ascontiguousarray(x)
    wb_rows = np.ascontiguousarray(wb_rows)
    words_bank = np.ascontiguousarray(words_bank, dtype=np.uint64)
    scales_bank = np.ascontiguousarray(scales_bank)
    ids = np.ascontiguousarray(user_ids, dtype=np.int32)
    T, d_in = x.shape
    n_rows = wb_rows.shape[0]
    U = words_bank.shape[0]
    y = np.empty((T, n_rows), dtype=np.float64)
    yb = np.empty_like(y)
    yd = np.empty_like(y)
    lib().orc_apply(_p(x), _dtype_of(x, xdtype), T, d_in, _p(wb_rows), _dtype_of(wb_rows, wdtype),
                    n_rows, _p(words_bank), _p(scales_bank), mode, g, sdtype, U, _p(ids), _p(y),
                    _p(yb), _p(yd))
    return y, yb, yd
