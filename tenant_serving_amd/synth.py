"""Seeded synthetic workloads for the BitDelta hot path.

This module holds no BitDelta arithmetic.  It describes the five workload
shapes (matrix sizes, user counts, batch composition, scale modes) and fills
tensors with the counter-based recipes of ``csrc/synth_core.h``:

* host fills (numpy) come from ``libbdsynth_host.so`` (gcc build) and feed the
  CPU oracle;
* device fills (torch tensors on the GPU) come from ``libbdsynth_dev.so``
  (hipcc build of the same header) and feed the GPU library.

Both evaluate the same integer hash and the same fixed sequence of IEEE
binary64 operations, so any row range of any tensor is bit-identical on both
sides; the oracle never receives data produced on the GPU.

Value recipes (readings of the workloads, stated once here):

* ``W_base ~ N(0, 0.02^2)``: centred Irwin-Hall(8) normal, rounded to the
  weight dtype.
* ``W_fine = round(W_base + delta)`` with ``delta ~ Laplace(0, b)`` computed in
  binary64, rounded to fp32 and then (bf16 weights) to bf16.
* Outliers (clipped MLP workload): each position independently, with
  probability 0.1 %, has its delta replaced by ``+-50 * b * sqrt(2)`` (50
  standard deviations of the Laplace law), fair sign.
* ``X ~ N(0, 1)`` rounded to the activation dtype.
* User ids: a permutation (one token per user), uniform draws, or Zipf(1.1)
  truncated to the user count (P(k) proportional to k^-1.1, id = k-1), in draw
  order.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_DIR = os.path.join(_HERE, "lib")

# dtype codes shared with the generator libraries
F32, BF16 = 0, 1
# scale modes (numbering of the public C ABI)
MATRIX, GROUP, ROW, COL = 0, 1, 2, 3
# scale dtypes
S_F32, S_F16 = 0, 2

KIND_WBASE, KIND_PERT, KIND_OUTLIER, KIND_X, KIND_IDS = 0, 1, 2, 3, 4
DEFAULT_SEED = 0


@dataclass(frozen=True)
class Matrix:
    name: str
    d_out: int
    d_in: int
    mode: int
    scale_dtype: int
    xgroup: int  # index of the activation tensor this matrix reads


@dataclass
class Workload:
    cid: int
    name: str
    dtype: int  # F32 or BF16 for weights and activations
    n_users: int
    T: int
    group_size: int
    clip_k: float
    b: float
    outlier_p: float
    ids_kind: str
    matrices: List[Matrix] = field(default_factory=list)
    xgroups: List[int] = field(default_factory=list)  # d_in of each activation tensor
    seed: int = DEFAULT_SEED

    @property
    def outlier_thresh53(self) -> int:
        return int(round(self.outlier_p * float(1 << 53))) if self.outlier_p > 0 else 0

    @property
    def outlier_mag(self) -> float:
        return 50.0 * self.b * math.sqrt(2.0)


def _llama_layer(layer: int, base_x: int):
    m = []
    for name, d_out, d_in, xg in (("q_proj", 4096, 4096, 0), ("k_proj", 1024, 4096, 0),
                                  ("v_proj", 1024, 4096, 0), ("o_proj", 4096, 4096, 1),
                                  ("gate_proj", 14336, 4096, 2), ("up_proj", 14336, 4096, 2),
                                  ("down_proj", 4096, 14336, 3)):
        m.append(Matrix(f"layers.{layer}.{name}", d_out, d_in, MATRIX, S_F32, base_x + xg))
    return m


def workload(cid: int, seed: int = DEFAULT_SEED) -> Workload:
    """The five workloads, numbered 1..5 (1 = tiny fp32 case)."""
    if cid == 1:
        return Workload(1, "tiny_f32_group128", F32, 1, 4, 128, 0.0, 1e-3, 0.0, "zeros",
                        [Matrix("w", 256, 512, GROUP, S_F32, 0)], [512], seed)
    if cid == 2:
        return Workload(2, "llama8b_q_proj_16users_decode", BF16, 16, 16, 128, 0.0, 5e-4, 0.0,
                        "perm", [Matrix("q_proj", 4096, 4096, MATRIX, S_F32, 0)], [4096], seed)
    if cid == 3:
        return Workload(3, "mlp_64users_group128_clip3", BF16, 64, 256, 128, 3.0, 5e-4, 1e-3,
                        "uniform",
                        [Matrix("gate_proj", 14336, 4096, GROUP, S_F32, 0),
                         Matrix("up_proj", 14336, 4096, GROUP, S_F32, 0),
                         Matrix("down_proj", 4096, 14336, GROUP, S_F32, 1)], [4096, 14336], seed)
    if cid == 4:
        return Workload(4, "qwen3_14b_mlp_32users_peraxis_mixed", BF16, 32, 8 * 128 + 120, 128, 0.0,
                        5e-4, 0.0, "zipf_mixed",
                        [Matrix("gate_proj", 17408, 5120, ROW, S_F16, 0),
                         Matrix("up_proj", 17408, 5120, ROW, S_F16, 0),
                         Matrix("down_proj", 5120, 17408, COL, S_F16, 1)], [5120, 17408], seed)
    if cid == 5:
        mats, xg = [], []
        for layer in range(32):
            mats += _llama_layer(layer, 4 * layer)
            xg += [4096, 4096, 4096, 14336]
        return Workload(5, "llama8b_32layer_stack_128users_decode512", BF16, 128, 512, 128, 0.0,
                        5e-4, 0.0, "zipf", mats, xg, seed)
    raise ValueError(f"unknown workload {cid}")


# ---------------------------------------------------------------- host library
_host = None


def _host_lib():
    global _host
    if _host is None:
        path = os.path.join(LIB_DIR, "libbdsynth_host.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        u64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.bds_key.argtypes = [u64] * 5
        lib.bds_key.restype = u64
        lib.bds_draw.argtypes = [u64, u64]
        lib.bds_draw.restype = u64
        lib.bds_uniform.argtypes = [u64, u64]
        lib.bds_uniform.restype = dbl
        lib.bds_laplace.argtypes = [u64, u64]
        lib.bds_laplace.restype = dbl
        lib.bds_normal.argtypes = [u64, u64]
        lib.bds_normal.restype = dbl
        lib.bds_fill_normal.argtypes = [vp, i32, u64, u64, u64, dbl]
        lib.bds_fill_normal.restype = None
        lib.bds_fill_fine.argtypes = [vp, i32, vp, u64, u64, u64, u64, dbl, u64, dbl]
        lib.bds_fill_fine.restype = None
        _host = lib
    return _host


def key(w: Workload, kind: int, user: int = 0, index: int = 0) -> int:
    return int(_host_lib().bds_key(w.seed, w.cid, kind, user, index))


def draw(k: int, i: int) -> int:
    return int(_host_lib().bds_draw(k, i))


def uniform(k: int, i: int) -> float:
    return float(_host_lib().bds_uniform(k, i))


def _np_dtype(dtype: int):
    return np.uint16 if dtype == BF16 else np.float32


def _rows_arg(rows: Optional[Sequence[int]], n_rows: int):
    return list(range(n_rows)) if rows is None else [int(r) for r in rows]


def host_normal(k: int, dtype: int, n_rows: int, d: int, sigma: float,
                rows: Optional[Sequence[int]] = None) -> np.ndarray:
    lib = _host_lib()
    rr = _rows_arg(rows, n_rows)
    out = np.empty((len(rr), d), dtype=_np_dtype(dtype))
    if rows is None:
        lib.bds_fill_normal(out.ctypes.data, dtype, k, 0, n_rows * d, sigma)
    else:
        for j, r in enumerate(rr):
            lib.bds_fill_normal(out[j].ctypes.data, dtype, k, r * d, d, sigma)
    return out


def host_wbase(w: Workload, m: int, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    mat = w.matrices[m]
    return host_normal(key(w, KIND_WBASE, 0, m), w.dtype, mat.d_out, mat.d_in, 0.02, rows)


def host_wfine(w: Workload, m: int, user: int, rows: Optional[Sequence[int]] = None,
               wbase: Optional[np.ndarray] = None) -> np.ndarray:
    mat = w.matrices[m]
    if wbase is None:
        wbase = host_wbase(w, m, rows)
    wbase = np.ascontiguousarray(wbase)
    lib = _host_lib()
    kp, ko = key(w, KIND_PERT, user, m), key(w, KIND_OUTLIER, user, m)
    out = np.empty_like(wbase)
    rr = _rows_arg(rows, mat.d_out)
    if rows is None:
        lib.bds_fill_fine(out.ctypes.data, w.dtype, wbase.ctypes.data, kp, ko, 0,
                          mat.d_out * mat.d_in, w.b, w.outlier_thresh53, w.outlier_mag)
    else:
        for j, r in enumerate(rr):
            lib.bds_fill_fine(out[j].ctypes.data, w.dtype, wbase[j].ctypes.data, kp, ko,
                              r * mat.d_in, mat.d_in, w.b, w.outlier_thresh53, w.outlier_mag)
    return out


def host_x(w: Workload, xg: int, tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    return host_normal(key(w, KIND_X, 0, xg), w.dtype, w.T, w.xgroups[xg], 1.0, tokens)


def zipf_cdf(n_users: int, s: float = 1.1) -> np.ndarray:
    p = np.arange(1, n_users + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(p)
    return c / c[-1]


def user_ids(w: Workload) -> np.ndarray:
    """int32[T] user id of every token (row of X), in batch order."""
    k = key(w, KIND_IDS)
    T, U = w.T, w.n_users
    if w.ids_kind == "zeros":
        return np.zeros(T, dtype=np.int32)
    if w.ids_kind == "perm":
        assert T == U
        d = np.array([draw(k, i) for i in range(T)], dtype=np.uint64)
        return np.argsort(d, kind="stable").astype(np.int32)
    if w.ids_kind == "uniform":
        return np.array([((draw(k, i) >> 32) * U) >> 32 for i in range(T)], dtype=np.int32)
    cdf = zipf_cdf(U)

    def z(i):
        return min(int(np.searchsorted(cdf, uniform(k, i), side="right")), U - 1)

    if w.ids_kind == "zipf":
        return np.array([z(i) for i in range(T)], dtype=np.int32)
    if w.ids_kind == "zipf_mixed":  # 8 prefill chunks of 128 rows, then decode rows
        ids = []
        for c in range(8):
            ids += [z(c)] * 128
        ids += [z(8 + j) for j in range(T - 8 * 128)]
        return np.array(ids, dtype=np.int32)
    raise ValueError(w.ids_kind)


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 (exact)."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def as_f32(a: np.ndarray, dtype: int) -> np.ndarray:
    return bf16_to_f32(a) if dtype == BF16 else a.astype(np.float32)


# -------------------------------------------------------------- device library
_dev = None


def _dev_lib():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (loads the HIP runtime torch was built with)
        path = os.path.join(LIB_DIR, "libbdsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        u64, i32, dbl, vp = ctypes.c_uint64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lib.bds_dev_fill_normal.argtypes = [vp, i32, u64, u64, u64, dbl, vp]
        lib.bds_dev_fill_normal.restype = i32
        lib.bds_dev_fill_fine.argtypes = [vp, i32, vp, u64, u64, u64, u64, dbl, u64, dbl, vp]
        lib.bds_dev_fill_fine.restype = i32
        _dev = lib
    return _dev


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _torch_dtype(dtype: int):
    import torch
    return torch.bfloat16 if dtype == BF16 else torch.float32


def dev_normal(k: int, dtype: int, n_rows: int, d: int, sigma: float, out=None, device="cuda"):
    import torch
    if out is None:
        out = torch.empty((n_rows, d), dtype=_torch_dtype(dtype), device=device)
    rc = _dev_lib().bds_dev_fill_normal(ctypes.c_void_p(out.data_ptr()), dtype, k, 0,
                                        n_rows * d, sigma, _stream())
    if rc != 0:
        raise RuntimeError(f"bds_dev_fill_normal failed ({rc})")
    return out


def dev_wbase(w: Workload, m: int, out=None):
    mat = w.matrices[m]
    return dev_normal(key(w, KIND_WBASE, 0, m), w.dtype, mat.d_out, mat.d_in, 0.02, out)


def dev_wfine(w: Workload, m: int, user: int, wbase, out=None):
    import torch
    mat = w.matrices[m]
    if out is None:
        out = torch.empty_like(wbase)
    rc = _dev_lib().bds_dev_fill_fine(
        ctypes.c_void_p(out.data_ptr()), w.dtype, ctypes.c_void_p(wbase.data_ptr()),
        key(w, KIND_PERT, user, m), key(w, KIND_OUTLIER, user, m), 0, mat.d_out * mat.d_in,
        w.b, w.outlier_thresh53, w.outlier_mag, _stream())
    if rc != 0:
        raise RuntimeError(f"bds_dev_fill_fine failed ({rc})")
    return out


def dev_x(w: Workload, xg: int, out=None):
    return dev_normal(key(w, KIND_X, 0, xg), w.dtype, w.T, w.xgroups[xg], 1.0, out)
