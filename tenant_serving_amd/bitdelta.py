"""Python binding of libbitdelta.so (include/bitdelta.h).

Argument marshalling only: every step of compression and apply runs in the
HIP kernels of the native library.  PyTorch provides the device memory (tensor
storage) and the stream (the current HIP stream of the tensor's device).  The
``bd_*`` functions mirror the C entry points one to one; ``compress``,
``apply`` and ``reconstruct`` additionally allocate outputs and workspace with
torch.  If the native library is missing or cannot be loaded, every call
raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libbitdelta.so")

# enums of the C ABI
BD_OK, BD_ERR_INVALID_ARG, BD_ERR_SHAPE, BD_ERR_DTYPE, BD_ERR_UNSUPPORTED = 0, 1, 2, 3, 4
BD_ERR_WORKSPACE, BD_ERR_DEVICE, BD_ERR_NONFINITE, BD_ERR_USER_ID, BD_ERR_BATCH = 5, 6, 7, 8, 9
BD_F32, BD_BF16, BD_F16 = 0, 1, 2
BD_SCALE_MATRIX, BD_SCALE_GROUP, BD_SCALE_ROW, BD_SCALE_COL = 0, 1, 2, 3
MODE_NAMES = {"matrix": BD_SCALE_MATRIX, "group": BD_SCALE_GROUP, "row": BD_SCALE_ROW,
              "col": BD_SCALE_COL}


class bd_compress_params(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("mode", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("clip_k", ctypes.c_float),
                ("scale_dtype", ctypes.c_int32)]


class BitDeltaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libbitdelta.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER(bd_compress_params)
        L.bd_abi_version.restype = ctypes.c_int
        L.bd_abi_version.argtypes = []
        L.bd_status_string.restype = ctypes.c_char_p
        L.bd_status_string.argtypes = [ctypes.c_int]
        L.bd_signs_bytes.restype = sz
        L.bd_signs_bytes.argtypes = [i64, i64]
        L.bd_scales_count.restype = i64
        L.bd_scales_count.argtypes = [P, i64, i64]
        L.bd_compress_workspace_bytes.restype = sz
        L.bd_compress_workspace_bytes.argtypes = [P, i64, i64]
        L.bd_apply_workspace_bytes.restype = sz
        L.bd_apply_workspace_bytes.argtypes = [P, i64, i32, i64, i64, ctypes.c_int, ctypes.c_int]
        L.bd_compress.restype = ctypes.c_int
        L.bd_compress.argtypes = [vp, vp, ctypes.c_int, i64, i64, P, vp, vp, vp, sz, vp]
        L.bd_quantize_base.restype = ctypes.c_int
        L.bd_quantize_base.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, vp]
        L.bd_apply_q8_workspace_bytes.restype = sz
        L.bd_apply_q8_workspace_bytes.argtypes = [P, i64, i32, i64, i64, ctypes.c_int,
                                                  ctypes.c_int]
        L.bd_apply_q8.restype = ctypes.c_int
        L.bd_apply_q8.argtypes = [vp, ctypes.c_int, i64, i64, vp, vp, i64, vp, vp, P, i32, vp, vp,
                                  ctypes.c_int, vp, sz, vp]
        L.bd_select_axis_workspace_bytes.restype = sz
        L.bd_select_axis_workspace_bytes.argtypes = [i64, i64, ctypes.c_float]
        L.bd_select_axis.restype = ctypes.c_int
        L.bd_select_axis.argtypes = [vp, vp, ctypes.c_int, i64, i64, ctypes.c_float, vp, vp, vp,
                                     sz, vp]
        L.bd_reconstruct.restype = ctypes.c_int
        L.bd_reconstruct.argtypes = [vp, vp, P, i64, i64, vp, ctypes.c_int, vp, ctypes.c_int, vp]
        L.bd_apply.restype = ctypes.c_int
        L.bd_apply.argtypes = [vp, ctypes.c_int, i64, i64, vp, i64, vp, vp, P, i32, vp, vp,
                               ctypes.c_int, vp, sz, vp]
        L.bd_apply_noalloc.restype = ctypes.c_int
        L.bd_apply_noalloc.argtypes = [vp, ctypes.c_int, i64, i64, vp, i64, vp, vp, P, i32, vp, vp,
                                       ctypes.c_int, vp, vp]
        L.bd_apply_paged_workspace_bytes.restype = sz
        L.bd_apply_paged_workspace_bytes.argtypes = [P, i64, i32, i64, i64, ctypes.c_int,
                                                     ctypes.c_int]
        L.bd_apply_paged.restype = ctypes.c_int
        L.bd_apply_paged.argtypes = [vp, ctypes.c_int, i64, i64, vp, i64, vp, vp, ctypes.c_uint64,
                                     ctypes.c_uint64, i32, P, vp, i32, vp, vp, ctypes.c_int, vp, sz,
                                     vp]
        L.bd_device_status.restype = ctypes.c_int
        L.bd_device_status.argtypes = [vp, vp]
        L.bd_batch_workspace_bytes.restype = sz
        L.bd_batch_workspace_bytes.argtypes = [i64, i32, i64, ctypes.c_int]
        L.bd_batch_prepare.restype = ctypes.c_int
        L.bd_batch_prepare.argtypes = [vp, ctypes.c_int, i64, i64, vp, i32, vp, sz, vp]
        L.bd_base_gemm.restype = ctypes.c_int
        L.bd_base_gemm.argtypes = [vp, ctypes.c_int, i64, i64, vp, i64, vp, vp]
        L.bd_delta_apply.restype = ctypes.c_int
        L.bd_delta_apply.argtypes = [vp, sz, vp, ctypes.c_int, i64, i64, i32, i64, vp, vp, P, vp,
                                     vp]
        L.bd_batch_encode.restype = ctypes.c_int
        L.bd_batch_encode.argtypes = [vp, sz, vp, ctypes.c_int, i64, i64, i32, vp, P, vp]
        L.bd_delta_apply_encoded.restype = ctypes.c_int
        L.bd_delta_apply_encoded.argtypes = [vp, sz, ctypes.c_int, i64, i64, i32, i64, vp, vp, P,
                                             vp, vp]
        L.bd_base_gemm_n_workspace_bytes.restype = sz
        L.bd_base_gemm_n_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i32, vp]
        L.bd_base_gemm_n.restype = ctypes.c_int
        L.bd_base_gemm_n.argtypes = [vp, ctypes.c_int, i64, i64, i32, vp, vp, vp, vp, sz, vp]
        L.bd_base_gemm_q8_n.restype = ctypes.c_int
        L.bd_base_gemm_q8_n.argtypes = [vp, ctypes.c_int, i64, i64, i32, vp, vp, vp, vp, vp, sz,
                                        vp]
        L.bd_delta_apply_encoded_n.restype = ctypes.c_int
        L.bd_delta_apply_encoded_n.argtypes = [vp, sz, ctypes.c_int, i64, i64, i32, i32, vp, vp,
                                               vp, P, vp, vp]
        L.bd_decode_prepare.restype = ctypes.c_int
        L.bd_decode_prepare.argtypes = [vp, ctypes.c_int, i64, i64, vp, i32, vp, P, vp, sz, vp]
        L.bd_decode_apply.restype = ctypes.c_int
        L.bd_decode_apply.argtypes = [vp, ctypes.c_int, i64, i64, vp, i64, vp, vp, P, i32, vp,
                                      ctypes.c_int, vp, sz, vp]
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().bd_status_string(int(s)).decode()


def params(mode="matrix", group_size: int = 128, clip_k: float = 0.0,
           scale_dtype: int = BD_F32, bits: int = 1) -> bd_compress_params:
    m = MODE_NAMES[mode] if isinstance(mode, str) else int(mode)
    return bd_compress_params(bits, m, group_size, clip_k, scale_dtype)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: Optional[torch.Tensor] = None, stream=None):
    if stream is not None:
        return ctypes.c_void_p(int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream))
    dev = t.device if t is not None else torch.device("cuda")
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BD_BF16
    if t.dtype == torch.float32:
        return BD_F32
    if t.dtype == torch.float16:
        return BD_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _torch_dtype(code: int):
    return {BD_F32: torch.float32, BD_BF16: torch.bfloat16, BD_F16: torch.float16}[code]


def _check(st: int, where: str):
    if st != BD_OK:
        raise BitDeltaError(st, where)


# Argument checks done before any pointer reaches the library: the C ABI takes raw
# device pointers, so a host tensor, a strided view, int64 user ids or a scales bank
# too small for the scale mode would otherwise be read as something else on the GPU.

def _dev(t, name: str, dtypes=None, shape=None, device=None, optional: bool = False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ids(user_ids, T, device):
    _dev(user_ids, "user_ids", (torch.int32,), (T,), device)


def _bank(signs_bank, scales_bank, p, n_users, d_out, d_in, device):
    _dev(signs_bank, "signs_bank", (torch.int64,), (n_users, d_out, d_in // 64), device)
    _scales(scales_bank, p, n_users, d_out, d_in, device)


def _scales(scales_bank, p, n_users, d_out, d_in, device, optional=False):
    if scales_bank is not None and isinstance(scales_bank, torch.Tensor):
        need = n_users * max(bd_scales_count(p, d_out, d_in), 0)
        if scales_bank.numel() < need:
            raise ValueError(f"scales_bank holds {scales_bank.numel()} values, the scale mode "
                             f"needs {need} ({n_users} users)")
    _dev(scales_bank, "scales_bank", (scales_dtype(p),), None, device, optional)


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


# ------------------------------------------------------------------ queries

def bd_signs_bytes(d_out: int, d_in: int) -> int:
    return int(lib().bd_signs_bytes(d_out, d_in))


def bd_scales_count(p: bd_compress_params, d_out: int, d_in: int) -> int:
    return int(lib().bd_scales_count(ctypes.byref(p), d_out, d_in))


def bd_compress_workspace_bytes(p: bd_compress_params, d_out: int, d_in: int) -> int:
    return int(lib().bd_compress_workspace_bytes(ctypes.byref(p), d_out, d_in))


def bd_select_axis_workspace_bytes(d_out: int, d_in: int, clip_k: float = 0.0) -> int:
    return int(lib().bd_select_axis_workspace_bytes(d_out, d_in, float(clip_k)))


def bd_apply_workspace_bytes(p: bd_compress_params, T: int, n_users: int, d_out: int, d_in: int,
                             x_dtype: int, y_dtype: int) -> int:
    return int(lib().bd_apply_workspace_bytes(ctypes.byref(p), T, n_users, d_out, d_in, x_dtype,
                                              y_dtype))


# -------------------------------------------------------------- entry points

def bd_compress(w_fine, w_base, p, signs_out, scales_out, workspace, stream=None) -> int:
    _dev(w_fine, "w_fine", (torch.float32, torch.bfloat16))
    d_out, d_in = w_fine.shape
    dev = w_fine.device
    _dev(w_base, "w_base", (w_fine.dtype,), (d_out, d_in), dev, optional=True)
    _dev(signs_out, "signs_out", (torch.int64,), (d_out, d_in // 64), dev)
    _scales(scales_out, p, 1, d_out, d_in, dev)
    _dev(workspace, "workspace", None, None, dev)
    return int(lib().bd_compress(_ptr(w_fine), _ptr(w_base), _dtype_code(w_fine), d_out, d_in,
                                 ctypes.byref(p), _ptr(signs_out), _ptr(scales_out),
                                 _ptr(workspace), _nbytes(workspace), _stream(w_fine, stream)))


def bd_reconstruct(signs, scales, p, d_out, d_in, w_base, out, stream=None) -> int:
    _dev(signs, "signs", (torch.int64,), (d_out, d_in // 64))
    dev = signs.device
    _scales(scales, p, 1, d_out, d_in, dev)
    _dev(w_base, "w_base", (torch.float32, torch.bfloat16), (d_out, d_in), dev, optional=True)
    _dev(out, "out", (torch.float32, torch.bfloat16), (d_out, d_in), dev)
    return int(lib().bd_reconstruct(_ptr(signs), _ptr(scales), ctypes.byref(p), d_out, d_in,
                                    _ptr(w_base), _dtype_code(w_base) if w_base is not None else 0,
                                    _ptr(out), _dtype_code(out), _stream(out, stream)))


def _apply_args(x, w_base_rows, signs_bank, scales_bank, p, n_users, user_ids, y, workspace,
                wdtypes=None):
    _dev(x, "x", (torch.float32, torch.bfloat16))
    T, d_in = x.shape
    dev = x.device
    d_out = w_base_rows.shape[0]
    _dev(w_base_rows, "w_base", wdtypes or (x.dtype,), (d_out, d_in), dev)
    _bank(signs_bank, scales_bank, p, n_users, d_out, d_in, dev)
    _ids(user_ids, T, dev)
    _dev(y, "y", (torch.float32, torch.bfloat16), (T, d_out), dev)
    _dev(workspace, "workspace", None, None, dev)
    return T, d_in, d_out


def bd_apply(x, w_base, signs_bank, scales_bank, p, n_users, user_ids, y, workspace,
             stream=None) -> int:
    T, d_in, d_out = _apply_args(x, w_base, signs_bank, scales_bank, p, n_users, user_ids, y,
                                 workspace)
    return int(lib().bd_apply(_ptr(x), _dtype_code(x), T, d_in, _ptr(w_base), d_out,
                              _ptr(signs_bank), _ptr(scales_bank), ctypes.byref(p), int(n_users),
                              _ptr(user_ids), _ptr(y), _dtype_code(y), _ptr(workspace),
                              _nbytes(workspace), _stream(x, stream)))


def bd_apply_noalloc(x, w_base, signs_bank, scales_bank, p, n_users, user_ids, y, status=None,
                     stream=None) -> int:
    """bd_apply without a workspace (the library's scratch; see include/bitdelta.h);
    status: optional int32[1] device tensor that receives the call's status word."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    T, d_in = x.shape
    dev = x.device
    d_out = w_base.shape[0]
    _dev(w_base, "w_base", (x.dtype,), (d_out, d_in), dev)
    _bank(signs_bank, scales_bank, p, n_users, d_out, d_in, dev)
    _ids(user_ids, T, dev)
    _dev(y, "y", (torch.float32, torch.bfloat16), (T, d_out), dev)
    _dev(status, "status", (torch.int32,), (1,), dev, optional=True)
    return int(lib().bd_apply_noalloc(_ptr(x), _dtype_code(x), T, d_in, _ptr(w_base), d_out,
                                      _ptr(signs_bank), _ptr(scales_bank), ctypes.byref(p),
                                      int(n_users), _ptr(user_ids), _ptr(y), _dtype_code(y),
                                      _ptr(status), _stream(x, stream)))


def bd_apply_paged_workspace_bytes(p, T: int, n_slots: int, d_out: int, d_in: int,
                                   x_dtype: int, y_dtype: int) -> int:
    return int(lib().bd_apply_paged_workspace_bytes(ctypes.byref(p), T, n_slots, d_out, d_in,
                                                    x_dtype, y_dtype))


def bd_apply_paged(x, w_base, signs_pool, scales_pool, signs_stride: int, scales_stride: int,
                   n_slots: int, p, slot_of_user, user_ids, y, workspace, stream=None) -> int:
    """bd_apply over banks in a pool of slots (include/bitdelta.h).  signs_pool and
    scales_pool: uint8 views that start at slot 0's signs / scales of this matrix and
    reach the last slot's; strides in bytes (0: dense [n_slots][...] banks of the bank
    dtypes instead); slot_of_user: int32[n_users] device table."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    T, d_in = x.shape
    dev = x.device
    d_out = w_base.shape[0]
    _dev(w_base, "w_base", (x.dtype,), (d_out, d_in), dev)
    n_sc = bd_scales_count(p, d_out, d_in)
    esz = 2 if p.scale_dtype == BD_F16 else 4
    for t, name, stride, need in ((signs_pool, "signs_pool", signs_stride, d_out * d_in // 8),
                                  (scales_pool, "scales_pool", scales_stride, n_sc * esz)):
        _dev(t, name, None, None, dev)
        span = (n_slots - 1) * (stride or need) + need if n_slots > 0 else 0
        if _nbytes(t) < span:
            raise ValueError(f"{name} holds {_nbytes(t)} bytes, {n_slots} slots need {span}")
    _dev(slot_of_user, "slot_of_user", (torch.int32,), None, dev)
    if slot_of_user.dim() != 1:
        raise ValueError("slot_of_user must be one-dimensional")
    _ids(user_ids, T, dev)
    _dev(y, "y", (torch.float32, torch.bfloat16), (T, d_out), dev)
    _dev(workspace, "workspace", None, None, dev)
    return int(lib().bd_apply_paged(_ptr(x), _dtype_code(x), T, d_in, _ptr(w_base), d_out,
                                    _ptr(signs_pool), _ptr(scales_pool), int(signs_stride),
                                    int(scales_stride), int(n_slots), ctypes.byref(p),
                                    _ptr(slot_of_user), slot_of_user.numel(), _ptr(user_ids),
                                    _ptr(y), _dtype_code(y), _ptr(workspace), _nbytes(workspace),
                                    _stream(x, stream)))


def bd_device_status(workspace, stream=None) -> int:
    _dev(workspace, "workspace")
    return int(lib().bd_device_status(_ptr(workspace), _stream(workspace, stream)))


def bd_batch_workspace_bytes(T: int, n_users: int, d_in: int, x_dtype: int) -> int:
    return int(lib().bd_batch_workspace_bytes(T, n_users, d_in, x_dtype))


def bd_batch_prepare(x, user_ids, n_users, batch, stream=None) -> int:
    _dev(x, "x", (torch.float32, torch.bfloat16))
    T, d_in = x.shape
    _ids(user_ids, T, x.device)
    _dev(batch, "batch", None, None, x.device)
    return int(lib().bd_batch_prepare(_ptr(x), _dtype_code(x), T, d_in, _ptr(user_ids),
                                      int(n_users), _ptr(batch), _nbytes(batch),
                                      _stream(x, stream)))


def bd_base_gemm(x, w_base, y, stream=None) -> int:
    _dev(x, "x", (torch.float32, torch.bfloat16))
    T, d_in = x.shape
    _dev(w_base, "w_base", (x.dtype,), (w_base.shape[0], d_in), x.device)
    _dev(y, "y", (torch.float32,), (T, w_base.shape[0]), x.device)
    return int(lib().bd_base_gemm(_ptr(x), _dtype_code(x), T, d_in, _ptr(w_base),
                                  w_base.shape[0], _ptr(y), _stream(x, stream)))


def bd_delta_apply(batch, x, n_users, signs_bank, scales_bank, p, y, stream=None) -> int:
    _dev(x, "x", (torch.float32, torch.bfloat16))
    T, d_in = x.shape
    dev = x.device
    _dev(y, "y", (torch.float32,), None, dev)
    if y.dim() != 2 or y.shape[0] != T:
        raise ValueError(f"y has shape {tuple(y.shape)}, expected ({T}, d_out)")
    d_out = y.shape[1]
    _bank(signs_bank, scales_bank, p, n_users, d_out, d_in, dev)
    _dev(batch, "batch", None, None, dev)
    return int(lib().bd_delta_apply(_ptr(batch), _nbytes(batch), _ptr(x), _dtype_code(x), T, d_in,
                                    int(n_users), d_out, _ptr(signs_bank), _ptr(scales_bank),
                                    ctypes.byref(p), _ptr(y), _stream(y, stream)))


def bd_batch_encode(batch, x, n_users, scales_bank, p, stream=None) -> int:
    _dev(x, "x", (torch.bfloat16,))
    T, d_in = x.shape
    dev = x.device
    _dev(batch, "batch", None, None, dev)
    if p.mode == BD_SCALE_COL:
        _scales(scales_bank, p, n_users, 1, d_in, dev)
    else:
        _dev(scales_bank, "scales_bank", None, None, dev, optional=True)
    return int(lib().bd_batch_encode(_ptr(batch), _nbytes(batch), _ptr(x), _dtype_code(x), T,
                                     d_in, int(n_users), _ptr(scales_bank), ctypes.byref(p),
                                     _stream(x, stream)))


def bd_delta_apply_encoded(batch, T, d_in, n_users, signs_bank, scales_bank, p, y,
                           stream=None) -> int:
    _dev(y, "y", (torch.float32,))
    dev = y.device
    if y.dim() != 2 or y.shape[0] != T:
        raise ValueError(f"y has shape {tuple(y.shape)}, expected ({T}, d_out)")
    d_out = y.shape[1]
    _bank(signs_bank, scales_bank, p, n_users, d_out, d_in, dev)
    _dev(batch, "batch", None, None, dev)
    return int(lib().bd_delta_apply_encoded(_ptr(batch), _nbytes(batch), BD_BF16, int(T),
                                            int(d_in), int(n_users), d_out, _ptr(signs_bank),
                                            _ptr(scales_bank), ctypes.byref(p), _ptr(y),
                                            _stream(y, stream)))


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def bd_base_gemm_n_workspace_bytes(x_dtype: int, T: int, d_in: int, d_outs) -> int:
    arr = (ctypes.c_int64 * len(d_outs))(*[int(d) for d in d_outs])
    return int(lib().bd_base_gemm_n_workspace_bytes(x_dtype, T, d_in, len(d_outs), arr))


def bd_base_gemm_n(x, w_bases, ys, workspace=None, stream=None) -> int:
    """Base products of up to 4 matrices that read x, in one launch (K split in ordered
    parts through `workspace` where that fills the chip better; None: no split)."""
    _dev(x, "x", (torch.float32, torch.bfloat16))
    T, d_in = x.shape
    if not 1 <= len(w_bases) <= 4 or len(ys) != len(w_bases):
        raise ValueError("1..4 matrices, one output each")
    for w, y in zip(w_bases, ys):
        _dev(w, "w_base", (x.dtype,), (w.shape[0], d_in), x.device)
        _dev(y, "y", (torch.float32,), (T, w.shape[0]), x.device)
    _dev(workspace, "workspace", None, None, x.device, optional=True)
    d_outs = (ctypes.c_int64 * len(ys))(*[w.shape[0] for w in w_bases])
    return int(lib().bd_base_gemm_n(_ptr(x), _dtype_code(x), T, d_in, len(ys),
                                    _ptr_array(w_bases), d_outs, _ptr_array(ys), _ptr(workspace),
                                    0 if workspace is None else _nbytes(workspace),
                                    _stream(x, stream)))


def bd_base_gemm_q8_n(x, wqs, wscales, ys, workspace=None, stream=None) -> int:
    """bd_base_gemm_n on INT8 base rows (quantize_base): up to 4 matrices that read x, in
    one launch; `workspace` as for bd_base_gemm_n (sized by its query, None: no split)."""
    _dev(x, "x", (torch.bfloat16,))
    T, d_in = x.shape
    if not 1 <= len(wqs) <= 4 or len(ys) != len(wqs) or len(wscales) != len(wqs):
        raise ValueError("1..4 matrices, one scale vector and one output each")
    for w, sc, y in zip(wqs, wscales, ys):
        _dev(w, "wq", (torch.int8,), (w.shape[0], d_in), x.device)
        _dev(sc, "wscales", (torch.float32,), (w.shape[0],), x.device)
        _dev(y, "y", (torch.float32,), (T, w.shape[0]), x.device)
    _dev(workspace, "workspace", None, None, x.device, optional=True)
    d_outs = (ctypes.c_int64 * len(ys))(*[w.shape[0] for w in wqs])
    return int(lib().bd_base_gemm_q8_n(_ptr(x), _dtype_code(x), T, d_in, len(ys), _ptr_array(wqs),
                                       _ptr_array(wscales), d_outs, _ptr_array(ys), _ptr(workspace),
                                       0 if workspace is None else _nbytes(workspace),
                                       _stream(x, stream)))


def bd_delta_apply_encoded_n(batch, T, d_in, n_users, signs_banks, scales_banks, p, ys,
                             stream=None) -> int:
    """Delta products of up to 4 matrices on one encoded batch, in one launch."""
    if not 1 <= len(ys) <= 4 or len(signs_banks) != len(ys) or len(scales_banks) != len(ys):
        raise ValueError("1..4 matrices, one bank and one output each")
    dev = ys[0].device if isinstance(ys[0], torch.Tensor) else None
    for sb, sc, y in zip(signs_banks, scales_banks, ys):
        _dev(y, "y", (torch.float32,), None, dev)
        if y.dim() != 2 or y.shape[0] != T:
            raise ValueError(f"y has shape {tuple(y.shape)}, expected ({T}, d_out)")
        _bank(sb, sc, p, n_users, y.shape[1], d_in, dev)
    _dev(batch, "batch", None, None, dev)
    d_outs = (ctypes.c_int64 * len(ys))(*[y.shape[1] for y in ys])
    return int(lib().bd_delta_apply_encoded_n(_ptr(batch), _nbytes(batch), BD_BF16, int(T),
                                              int(d_in), int(n_users), len(ys), d_outs,
                                              _ptr_array(signs_banks), _ptr_array(scales_banks),
                                              ctypes.byref(p), _ptr_array(ys),
                                              _stream(ys[0], stream)))


def bd_decode_prepare(x, user_ids, n_users, scales_bank, p, workspace, stream=None) -> int:
    _dev(x, "x", (torch.float32, torch.bfloat16))
    T, d_in = x.shape
    dev = x.device
    _ids(user_ids, T, dev)
    if p.mode == BD_SCALE_COL:
        _scales(scales_bank, p, n_users, 1, d_in, dev)
    else:
        _dev(scales_bank, "scales_bank", None, None, dev, optional=True)
    _dev(workspace, "workspace", None, None, dev)
    return int(lib().bd_decode_prepare(_ptr(x), _dtype_code(x), T, d_in, _ptr(user_ids),
                                       int(n_users), _ptr(scales_bank), ctypes.byref(p),
                                       _ptr(workspace), _nbytes(workspace), _stream(x, stream)))


def bd_decode_apply(x, w_base, signs_bank, scales_bank, p, n_users, y, workspace,
                    stream=None) -> int:
    _dev(x, "x", (torch.float32, torch.bfloat16))
    T, d_in = x.shape
    dev = x.device
    d_out = w_base.shape[0]
    _dev(w_base, "w_base", (x.dtype,), (d_out, d_in), dev)
    _bank(signs_bank, scales_bank, p, n_users, d_out, d_in, dev)
    _dev(y, "y", (torch.float32, torch.bfloat16), (T, d_out), dev)
    _dev(workspace, "workspace", None, None, dev)
    return int(lib().bd_decode_apply(_ptr(x), _dtype_code(x), T, d_in, _ptr(w_base),
                                     d_out, _ptr(signs_bank), _ptr(scales_bank),
                                     ctypes.byref(p), int(n_users), _ptr(y), _dtype_code(y),
                                     _ptr(workspace), _nbytes(workspace), _stream(x, stream)))


# ------------------------------------------------------- allocating helpers

def workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns >= 256-byte aligned blocks
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def scales_dtype(p: bd_compress_params):
    return torch.float16 if p.scale_dtype == BD_F16 else torch.float32


def compress(w_fine: torch.Tensor, w_base: Optional[torch.Tensor], p: bd_compress_params,
             signs_out=None, scales_out=None, ws=None, stream=None,
             check: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    d_out, d_in = w_fine.shape
    dev = w_fine.device
    if signs_out is None:
        signs_out = torch.empty((d_out, d_in // 64), dtype=torch.int64, device=dev)
    n_sc = bd_scales_count(p, d_out, d_in)
    if n_sc < 0:
        raise BitDeltaError(BD_ERR_INVALID_ARG, "bd_scales_count")
    if scales_out is None:
        scales_out = torch.empty(n_sc, dtype=scales_dtype(p), device=dev)
    if ws is None:
        ws = workspace(bd_compress_workspace_bytes(p, d_out, d_in), dev)
    _check(bd_compress(w_fine, w_base, p, signs_out, scales_out, ws, stream), "bd_compress")
    if check:
        _check(bd_device_status(ws, stream), "bd_compress (device)")
    return signs_out, scales_out


def bd_select_axis(w_fine, w_base, clip_k, errors, axis, workspace, stream=None) -> int:
    _dev(w_fine, "w_fine", (torch.float32, torch.bfloat16))
    d_out, d_in = w_fine.shape
    dev = w_fine.device
    _dev(w_base, "w_base", (w_fine.dtype,), (d_out, d_in), dev, optional=True)
    _dev(errors, "errors", (torch.float64,), (2,), dev, optional=True)
    _dev(axis, "axis", (torch.int32,), (1,), dev, optional=True)
    _dev(workspace, "workspace", None, None, dev)
    return int(lib().bd_select_axis(_ptr(w_fine), _ptr(w_base), _dtype_code(w_fine), d_out, d_in,
                                    float(clip_k), _ptr(errors), _ptr(axis), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream(w_fine, stream)))


def bd_quantize_base(w, q_out, scales_out, stream=None) -> int:
    _dev(w, "w", (torch.float32, torch.bfloat16))
    d_out, d_in = w.shape
    _dev(q_out, "q_out", (torch.int8,), (d_out, d_in), w.device)
    _dev(scales_out, "scales_out", (torch.float32,), (d_out,), w.device)
    return int(lib().bd_quantize_base(_ptr(w), _dtype_code(w), d_out, d_in, _ptr(q_out),
                                      _ptr(scales_out), _stream(w, stream)))


def bd_apply_q8(x, wq, wscales, signs_bank, scales_bank, p, n_users, user_ids, y, workspace,
                stream=None) -> int:
    T, d_in, d_out = _apply_args(x, wq, signs_bank, scales_bank, p, n_users, user_ids, y,
                                 workspace, wdtypes=(torch.int8,))
    _dev(wscales, "wscales", (torch.float32,), (d_out,), x.device)
    return int(lib().bd_apply_q8(_ptr(x), _dtype_code(x), T, d_in, _ptr(wq), _ptr(wscales), d_out,
                                 _ptr(signs_bank), _ptr(scales_bank), ctypes.byref(p),
                                 int(n_users), _ptr(user_ids), _ptr(y), _dtype_code(y),
                                 _ptr(workspace), _nbytes(workspace),
                                 _stream(x, stream)))


def quantize_base(w: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """INT8 rows and their fp32 scales (bd_quantize_base)."""
    d_out, d_in = w.shape
    q = torch.empty((d_out, d_in), dtype=torch.int8, device=w.device)
    s = torch.empty(d_out, dtype=torch.float32, device=w.device)
    _check(bd_quantize_base(w, q, s, stream), "bd_quantize_base")
    return q, s


def bd_apply_q8_workspace_bytes(p, T: int, n_users: int, d_out: int, d_in: int, x_dtype: int,
                                y_dtype: int) -> int:
    return int(lib().bd_apply_q8_workspace_bytes(ctypes.byref(p), T, n_users, d_out, d_in,
                                                 x_dtype, y_dtype))


def apply_q8(x, wq, wscales, signs_bank, scales_bank, p, user_ids, y_dtype=torch.float32,
             ws=None, stream=None, check: bool = False) -> torch.Tensor:
    T, d_in = x.shape
    d_out = wq.shape[0]
    U = signs_bank.shape[0]
    y = torch.empty((T, d_out), dtype=y_dtype, device=x.device)
    if ws is None:
        ws = workspace(bd_apply_q8_workspace_bytes(p, T, U, d_out, d_in, _dtype_code(x),
                                                   _dtype_code(y)), x.device)
    _check(bd_apply_q8(x, wq, wscales, signs_bank, scales_bank, p, U, user_ids, y, ws, stream),
           "bd_apply_q8")
    if check:
        _check(bd_device_status(ws, stream), "bd_apply_q8 (device)")
    return y


def select_axis(w_fine: torch.Tensor, w_base: Optional[torch.Tensor], clip_k: float = 0.0,
                ws=None, stream=None, check: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Returns (errors float64[2] = {ROW, COL}, axis int32[1]) on the device."""
    d_out, d_in = w_fine.shape
    dev = w_fine.device
    errors = torch.empty(2, dtype=torch.float64, device=dev)
    axis = torch.empty(1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(bd_select_axis_workspace_bytes(d_out, d_in, clip_k), dev)
    _check(bd_select_axis(w_fine, w_base, clip_k, errors, axis, ws, stream), "bd_select_axis")
    if check:
        _check(bd_device_status(ws, stream), "bd_select_axis (device)")
    return errors, axis


def reconstruct(signs, scales, p, d_out, d_in, w_base=None, out_dtype=torch.float32, stream=None):
    out = torch.empty((d_out, d_in), dtype=out_dtype, device=signs.device)
    _check(bd_reconstruct(signs, scales, p, d_out, d_in, w_base, out, stream), "bd_reconstruct")
    return out


def apply(x: torch.Tensor, w_base: torch.Tensor, signs_bank: torch.Tensor,
          scales_bank: torch.Tensor, p: bd_compress_params, user_ids: torch.Tensor,
          y: Optional[torch.Tensor] = None, y_dtype=torch.float32, ws=None, stream=None,
          check: bool = False) -> torch.Tensor:
    T, d_in = x.shape
    d_out = w_base.shape[0]
    n_users = signs_bank.shape[0]
    if y is None:
        y = torch.empty((T, d_out), dtype=y_dtype, device=x.device)
    if ws is None:
        ws = workspace(bd_apply_workspace_bytes(p, T, n_users, d_out, d_in, _dtype_code(x),
                                                _dtype_code(y)), x.device)
    _check(bd_apply(x, w_base, signs_bank, scales_bank, p, n_users, user_ids, y, ws, stream),
           "bd_apply")
    if check:
        _check(bd_device_status(ws, stream), "bd_apply (device)")
    return y
