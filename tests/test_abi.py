"""Host-only checks of the C ABI library: it loads, exports what the header
declares, answers size queries, and rejects bad arguments before enqueueing
anything (every call below fails validation, so no kernel is launched)."""
import ctypes
import os
import re

import pytest

torch = pytest.importorskip("torch")  # loads the HIP runtime the library binds to

from tenant_serving_amd import bitdelta as B  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "bitdelta.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bd_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = B.lib()
    names = header_functions()
    assert "bd_compress" in names and "bd_apply" in names and "bd_reconstruct" in names
    for n in names:
        assert hasattr(lib, n), f"missing export {n}"
    assert lib.bd_abi_version() == 3


def test_status_strings():
    for s in range(10):
        assert B.status_string(s) and B.status_string(s) != "unknown status"


def test_size_queries():
    assert B.bd_signs_bytes(4096, 4096) == 4096 * 4096 // 8
    assert B.bd_signs_bytes(4096, 100) == 0
    p = B.params("group", 128)
    assert B.bd_scales_count(p, 256, 512) == 256 * 4
    assert B.bd_scales_count(B.params("row"), 17408, 5120) == 17408
    assert B.bd_scales_count(B.params("col"), 5120, 17408) == 17408
    assert B.bd_scales_count(B.params("matrix"), 7, 64) == 1
    assert B.bd_scales_count(B.params("group", 100), 8, 512) == -1
    assert B.bd_compress_workspace_bytes(p, 256, 512) >= 256
    assert B.bd_apply_workspace_bytes(p, 16, 4, 256, 512, B.BD_BF16, B.BD_F32) > 0


def test_llama8b_stack_signs_bytes():
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096),
              (14336, 4096), (4096, 14336)]
    assert 32 * sum(B.bd_signs_bytes(o, i) for o, i in shapes) == 872_415_232


def _compress_raw(p, d_out=64, d_in=128, wf=1, ws=1, ws_bytes=1 << 20, dtype=B.BD_BF16,
                  signs=1, scales=1):
    L = B.lib()
    vp = ctypes.c_void_p
    return L.bd_compress(vp(wf) if wf else None, None, dtype, d_out, d_in,
                         ctypes.byref(p) if p is not None else None, vp(signs) if signs else None,
                         vp(scales) if scales else None, vp(ws) if ws else None, ws_bytes, None)


def test_compress_rejects_bad_arguments_synchronously():
    ok = B.params("matrix")
    assert _compress_raw(None) == B.BD_ERR_INVALID_ARG
    assert _compress_raw(ok, wf=0) == B.BD_ERR_INVALID_ARG
    assert _compress_raw(ok, signs=0) == B.BD_ERR_INVALID_ARG
    assert _compress_raw(ok, d_in=100) == B.BD_ERR_SHAPE
    assert _compress_raw(ok, d_out=0) == B.BD_ERR_SHAPE
    assert _compress_raw(ok, dtype=B.BD_F16) == B.BD_ERR_DTYPE
    assert _compress_raw(B.params("matrix", bits=2)) == B.BD_ERR_UNSUPPORTED
    assert _compress_raw(B.params("group", 100)) == B.BD_ERR_UNSUPPORTED
    assert _compress_raw(B.params("group", 256), d_in=192) == B.BD_ERR_SHAPE
    assert _compress_raw(B.params("matrix", scale_dtype=B.BD_BF16)) == B.BD_ERR_DTYPE
    assert _compress_raw(B.params("matrix", clip_k=float("nan"))) == B.BD_ERR_INVALID_ARG
    assert _compress_raw(ok, ws=0) == B.BD_ERR_WORKSPACE
    assert _compress_raw(ok, ws_bytes=8) == B.BD_ERR_WORKSPACE
    assert _compress_raw(ok, ws=256 + 8) == B.BD_ERR_WORKSPACE      # misaligned workspace
    assert _compress_raw(ok, wf=256 + 8, ws=1 << 12) == B.BD_ERR_INVALID_ARG  # misaligned input


def test_apply_rejects_bad_arguments_synchronously():
    L = B.lib()
    vp = ctypes.c_void_p

    def call(p=B.params("matrix"), T=16, d_in=128, d_out=64, U=4, xd=B.BD_BF16, yd=B.BD_F32,
             ws=1 << 12, ws_bytes=1 << 30, x=1 << 12):
        return L.bd_apply(vp(x) if x else None, xd, T, d_in, vp(1 << 12), d_out, vp(1 << 12),
                          vp(1 << 12), ctypes.byref(p), U, vp(1 << 12), vp(1 << 12), yd,
                          vp(ws) if ws else None, ws_bytes, None)

    assert call(d_in=96) == B.BD_ERR_SHAPE
    assert call(xd=B.BD_F16) == B.BD_ERR_DTYPE
    assert call(yd=B.BD_F16) == B.BD_ERR_DTYPE
    assert call(T=-1) == B.BD_ERR_INVALID_ARG
    assert call(U=-2) == B.BD_ERR_INVALID_ARG
    assert call(p=B.params("group", 1024)) == B.BD_ERR_UNSUPPORTED  # groups of 8..512 columns
    assert call(p=B.params("group", 48)) == B.BD_ERR_UNSUPPORTED    # powers of two
    assert call(T=9000) == B.BD_ERR_UNSUPPORTED
    assert call(ws=0) == B.BD_ERR_WORKSPACE
    assert call(ws_bytes=16) == B.BD_ERR_WORKSPACE
    assert call(x=0) == B.BD_ERR_INVALID_ARG
    assert call(x=(1 << 12) + 2) == B.BD_ERR_INVALID_ARG


def test_paged_apply_rejects_bad_arguments_synchronously():
    L = B.lib()
    vp = ctypes.c_void_p
    p = B.params("row", 128, 0.0, B.BD_F16)
    d_out, d_in, T, K = 64, 128, 16, 3
    sbytes, cbytes = d_out * d_in // 8, d_out * 2
    need = B.bd_apply_paged_workspace_bytes(p, T, K, d_out, d_in, B.BD_BF16, B.BD_F32)
    assert need >= B.bd_apply_workspace_bytes(p, T, K, d_out, d_in, B.BD_BF16, B.BD_F32) + T * 4
    assert B.bd_apply_paged_workspace_bytes(p, T, K, d_out, 96, B.BD_BF16, B.BD_F32) == 0

    def call(ss=4096, cs=4096, d_in=d_in, ws=1 << 12, ws_bytes=1 << 30, ids=1 << 12, table=1 << 12,
             n_users=5, xd=B.BD_BF16):
        return L.bd_apply_paged(vp(1 << 12), xd, T, d_in, vp(1 << 12), d_out, vp(1 << 12),
                                vp(1 << 12), ss, cs, K, ctypes.byref(p), vp(table) if table else None,
                                n_users, vp(ids) if ids else None, vp(1 << 12), B.BD_F32,
                                vp(ws) if ws else None, ws_bytes, None)

    assert call(d_in=96) == B.BD_ERR_SHAPE
    assert call(xd=B.BD_F16) == B.BD_ERR_DTYPE
    assert call(ss=sbytes - 16) == B.BD_ERR_INVALID_ARG   # a slot smaller than one bank
    assert call(ss=sbytes + 8) == B.BD_ERR_INVALID_ARG    # not a multiple of 16
    assert call(cs=cbytes - 2) == B.BD_ERR_INVALID_ARG
    assert call(n_users=-1) == B.BD_ERR_INVALID_ARG
    assert call(ws=0) == B.BD_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == B.BD_ERR_WORKSPACE
    assert call(ids=0) == B.BD_ERR_INVALID_ARG
    assert call(table=0) == B.BD_ERR_INVALID_ARG
    assert call(table=(1 << 12) + 2) == B.BD_ERR_INVALID_ARG


def _select_raw(d_out=64, d_in=128, dtype=B.BD_BF16, clip_k=0.0, wf=1 << 12, ws=1 << 16,
                ws_bytes=1 << 30, errors=1 << 20, axis=1 << 20):
    # fake, never dereferenced device addresses: every case fails before any launch
    L = B.lib()
    return int(L.bd_select_axis(wf, None, dtype, d_out, d_in, clip_k, errors, axis, ws, ws_bytes,
                                None))


def test_select_axis_sizes_and_synchronous_errors():
    assert B.bd_select_axis_workspace_bytes(256, 512, 0.0) > 0
    assert B.bd_select_axis_workspace_bytes(256, 512, 3.0) > B.bd_select_axis_workspace_bytes(256, 512, 0.0)
    assert B.bd_select_axis_workspace_bytes(256, 100, 0.0) == 0
    assert _select_raw(wf=0) == B.BD_ERR_INVALID_ARG
    assert _select_raw(d_in=100) == B.BD_ERR_SHAPE
    assert _select_raw(d_out=0) == B.BD_ERR_SHAPE
    assert _select_raw(dtype=B.BD_F16) == B.BD_ERR_DTYPE
    assert _select_raw(clip_k=float("nan")) == B.BD_ERR_INVALID_ARG
    assert _select_raw(ws=0) == B.BD_ERR_WORKSPACE
    assert _select_raw(ws_bytes=8) == B.BD_ERR_WORKSPACE
    assert _select_raw(ws=256 + 8) == B.BD_ERR_WORKSPACE
    assert _select_raw(wf=256 + 8) == B.BD_ERR_INVALID_ARG
    assert _select_raw(errors=(1 << 20) + 4) == B.BD_ERR_INVALID_ARG


def test_int8_base_entry_points_reject_bad_arguments_synchronously():
    L = B.lib()
    # fake, never dereferenced device addresses: every case fails before any launch
    assert L.bd_quantize_base(None, B.BD_BF16, 64, 128, 1 << 12, 1 << 12, None) == B.BD_ERR_INVALID_ARG
    assert L.bd_quantize_base(1 << 12, B.BD_F16, 64, 128, 1 << 12, 1 << 12, None) == B.BD_ERR_DTYPE
    assert L.bd_quantize_base(1 << 12, B.BD_BF16, 0, 128, 1 << 12, 1 << 12, None) == B.BD_ERR_SHAPE

    def q8(p, T=4, d_in=512, xdt=B.BD_BF16, wq=1 << 12, ws=1 << 16, ws_bytes=1 << 30):
        return int(L.bd_apply_q8(1 << 12, xdt, T, d_in, wq, 1 << 12, 64, 1 << 12, 1 << 12,
                                 ctypes.byref(p), 2, 1 << 12, 1 << 12, B.BD_F32, ws, ws_bytes, None))

    assert q8(B.params("group", 256), d_in=384) == B.BD_ERR_SHAPE  # groups divide d_in
    assert q8(B.params("matrix"), T=9000) == B.BD_ERR_UNSUPPORTED
    assert q8(B.params("matrix"), xdt=B.BD_F32) == B.BD_ERR_UNSUPPORTED
    p = B.params("row", 128, 0.0, B.BD_F16)
    dec = B.bd_apply_q8_workspace_bytes(p, 4, 2, 64, 512, B.BD_BF16, B.BD_F32)
    gen = B.bd_apply_q8_workspace_bytes(p, 4, 2, 64, 4608, B.BD_BF16, B.BD_F32)  # past decode
    assert dec > 0 and gen >= B.bd_batch_workspace_bytes(4, 2, 4608, B.BD_BF16)
    assert q8(p, d_in=4608, ws_bytes=gen - 1) == B.BD_ERR_WORKSPACE
    assert q8(B.params("matrix"), d_in=100) == B.BD_ERR_SHAPE
    assert q8(B.params("matrix"), ws=0) == B.BD_ERR_WORKSPACE
    assert q8(B.params("matrix"), wq=0) == B.BD_ERR_INVALID_ARG
    assert q8(B.params("matrix"), wq=(1 << 12) + 8) == B.BD_ERR_INVALID_ARG


def test_prepared_batch_entry_points_check_the_batch_size():
    """bd_delta_apply, bd_batch_encode and bd_delta_apply_encoded write into or read a
    prepared batch whose size depends on T and d_in: a smaller buffer is rejected
    before anything is enqueued (fake, never dereferenced device addresses)."""
    L = B.lib()
    vp = ctypes.c_void_p
    p = B.params("matrix")
    T, U, d_in, d_out = 64, 8, 512, 256
    need = B.bd_batch_workspace_bytes(T, U, d_in, B.BD_BF16)
    assert need > 0
    a = vp(1 << 12)

    def delta(nb):
        return L.bd_delta_apply(a, nb, a, B.BD_BF16, T, d_in, U, d_out, a, a, ctypes.byref(p), a, None)

    def enc(nb, xd=B.BD_BF16):
        return L.bd_batch_encode(a, nb, a, xd, T, d_in, U, None, ctypes.byref(p), None)

    def applied(nb, xd=B.BD_BF16):
        return L.bd_delta_apply_encoded(a, nb, xd, T, d_in, U, d_out, a, a, ctypes.byref(p), a, None)

    assert delta(need - 256) == B.BD_ERR_WORKSPACE
    assert enc(need - 256) == B.BD_ERR_WORKSPACE
    assert applied(need - 256) == B.BD_ERR_WORKSPACE
    assert enc(need, xd=B.BD_F32) == B.BD_ERR_DTYPE
    assert applied(need, xd=B.BD_F32) == B.BD_ERR_DTYPE
    assert L.bd_batch_encode(a, need, None, B.BD_BF16, T, d_in, U, None, ctypes.byref(p),
                             None) == B.BD_ERR_INVALID_ARG
    # COL encodings fold in the column scales: they are required
    pc = B.params("col", scale_dtype=B.BD_F16)
    assert L.bd_batch_encode(a, need, a, B.BD_BF16, T, d_in, U, None, ctypes.byref(pc),
                             None) == B.BD_ERR_INVALID_ARG


def test_binding_rejects_host_strided_and_mistyped_tensors():
    """The Python binding checks device, contiguity, dtype and shape before any
    pointer reaches the library (a host pointer or int64 ids would otherwise be read
    as device data)."""
    p = B.params("matrix")
    T, U, d_out, d_in = 4, 2, 64, 128
    cpu = torch.device("cpu")
    x = torch.zeros(T, d_in, dtype=torch.bfloat16, device=cpu)
    wb = torch.zeros(d_out, d_in, dtype=torch.bfloat16, device=cpu)
    signs = torch.zeros(U, d_out, d_in // 64, dtype=torch.int64, device=cpu)
    scales = torch.zeros(U, 1, dtype=torch.float32, device=cpu)
    ids = torch.zeros(T, dtype=torch.int32, device=cpu)
    y = torch.zeros(T, d_out, dtype=torch.float32, device=cpu)
    ws = torch.zeros(1 << 16, dtype=torch.uint8, device=cpu)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.bd_apply(x, wb, signs, scales, p, U, ids, y, ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.bd_compress(wb, wb, p, signs[0], scales[0], ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.bd_batch_prepare(x, ids, U, ws)
    # each argument's dtype, shape and contiguity are checked before its device, so the
    # checks themselves run here on host tensors
    with pytest.raises(TypeError, match="int64"):
        B._ids(torch.zeros(T, dtype=torch.int64), T, None)
    with pytest.raises(ValueError, match="shape"):
        B._ids(torch.zeros(T + 1, dtype=torch.int32), T, None)
    with pytest.raises(ValueError, match="shape"):
        B._bank(signs[:, :32].contiguous(), scales, p, U, d_out, d_in, None)
    with pytest.raises(ValueError, match="contiguous"):
        B._dev(torch.zeros(d_out, T).t(), "y", (torch.float32,), (T, d_out))
    with pytest.raises(ValueError, match="scales_bank holds"):
        B._scales(scales, B.params("row"), U, d_out, d_in, None)  # (U, 1) for ROW
    with pytest.raises(TypeError):
        B._scales(scales.half(), p, U, d_out, d_in, None)
    with pytest.raises(TypeError):
        B._bank(signs.int(), scales, p, U, d_out, d_in, None)
    with pytest.raises(TypeError):
        B._dev([1, 2], "x")
    with pytest.raises(ValueError, match="required"):
        B._dev(None, "x")
