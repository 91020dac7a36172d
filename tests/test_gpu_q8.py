"""The INT8 base: bd_quantize_base against the oracle's row quantizer (codes and
scales bit for bit: both divide in binary32, correctly rounded), and bd_apply_q8
against the oracle's apply on the oracle's own INT8 rows (bf16 bar, max|err| <= 2e-2
rms; the delta term alone within 5e-3 rms, 1e-2 for COL, and the encoding's
element-wise bounds; the base term is exact products of bf16 tokens and integer codes,
accumulated in fp32 and scaled once per row).  Decode batches take the one-launch
kernel; the others (more than 16 tokens, COL and GROUP scales, rows wider than 4096)
the prepared batch with the tiled base product from the codes, over every tile shape
(64 x 64 to 256 x 256), ragged token and row counts included."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (DEV, TOL_BF16, assert_delta_within_bound, custom, gpu_bank, max_err_vs_rms,
                      o_sdtype, oracle_bank, to_np, tol_delta)
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [S.BF16, S.F32])
def test_quantize_base_matches_oracle(dtype):
    w = custom(130, 576, dtype, cid=2300)
    wb_dev = S.dev_wbase(w, 0)
    q, s = B.quantize_base(wb_dev)
    torch.cuda.synchronize()
    oq, os_ = O.quantize_rows(S.host_wbase(w, 0), dtype=O.BF16 if dtype == S.BF16 else O.F32)
    assert np.array_equal(to_np(q), oq)
    assert np.array_equal(to_np(s), os_)


def test_quantize_base_marks_rows_with_non_finite_weights():
    w = custom(40, 512, S.F32, cid=2310)
    wb = S.host_wbase(w, 0).copy()
    wb[3, 17] = np.nan
    wb[11, 0] = np.inf
    wb[30, 511] = -np.inf
    q, s = B.quantize_base(torch.from_numpy(wb).to(DEV))
    torch.cuda.synchronize()
    oq, os_ = O.quantize_rows(wb, dtype=O.F32)
    assert np.array_equal(to_np(q), oq)
    assert np.array_equal(to_np(s), os_, equal_nan=True)
    assert np.isnan(os_[[3, 11, 30]]).all()


CASES = [
    # (mode, scale dtype, d_out, d_in, ids, n_users, y dtype)
    ("matrix", B.BD_F32, 200, 1024, np.random.default_rng(1).permutation(16).astype(np.int32), 16, torch.float32),
    ("row", B.BD_F16, 130, 1088, np.array([2, 0, -1, 2, 1, 2, 0], np.int32), 3, torch.bfloat16),
    ("matrix", B.BD_F32, 64, 4096, np.array([1, 1, 0], np.int32), 2, torch.float32),
    # the prepared-batch path with the tiled INT8 product
    ("matrix", B.BD_F32, 200, 1024, np.random.default_rng(2).integers(-1, 4, 40).astype(np.int32), 4, torch.float32),
    ("row", B.BD_F16, 130, 4608, np.array([0, 2, 1, 1, -1, 0, 2, 2, 0], np.int32), 3, torch.bfloat16),
    ("col", B.BD_F16, 96, 1088, np.random.default_rng(3).integers(0, 3, 12).astype(np.int32), 3, torch.float32),
    ("group", B.BD_F32, 136, 2048, np.random.default_rng(4).integers(-1, 5, 70).astype(np.int32), 5, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[2]}x{c[3]}-T{len(c[4])}")
def test_apply_on_int8_base_matches_oracle(case):
    mode, sd, d_out, d_in, ids, U, ydt = case
    T = len(ids)
    w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=2400 + d_out)
    p = B.params(mode, 128, 0.0, sd)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(U))
    q, s = B.quantize_base(wb_dev)
    ids_dev = torch.from_numpy(ids).to(DEV)
    y = B.apply_q8(x_dev, q, s, signs, scales, p, ids_dev, y_dtype=ydt, check=True)
    y0 = B.apply_q8(x_dev, torch.zeros_like(q), s, signs, scales, p, ids_dev, check=True)
    torch.cuda.synchronize()
    wb = S.host_wbase(w, 0)
    oq, os_ = O.quantize_rows(wb, dtype=O.BF16)
    assert np.array_equal(to_np(q), oq) and np.array_equal(to_np(s), os_)
    words, osc = oracle_bank(w, 0, wb, p, range(U))
    yr, yb, yd = O.apply_q8(S.host_x(w, 0), oq, os_, words, osc, p.mode, ids, g=128,
                            sdtype=o_sdtype(p))
    err, rms = max_err_vs_rms(y.float().cpu().numpy(), yr)
    assert err <= TOL_BF16 * rms, (err, rms)
    err0, rms0 = max_err_vs_rms(y0.cpu().numpy(), yd)
    assert err0 <= tol_delta(mode) * rms0, (err0, rms0)
    assert_delta_within_bound(y0.cpu().numpy(), yd, S.host_x(w, 0), osc, p, ids)
    assert np.all(y0.cpu().numpy()[ids < 0] == 0)


TILE_CASES = [
    # (d_out, d_in, T): the tile each takes (256 x 256, 128 x 128, 64 x 64), ragged edges
    (14336, 1024, 1024),
    (4100, 2048, 1000),
    (700, 1536, 333),
]


@pytest.mark.parametrize("case", TILE_CASES, ids=lambda c: f"{c[0]}x{c[1]}-T{c[2]}")
def test_tiled_int8_product_over_tile_shapes(case):
    """The base product alone (no valid user: every id -1) on every tile shape, all
    tokens of sampled rows against the oracle's base term on the oracle's INT8 rows."""
    d_out, d_in, T = case
    w = custom(d_out, d_in, S.BF16, n_users=1, T=T, cid=2450 + d_out % 97)
    p = B.params("matrix")
    wb_dev = S.dev_wbase(w, 0)
    q, s = B.quantize_base(wb_dev)
    signs = torch.zeros((1, d_out, d_in // 64), dtype=torch.int64, device=DEV)
    sc = torch.zeros((1, 1), dtype=torch.float32, device=DEV)
    ids = np.full(T, -1, np.int32)
    y = B.apply_q8(S.dev_x(w, 0), q, s, signs, sc, p, torch.from_numpy(ids).to(DEV), check=True)
    rows = sorted({0, 1, d_out - 1} | set(np.random.default_rng(d_out).choice(d_out, 61, replace=False).tolist()))
    oq, os_ = O.quantize_rows(S.host_wbase(w, 0, rows), dtype=O.BF16)
    words = np.zeros((1, len(rows), d_in // 64), np.uint64)
    _, yb, _ = O.apply_q8(S.host_x(w, 0), oq, os_, words, np.zeros((1, 1), np.float32), p.mode,
                          ids, g=128)
    err, rms = max_err_vs_rms(y.cpu().numpy()[:, rows], yb)
    assert err <= 1e-5 * rms, (err, rms)  # exact products, fp32 sums of d_in terms


GROUPED_Q8_CASES = [
    ((4096, 1024, 1024), 4096, 512),   # q|k|v of the 8B layer: K split in 4
    ((4096,), 14336, 512),             # down: K split in 8
    ((1028, 1028, 1024), 8192, 300),   # ragged rows and tokens, split
    ((14336, 14336), 4096, 512),       # gate|up: no split
    ((512, 640), 1024, 40),            # small batch: the small tiles
]


@pytest.mark.parametrize("d_outs,d_in,T", GROUPED_Q8_CASES,
                         ids=lambda c: str(c) if not isinstance(c, tuple) else "x".join(map(str, c)))
def test_grouped_int8_gemm(d_outs, d_in, T):
    """bd_base_gemm_q8_n (INT8 rows of up to 4 matrices on one launch, K split through
    the workspace where bd_base_gemm_n would split): every token of sampled rows of every
    matrix against the oracle's base term on the oracle's INT8 rows (exact products,
    fp32 sums: 1e-5 rms), against the unsplit call within fp32 summation order, and bit
    for bit from one call to the next."""
    mats = [custom(d, d_in, S.BF16, T=T, cid=2900 + i) for i, d in enumerate(d_outs)]
    qs = [B.quantize_base(S.dev_wbase(w, 0)) for w in mats]
    x = S.dev_x(mats[0], 0)
    need = B.bd_base_gemm_n_workspace_bytes(B.BD_BF16, T, d_in, d_outs)
    ws = B.workspace(need, DEV) if need > 0 else None
    ys = [torch.empty(T, d, device=DEV) for d in d_outs]
    ys2 = [torch.empty(T, d, device=DEV) for d in d_outs]
    yn = [torch.empty(T, d, device=DEV) for d in d_outs]
    wq, wsc = [q for q, _ in qs], [sc for _, sc in qs]
    assert B.bd_base_gemm_q8_n(x, wq, wsc, ys, workspace=ws) == B.BD_OK
    assert B.bd_base_gemm_q8_n(x, wq, wsc, ys2, workspace=ws) == B.BD_OK
    assert B.bd_base_gemm_q8_n(x, wq, wsc, yn) == B.BD_OK  # no workspace: no split
    torch.cuda.synchronize()
    x_np = S.host_x(mats[0], 0)
    ids = np.full(T, -1, np.int32)
    for i, d in enumerate(d_outs):
        assert torch.equal(ys[i], ys2[i])
        rows = sorted({0, d - 1} | set(np.random.default_rng(d + i).choice(d, 40, replace=False).tolist()))
        oq, os_ = O.quantize_rows(S.host_wbase(mats[i], 0, rows), dtype=O.BF16)
        _, yb, _ = O.apply_q8(x_np, oq, os_, np.zeros((1, len(rows), d_in // 64), np.uint64),
                              np.zeros((1, 1), np.float32), O.MATRIX, ids)
        err, rms = max_err_vs_rms(ys[i].cpu().numpy()[:, rows], yb)
        assert err <= 1e-5 * rms, (i, err, rms)
        err, rms = max_err_vs_rms(ys[i].cpu().numpy(), yn[i].cpu().numpy().astype(np.float64))
        assert err <= 1e-5 * rms, (i, err, rms)


def test_grouped_int8_gemm_rejections():
    x = torch.zeros((128, 512), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((64, 512), dtype=torch.int8, device=DEV)
    s = torch.ones(64, dtype=torch.float32, device=DEV)
    y = torch.empty((128, 64), dtype=torch.float32, device=DEV)
    lib, c = B.lib(), __import__("ctypes")
    d = (c.c_int64 * 1)(64)
    P = (c.c_void_p * 1)
    args = lambda xd, din, wq, sc, yy: (x.data_ptr(), xd, 128, din, 1, wq, sc, d, yy, None, 0, None)
    ok = (P(q.data_ptr()), P(s.data_ptr()), P(y.data_ptr()))
    assert lib.bd_base_gemm_q8_n(*args(B.BD_F32, 512, *ok)) == B.BD_ERR_DTYPE
    assert lib.bd_base_gemm_q8_n(*args(B.BD_BF16, 500, *ok)) == B.BD_ERR_SHAPE
    assert lib.bd_base_gemm_q8_n(*args(B.BD_BF16, 512, P(None), ok[1], ok[2])) == B.BD_ERR_INVALID_ARG
    assert lib.bd_base_gemm_q8_n(*args(B.BD_BF16, 512, ok[0], P(s.data_ptr() + 2), ok[2])) == \
        B.BD_ERR_INVALID_ARG


def test_apply_q8_rejects_what_it_does_not_serve():
    p = B.params("matrix")
    x = torch.zeros((4, 512), dtype=torch.float32, device=DEV)  # fp32 activations
    q = torch.zeros((64, 512), dtype=torch.int8, device=DEV)
    s = torch.ones(64, dtype=torch.float32, device=DEV)
    signs = torch.zeros((1, 64, 8), dtype=torch.int64, device=DEV)
    sc = torch.zeros((1, 1), dtype=torch.float32, device=DEV)
    ids = torch.zeros(4, dtype=torch.int32, device=DEV)
    y = torch.empty((4, 64), dtype=torch.float32, device=DEV)
    ws = B.workspace(1 << 20, DEV)
    assert B.bd_apply_q8(x, q, s, signs, sc, p, 1, ids, y, ws) == B.BD_ERR_UNSUPPORTED
