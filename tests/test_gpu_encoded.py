"""The two halves of the delta product (bd_batch_encode, bd_delta_apply_encoded): one
encoding of the activations shared by several matrices gives, bit for bit, what
bd_delta_apply gives per matrix; a product asked of a batch encoded for another
scale mode adds nothing and reports BD_ERR_BATCH; the result matches the oracle."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, custom, gpu_bank, max_err_vs_rms, o_sdtype, oracle_bank, tol_delta
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mode", ["matrix", "row", "group"])
def test_shared_encoding_equals_per_matrix_delta_apply(mode):
    T, U, d_in = 70, 5, 1152  # several tiles, a ragged 512-column unit
    ids = np.array([(7 * t) % (U + 1) - 1 for t in range(T)], dtype=np.int32)  # -1 .. U-1
    p = B.params(mode, 128, 0.0, B.BD_F16 if mode == "row" else B.BD_F32)
    mats = []
    for k, d_out in enumerate((96, 200)):
        w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=2600 + k)
        wb = S.dev_wbase(w, 0)
        signs, scales = gpu_bank(w, 0, wb, p, list(range(U)))
        mats.append((w, wb, signs, scales))
    x = S.dev_x(mats[0][0], 0)
    ids_dev = torch.from_numpy(ids).to(DEV)
    bt = B.workspace(B.bd_batch_workspace_bytes(T, U, d_in, B.BD_BF16), DEV)
    assert B.bd_batch_prepare(x, ids_dev, U, bt) == B.BD_OK
    ref = []
    for w, wb, signs, scales in mats:
        y = torch.zeros(T, wb.shape[0], device=DEV)
        assert B.bd_delta_apply(bt, x, U, signs, scales, p, y) == B.BD_OK
        ref.append(y)
    assert B.bd_batch_encode(bt, x, U, None, p) == B.BD_OK
    for (w, wb, signs, scales), yr in zip(mats, ref):
        y = torch.zeros(T, wb.shape[0], device=DEV)
        assert B.bd_delta_apply_encoded(bt, T, d_in, U, signs, scales, p, y) == B.BD_OK
        torch.cuda.synchronize()
        assert torch.equal(y, yr)
    assert B.bd_device_status(bt) == B.BD_OK
    # and the delta term against the oracle (zero base)
    w, wb, signs, scales = mats[1]
    y = torch.zeros(T, wb.shape[0], device=DEV)
    assert B.bd_delta_apply_encoded(bt, T, d_in, U, signs, scales, p, y) == B.BD_OK
    wb_np = S.host_wbase(w, 0)
    words, scs = oracle_bank(w, 0, wb_np, p, list(range(U)))
    _, _, yd = O.apply(S.host_x(mats[0][0], 0), wb_np, words, scs, p.mode, ids,
                       g=p.group_size, sdtype=o_sdtype(p))
    err, rms = max_err_vs_rms(y.cpu().numpy(), yd)
    assert err <= tol_delta(mode) * rms, (mode, err, rms)


def test_product_on_another_modes_encoding_reports_batch_error():
    T, U, d_in, d_out = 20, 2, 512, 64
    ids = torch.zeros(T, dtype=torch.int32, device=DEV)
    x = torch.randn(T, d_in, device=DEV).to(torch.bfloat16)
    bt = B.workspace(B.bd_batch_workspace_bytes(T, U, d_in, B.BD_BF16), DEV)
    assert B.bd_batch_prepare(x, ids, U, bt) == B.BD_OK
    pg, pm = B.params("group", 128), B.params("matrix")
    signs = torch.zeros(U, d_out, d_in // 64, dtype=torch.int64, device=DEV)
    sc_m = torch.ones(U, 1, device=DEV)
    # prepared but never encoded: nothing is added
    y = torch.zeros(T, d_out, device=DEV)
    assert B.bd_delta_apply_encoded(bt, T, d_in, U, signs, sc_m, pm, y) == B.BD_OK
    assert B.bd_device_status(bt) == B.BD_ERR_BATCH
    assert torch.count_nonzero(y) == 0
    # encoded for GROUP, applied as MATRIX: nothing is added
    assert B.bd_batch_prepare(x, ids, U, bt) == B.BD_OK
    assert B.bd_device_status(bt) == B.BD_OK
    assert B.bd_batch_encode(bt, x, U, None, pg) == B.BD_OK
    assert B.bd_delta_apply_encoded(bt, T, d_in, U, signs, sc_m, pm, y) == B.BD_OK
    assert B.bd_device_status(bt) == B.BD_ERR_BATCH
    assert torch.count_nonzero(y) == 0


def test_grouped_calls_equal_per_matrix_calls():
    """bd_base_gemm_n and bd_delta_apply_encoded_n on q/k/v-like matrices of one input
    (row counts that pick different tile shapes and row tiles alone) give, bit for bit,
    the per-matrix calls."""
    T, U, d_in = 200, 6, 1024
    ids = np.array([(t * 5) % U if t % 7 else -1 for t in range(T)], dtype=np.int32)
    p = B.params("matrix")
    mats = []
    for k, d_out in enumerate((512, 128, 128, 72)):
        w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=2700 + k)
        wb = S.dev_wbase(w, 0)
        signs, scales = gpu_bank(w, 0, wb, p, list(range(U)))
        mats.append((wb, signs, scales))
    x = S.dev_x(custom(64, d_in, S.BF16, T=T, cid=2710), 0)
    ids_dev = torch.from_numpy(ids).to(DEV)
    bt = B.workspace(B.bd_batch_workspace_bytes(T, U, d_in, B.BD_BF16), DEV)
    assert B.bd_batch_prepare(x, ids_dev, U, bt) == B.BD_OK
    assert B.bd_batch_encode(bt, x, U, None, p) == B.BD_OK
    ref = []
    for wb, signs, scales in mats:
        y = torch.empty(T, wb.shape[0], device=DEV)
        assert B.bd_base_gemm(x, wb, y) == B.BD_OK
        assert B.bd_delta_apply_encoded(bt, T, d_in, U, signs, scales, p, y) == B.BD_OK
        ref.append(y)
    ys = [torch.empty(T, wb.shape[0], device=DEV) for wb, _, _ in mats]
    assert B.bd_base_gemm_n(x, [m[0] for m in mats], ys) == B.BD_OK
    assert B.bd_delta_apply_encoded_n(bt, T, d_in, U, [m[1] for m in mats], [m[2] for m in mats],
                                      p, ys) == B.BD_OK
    torch.cuda.synchronize()
    assert B.bd_device_status(bt) == B.BD_OK
    for y, yr in zip(ys, ref):
        assert torch.equal(y, yr)


@pytest.mark.parametrize("d_outs,d_in,T,split", [
    ((4096, 1024, 1024), 4096, 512, False),  # q|k|v: 128 x 128, whole K
    ((4096,), 14336, 512, True),             # down: 128 x 256, 4 parts
    ((1028, 1028, 1024), 8192, 300, True),   # ragged rows, T: 128 x 256, 4 parts
    ((14336, 14336), 4096, 256, True),       # gate|up at 256 tokens: 256 x 256, 2 parts
    ((4096,), 14336, 256, True)])            # down at 256 tokens: 128 x 128, 4 parts
def test_grouped_gemm_with_k_split(d_outs, d_in, T, split):
    """bd_base_gemm_n with a workspace (K split in ordered parts where the plan splits):
    against the oracle's base term on sampled rows of every matrix (exact bf16 products,
    fp32 sums: 1e-5 rms), against the launch without a workspace within the sum of both
    bounds, and bit for bit from one call to the next."""
    need = B.bd_base_gemm_n_workspace_bytes(B.BD_BF16, T, d_in, d_outs)
    assert (need > 0) == split
    ws_ = [custom(d, d_in, S.BF16, T=T, cid=2750 + i) for i, d in enumerate(d_outs)]
    wbs = [S.dev_wbase(w, 0) for w in ws_]
    x = S.dev_x(ws_[0], 0)
    ws = B.workspace(need, DEV)
    ys = [torch.empty(T, d, device=DEV) for d in d_outs]
    assert B.bd_base_gemm_n(x, wbs, ys, workspace=ws) == B.BD_OK
    ys2 = [torch.empty(T, d, device=DEV) for d in d_outs]
    assert B.bd_base_gemm_n(x, wbs, ys2, workspace=ws) == B.BD_OK
    yn = [torch.empty(T, d, device=DEV) for d in d_outs]
    assert B.bd_base_gemm_n(x, wbs, yn) == B.BD_OK  # no workspace: no split
    torch.cuda.synchronize()
    x_np = S.host_x(ws_[0], 0)
    ids = np.full(T, -1, np.int32)
    for i, d in enumerate(d_outs):
        assert torch.equal(ys[i], ys2[i])
        rows = sorted({0, d - 1} | set(np.random.default_rng(d).choice(d, 40, replace=False).tolist()))
        _, yb, _ = O.apply(x_np, S.host_wbase(ws_[i], 0, rows), np.zeros((1, len(rows), d_in // 64), np.uint64),
                           np.zeros((1, 1), np.float32), O.MATRIX, ids)
        err, rms = max_err_vs_rms(ys[i].cpu().numpy()[:, rows], yb)
        assert err <= 1e-5 * rms, (i, err, rms)
        # two fp32 summation orders (K parts, tile shape), each within 1e-5 rms of the
        # binary64 product: their difference within the sum of the two bounds
        err, rms = max_err_vs_rms(ys[i].cpu().numpy(), yn[i].cpu().numpy().astype(np.float64))
        assert err <= 2e-5 * rms, (i, err, rms)
