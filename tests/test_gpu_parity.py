"""GPU parity of the HIP library against the CPU oracle on small shapes that
still span several tiles and a ragged tail (d_in = 512 + 64, d_out not a
multiple of the 64-row tile).  Inputs come from the seeded generator: host
fills feed the oracle, device fills feed the library.  Bar: packed signs
bit-exact, scales within 1e-6 relative, outputs within max|err| <= 1e-4 rms
(fp32) or 2e-2 rms (bf16) of the oracle, plus the same rule on the delta term
alone (base weight zero)."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (DEV, TOL_BF16, TOL_F32, assert_delta_within_bound, custom, gpu_bank,
                      max_err_vs_rms, o_sdtype,
                      oracle_bank, rel_err_ok, scales_as_f64, to_np, tol_delta)
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

pytestmark = pytest.mark.gpu


def test_device_generator_matches_host_generator():
    for dtype in (S.F32, S.BF16):
        w = custom(70, 576, dtype, outlier_p=0.01, cid=1001)
        wb_dev = S.dev_wbase(w, 0)
        wf_dev = S.dev_wfine(w, 0, 3, wb_dev)
        wb = S.host_wbase(w, 0)
        assert np.array_equal(to_np(wb_dev), wb)
        assert np.array_equal(to_np(wf_dev), S.host_wfine(w, 0, 3, wbase=wb))


COMPRESS_CASES = [
    # (dtype, mode, group, clip, scale dtype, base given, d_out, d_in)
    (S.F32, "group", 128, 0.0, B.BD_F32, True, 256, 512),
    (S.F32, "matrix", 128, 3.0, B.BD_F32, True, 50, 576),
    (S.F32, "group", 64, 3.0, B.BD_F32, False, 50, 576),
    (S.BF16, "matrix", 128, 0.0, B.BD_F32, True, 300, 1024),
    (S.BF16, "matrix", 128, 3.0, B.BD_F32, True, 33, 576),
    (S.BF16, "group", 128, 3.0, B.BD_F32, True, 100, 1152),
    (S.BF16, "group", 32, 0.0, B.BD_F16, True, 17, 576),
    (S.BF16, "row", 128, 0.0, B.BD_F16, True, 130, 576),
    (S.BF16, "col", 128, 0.0, B.BD_F16, True, 130, 576),
    (S.BF16, "row", 128, 3.0, B.BD_F32, False, 65, 1024),
    (S.BF16, "col", 128, 3.0, B.BD_F32, True, 200, 640),
]


@pytest.mark.parametrize("case", COMPRESS_CASES, ids=lambda c: f"{c[0]}-{c[1]}{c[2]}-clip{c[3]}-s{c[4]}-base{int(c[5])}-{c[6]}x{c[7]}")
def test_compress_parity(case):
    dtype, mode, g, clip, sd, has_base, d_out, d_in = case
    w = custom(d_out, d_in, dtype, outlier_p=0.002 if clip else 0.0, cid=1100 + d_out)
    p = B.params(mode, g, clip, sd)
    wb_dev = S.dev_wbase(w, 0)
    wf_dev = S.dev_wfine(w, 0, 0, wb_dev)
    wb = S.host_wbase(w, 0)
    wf = S.host_wfine(w, 0, 0, wbase=wb)
    if not has_base:  # the library then takes w_fine as the delta itself
        wf = host_delta(wf, wb, dtype)  # prepared on the host, uploaded to the device
        wf_dev = upload(wf, dtype)
    signs, scales = B.compress(wf_dev, wb_dev if has_base else None, p, check=True)
    words, osc, st, bad = O.compress(wf, wb if has_base else None, p.mode, g=g, clip_k=clip,
                                     sdtype=o_sdtype(p), dtype=dtype)
    assert bad == 0
    assert np.array_equal(to_np(signs), words)
    assert rel_err_ok(scales_as_f64(to_np(scales), p), scales_as_f64(osc, p))


def host_delta(wf, wb, dtype):
    d = S.as_f32(wf, dtype) - S.as_f32(wb, dtype)
    if dtype == S.F32:
        return d
    u = d.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def upload(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if dtype == S.BF16 else np.float32))
    t = t.view(torch.bfloat16) if dtype == S.BF16 else t
    return t.to(DEV)


def test_compress_zero_and_negative_zero_deltas_map_to_plus_one():
    w = custom(64, 512, S.F32, cid=1200)
    wb = S.host_wbase(w, 0)
    wf = S.host_wfine(w, 0, 0, wbase=wb)
    wf[:, :128] = wb[:, :128]      # exact zero deltas
    wf[:3, 128:192] = -0.0         # -0.0 - 0.0 = -0.0 deltas
    wb[:3, 128:192] = 0.0
    p = B.params("group", 128)
    signs, scales = B.compress(upload(wf, S.F32), upload(wb, S.F32), p, check=True)
    words, osc, _, _ = O.compress(wf, wb, p.mode, g=128, dtype=S.F32)
    got = to_np(signs)
    assert np.array_equal(got, words)
    assert (got[:, :2] == np.uint64(0xFFFFFFFFFFFFFFFF)).all()
    assert np.array_equal(to_np(scales), osc)


def test_compress_nonfinite_sets_status():
    w = custom(64, 512, S.F32, cid=1201)
    wb_dev = S.dev_wbase(w, 0)
    wf_dev = S.dev_wfine(w, 0, 0, wb_dev)
    wf_dev[5, 7] = float("nan")
    p = B.params("matrix")
    ws = B.workspace(B.bd_compress_workspace_bytes(p, 64, 512), DEV)
    B.compress(wf_dev, wb_dev, p, ws=ws)
    assert B.bd_device_status(ws) == B.BD_ERR_NONFINITE
    wf_dev[5, 7] = 0.0
    B.compress(wf_dev, wb_dev, p, ws=ws)   # the status word is reset by every call
    assert B.bd_device_status(ws) == B.BD_OK


def _ids_mixed(T_users=(0, 1, 17, 70, 3), extra_none=2, seed=5):
    ids = []
    for u, n in enumerate(T_users):
        ids += [u] * n
    ids += [-1] * extra_none
    rng = np.random.default_rng(seed)
    rng.shuffle(ids)
    return np.array(ids, dtype=np.int32)


APPLY_CASES = [
    # (dtype, mode, group, scale dtype, d_out, d_in, y dtype)
    (S.BF16, "matrix", 128, B.BD_F32, 80, 576, torch.float32),
    (S.BF16, "group", 128, B.BD_F32, 130, 1152, torch.float32),
    (S.BF16, "group", 256, B.BD_F32, 64, 1024, torch.bfloat16),
    (S.BF16, "row", 128, B.BD_F16, 200, 576, torch.float32),
    (S.BF16, "col", 128, B.BD_F16, 96, 1088, torch.float32),
    (S.F32, "group", 128, B.BD_F32, 80, 640, torch.float32),
    (S.F32, "matrix", 128, B.BD_F32, 33, 512, torch.float32),
    (S.F32, "col", 128, B.BD_F16, 40, 640, torch.float32),
]


@pytest.mark.parametrize("case", APPLY_CASES, ids=lambda c: f"{c[0]}-{c[1]}{c[2]}-s{c[3]}-{c[4]}x{c[5]}-{str(c[6])[6:]}")
def test_apply_parity(case):
    dtype, mode, g, sd, d_out, d_in, ydt = case
    ids = _ids_mixed()
    T, U = len(ids), 5
    w = custom(d_out, d_in, dtype, n_users=U, T=T, b=5e-3, cid=1300 + d_out + d_in)
    p = B.params(mode, g, 0.0, sd)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(U))
    ids_dev = torch.from_numpy(ids).to(DEV)
    y = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, y_dtype=ydt, check=True)

    wb = S.host_wbase(w, 0)
    x = S.host_x(w, 0)
    words, osc = oracle_bank(w, 0, wb, p, range(U))
    assert np.array_equal(to_np(signs), words)
    assert rel_err_ok(scales_as_f64(to_np(scales), p), scales_as_f64(osc, p))
    yr, yb, yd = O.apply(x, wb, words, osc, p.mode, ids, g=g, sdtype=o_sdtype(p))
    tol = TOL_F32 if dtype == S.F32 else TOL_BF16
    got = y.float().cpu().numpy()
    err, rms = max_err_vs_rms(got, yr)
    assert err <= tol * rms, (err, rms)
    # the delta term alone: same bank, zero base weight
    y0 = B.apply(x_dev, torch.zeros_like(wb_dev), signs, scales, p, ids_dev, check=True)
    err0, rms0 = max_err_vs_rms(y0.cpu().numpy(), yd)
    tol0 = TOL_F32 if dtype == S.F32 else tol_delta(mode)
    assert err0 <= tol0 * rms0, (err0, rms0)
    if dtype == S.BF16:
        assert_delta_within_bound(y0.cpu().numpy(), yd, x, osc, p, ids)
    assert np.all(y0.cpu().numpy()[ids < 0] == 0)


@pytest.mark.parametrize("mode", ["matrix", "group"])
def test_apply_parity_large_batch(mode):
    # T * d_in above the single-block reorder threshold: separate prep kernel,
    # users with 0, 1, 31, 32, 33 and 150 tokens (item splits at 32)
    ids = _ids_mixed(T_users=(150, 0, 1, 31, 32, 33, 5), extra_none=7, seed=11)
    T, U = len(ids), 7
    d_out, d_in = 136, 1024
    w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=1350)
    p = B.params(mode, 128)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(U))
    ids_dev = torch.from_numpy(ids).to(DEV)
    y = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, check=True)
    wb = S.host_wbase(w, 0)
    words, osc = oracle_bank(w, 0, wb, p, range(U))
    yr, yb, yd = O.apply(S.host_x(w, 0), wb, words, osc, p.mode, ids, g=128)
    err, rms = max_err_vs_rms(y.cpu().numpy(), yr)
    assert err <= TOL_BF16 * rms, (err, rms)
    y0 = B.apply(x_dev, torch.zeros_like(wb_dev), signs, scales, p, ids_dev, check=True)
    err0, rms0 = max_err_vs_rms(y0.cpu().numpy(), yd)
    assert err0 <= tol_delta(mode) * rms0, (err0, rms0)
    assert_delta_within_bound(y0.cpu().numpy(), yd, S.host_x(w, 0), osc, p, ids)


# MATRIX / ROW / COL batches take one of two delta kernels: the persistent one for
# batches of few tokens per user (fewer than 16 on average) on rows whose groups of
# 512-column units are at least 7 wide, the per-tile one otherwise.  Each route and mode:
# (name, d_in, tokens per user (users 0..), unassigned tokens)
ROUTE_CASES = [
    ("persistent", 4096, (20, 1, 3, 0, 2, 5, 1, 4), 3),           # 36 tokens, 8 users
    ("persistent_two_groups", 7168, (20, 1, 3, 0, 2, 5, 1, 4), 3),  # 14 units: 2 groups of 7
    ("per_tile", 4096, (40, 9), 2),                                  # 49 tokens, 2 users
]


@pytest.mark.parametrize("mode", ["matrix", "row", "col"])
@pytest.mark.parametrize("route", ROUTE_CASES, ids=lambda c: c[0])
def test_apply_parity_delta_routes(route, mode):
    _, d_in, users, extra = route
    ids = _ids_mixed(T_users=users, extra_none=extra, seed=21)
    T, U = len(ids), len(users)
    d_out = 200  # a ragged 128-row chunk
    w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=1370 + d_in // 512)
    p = B.params(mode, 128, 0.0, B.BD_F32 if mode == "matrix" else B.BD_F16)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(U))
    ids_dev = torch.from_numpy(ids).to(DEV)
    y = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, check=True)
    wb = S.host_wbase(w, 0)
    words, osc = oracle_bank(w, 0, wb, p, range(U))
    yr, yb, yd = O.apply(S.host_x(w, 0), wb, words, osc, p.mode, ids, g=128, sdtype=o_sdtype(p))
    err, rms = max_err_vs_rms(y.cpu().numpy(), yr)
    assert err <= TOL_BF16 * rms, (err, rms)
    y0 = B.apply(x_dev, torch.zeros_like(wb_dev), signs, scales, p, ids_dev, check=True)
    err0, rms0 = max_err_vs_rms(y0.cpu().numpy(), yd)
    assert err0 <= tol_delta(mode) * rms0, (err0, rms0)
    assert_delta_within_bound(y0.cpu().numpy(), yd, S.host_x(w, 0), osc, p, ids)
    assert np.all(y0.cpu().numpy()[ids < 0] == 0)
    y1 = B.apply(x_dev, torch.zeros_like(wb_dev), signs, scales, p, ids_dev, check=True)
    assert torch.equal(y0, y1)  # repeat calls agree bit for bit


@pytest.mark.parametrize("mode", ["matrix", "col"])
def test_apply_parity_single_wave_grouping(mode):
    # T <= 64 takes the one-wave grouping kernel; a 40-token user spans two items
    ids = _ids_mixed(T_users=(40, 15, 0, 5), extra_none=3, seed=13)
    T, U = len(ids), 4
    d_out, d_in = 100, 1536
    w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=1360)
    p = B.params(mode, 128, 0.0, B.BD_F16 if mode == "col" else B.BD_F32)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(U))
    ids_dev = torch.from_numpy(ids).to(DEV)
    y = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, check=True)
    wb = S.host_wbase(w, 0)
    words, osc = oracle_bank(w, 0, wb, p, range(U))
    yr, yb, yd = O.apply(S.host_x(w, 0), wb, words, osc, p.mode, ids, g=128, sdtype=o_sdtype(p))
    err, rms = max_err_vs_rms(y.cpu().numpy(), yr)
    assert err <= TOL_BF16 * rms, (err, rms)
    y0 = B.apply(x_dev, torch.zeros_like(wb_dev), signs, scales, p, ids_dev, check=True)
    err0, rms0 = max_err_vs_rms(y0.cpu().numpy(), yd)
    assert err0 <= tol_delta(mode) * rms0, (err0, rms0)
    assert_delta_within_bound(y0.cpu().numpy(), yd, S.host_x(w, 0), osc, p, ids)


def test_apply_out_of_range_user_gets_base_and_status():
    w = custom(64, 512, S.BF16, n_users=2, T=4, cid=1400)
    p = B.params("matrix")
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(2))
    ids = torch.tensor([0, 7, -1, 1], dtype=torch.int32, device=DEV)
    ws = B.workspace(B.bd_apply_workspace_bytes(p, 4, 2, 64, 512, B.BD_BF16, B.BD_F32), DEV)
    y = B.apply(x_dev, wb_dev, signs, scales, p, ids, ws=ws)
    assert B.bd_device_status(ws) == B.BD_ERR_USER_ID
    base = B.apply(x_dev, wb_dev, signs, scales, p, torch.full_like(ids, -1), ws=ws)
    assert B.bd_device_status(ws) == B.BD_OK
    assert torch.equal(y[1], base[1]) and torch.equal(y[2], base[2])
    assert not torch.equal(y[0], base[0])


@pytest.mark.parametrize("mode", ["matrix", "group"])
def test_apply_without_valid_users_is_the_base_product(mode):
    """A many-token batch whose ids are all -1 has no tile of delta products: y is the
    base product and the status word stays clear."""
    w = custom(72, 1024, S.BF16, n_users=2, T=40, cid=1420)
    p = B.params(mode)
    wb_dev = S.dev_wbase(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(2))
    ids = np.full(40, -1, np.int32)
    y = B.apply(S.dev_x(w, 0), wb_dev, signs, scales, p, torch.from_numpy(ids).to(DEV), check=True)
    wb = S.host_wbase(w, 0)
    words, osc = oracle_bank(w, 0, wb, p, range(2))
    _, yb, yd = O.apply(S.host_x(w, 0), wb, words, osc, p.mode, ids)
    assert np.all(yd == 0)
    err, rms = max_err_vs_rms(y.cpu().numpy(), yb)
    assert err <= 1e-5 * rms, (err, rms)


@pytest.mark.parametrize("g,T,sd", [(32, 40, B.BD_F32), (64, 9, B.BD_F16), (16, 100, B.BD_F32)])
def test_apply_small_groups(g, T, sd):
    """bf16 GROUP scales with groups under 128 columns (the plain per-row kernel): y and
    the delta term against the oracle; the delta term is fp32 sums of exact bf16
    products, so it is held to 1e-5 rms.  Also under the INT8 base."""
    U = 4
    ids = np.random.default_rng(g + T).integers(-1, U, T).astype(np.int32)
    w = custom(136, 1152, S.BF16, n_users=U, T=T, b=5e-3, cid=1440 + g)
    p = B.params("group", g, 0.0, sd)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(U))
    ids_dev = torch.from_numpy(ids).to(DEV)
    y = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, check=True)
    y0 = B.apply(x_dev, torch.zeros_like(wb_dev), signs, scales, p, ids_dev, check=True)
    wb = S.host_wbase(w, 0)
    words, osc = oracle_bank(w, 0, wb, p, range(U))
    assert np.array_equal(to_np(signs), words)
    x = S.host_x(w, 0)
    yr, _, yd = O.apply(x, wb, words, osc, p.mode, ids, g=g, sdtype=o_sdtype(p))
    err, rms = max_err_vs_rms(y.cpu().numpy(), yr)
    assert err <= TOL_BF16 * rms, (err, rms)
    err0, rms0 = max_err_vs_rms(y0.cpu().numpy(), yd)
    assert err0 <= 1e-5 * rms0, (err0, rms0)
    q, qs = B.quantize_base(wb_dev)
    y8 = B.apply_q8(x_dev, q, qs, signs, scales, p, ids_dev, check=True)
    oq, os_ = O.quantize_rows(wb, dtype=O.BF16)
    y8r, _, _ = O.apply_q8(x, oq, os_, words, osc, p.mode, ids, g=g, sdtype=o_sdtype(p))
    err8, rms8 = max_err_vs_rms(y8.cpu().numpy(), y8r)
    assert err8 <= TOL_BF16 * rms8, (err8, rms8)


def test_apply_empty_batch_is_a_noop():
    w = custom(64, 512, S.BF16, n_users=2, T=0, cid=1401)
    p = B.params("matrix")
    wb_dev = S.dev_wbase(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(2))
    x = torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)
    y = B.apply(x, wb_dev, signs, scales, p, torch.empty(0, dtype=torch.int32, device=DEV), check=True)
    assert y.shape == (0, 64)


def test_apply_is_deterministic():
    ids = _ids_mixed(seed=9)
    w = custom(192, 1024, S.BF16, n_users=5, T=len(ids), cid=1402)
    p = B.params("group", 128)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(5))
    ids_dev = torch.from_numpy(ids).to(DEV)
    y1 = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev)
    y2 = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev)
    assert torch.equal(y1, y2)
    s2, c2 = gpu_bank(w, 0, wb_dev, p, range(5))
    assert torch.equal(signs, s2) and torch.equal(scales, c2)


@pytest.mark.parametrize("mode,sd", [("group", B.BD_F32), ("row", B.BD_F16), ("col", B.BD_F16), ("matrix", B.BD_F32)])
def test_reconstruct_parity(mode, sd):
    w = custom(96, 576, S.BF16, cid=1500)
    p = B.params(mode, 64, 0.0, sd)
    wb_dev = S.dev_wbase(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, [0])
    rec = B.reconstruct(signs[0], scales[0], p, 96, 576)
    ref = O.reconstruct(to_np(signs[0]), to_np(scales[0]), p.mode, 96, 576, g=64, sdtype=o_sdtype(p))
    assert np.array_equal(rec.cpu().numpy().astype(np.float64), ref)  # +-scale is exact in fp32
    merged = B.reconstruct(signs[0], scales[0], p, 96, 576, w_base=wb_dev, out_dtype=torch.bfloat16)
    refm = O.reconstruct(to_np(signs[0]), to_np(scales[0]), p.mode, 96, 576, g=64, sdtype=o_sdtype(p),
                         wb=to_np(wb_dev), wdtype=O.BF16)
    got = merged.float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - refm) <= 2.0 ** -8 * np.abs(refm) + 1e-30)
