"""GPU parity of the decode paths (bf16, at most 16 tokens): the single-launch
kernel (MATRIX/ROW scales, d_in up to 5120) and the two-launch one (prepare +
apply; also COL scales and wider rows).  bd_apply against the CPU oracle on the
same seeded inputs, for the whole output and for the delta term alone, over
ragged shapes (d_in not a multiple of 128 or 512, d_out not a multiple of 16),
repeated users, invalid ids, a batch without any valid user, one token, unit
counts that do not divide evenly over the kernels' waves, the widest rows the
single-launch kernel stages and the first width past it."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (DEV, TOL_BF16, assert_delta_within_bound, custom, gpu_bank, max_err_vs_rms,
                      o_sdtype, oracle_bank,
                      rel_err_ok, scales_as_f64, to_np, tol_delta)
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

pytestmark = pytest.mark.gpu


def _shuffled(groups, n_invalid=0, seed=0):
    ids = []
    for u, n in groups:
        ids += [u] * n
    ids += [-1] * n_invalid
    rng = np.random.default_rng(seed)
    rng.shuffle(ids)
    return np.array(ids, dtype=np.int32)


CASES = [
    # (name, mode, scale dtype, d_out, d_in, ids, n_users, y dtype)
    ("mixed7", "matrix", B.BD_F32, 80, 576, np.array([2, 0, -1, 2, 1, 2, 0], np.int32), 3, torch.float32),
    ("16users", "matrix", B.BD_F32, 200, 1024, np.random.default_rng(1).permutation(16).astype(np.int32), 16, torch.bfloat16),
    ("row-repeat", "row", B.BD_F16, 130, 1088, _shuffled([(0, 5), (1, 3), (3, 8)], seed=2), 4, torch.float32),
    ("col-invalid", "col", B.BD_F16, 96, 576, _shuffled([(1, 2), (0, 4), (2, 1)], n_invalid=2, seed=3), 3, torch.float32),
    ("one-token", "matrix", B.BD_F32, 64, 512, np.array([1], np.int32), 2, torch.float32),
    ("odd-units", "matrix", B.BD_F32, 48, 2560, _shuffled([(u, 1) for u in range(12)], n_invalid=2, seed=4), 12, torch.float32),
    ("d_in-64", "row", B.BD_F32, 40, 64, np.array([0, 1, 1, 0, 2], np.int32), 3, torch.float32),
    ("nine-users", "col", B.BD_F32, 33, 1152, _shuffled([(u, 1 + u % 2) for u in range(9)], seed=5), 9, torch.bfloat16),
    ("widest-staged", "matrix", B.BD_F32, 48, 5120, np.random.default_rng(6).permutation(16).astype(np.int32), 16, torch.float32),
    ("past-staged", "row", B.BD_F16, 40, 5632, _shuffled([(0, 4), (2, 5), (1, 3)], n_invalid=1, seed=8), 3, torch.float32),
    ("nine-units", "row", B.BD_F16, 64, 4608, _shuffled([(u, 1) for u in range(14)], n_invalid=2, seed=9), 14, torch.bfloat16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_decode_parity(case):
    name, mode, sd, d_out, d_in, ids, U, ydt = case
    T = len(ids)
    w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=1700 + d_out + d_in)
    p = B.params(mode, 128, 0.0, sd)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(U))
    ids_dev = torch.from_numpy(ids).to(DEV)
    y = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, y_dtype=ydt, check=True)
    y0 = B.apply(x_dev, torch.zeros_like(wb_dev), signs, scales, p, ids_dev, check=True)

    wb = S.host_wbase(w, 0)
    words, osc = oracle_bank(w, 0, wb, p, range(U))
    assert np.array_equal(to_np(signs), words)
    assert rel_err_ok(scales_as_f64(to_np(scales), p), scales_as_f64(osc, p))
    yr, yb, yd = O.apply(S.host_x(w, 0), wb, words, osc, p.mode, ids, g=128, sdtype=o_sdtype(p))
    err, rms = max_err_vs_rms(y.float().cpu().numpy(), yr)
    assert err <= TOL_BF16 * rms, (name, err, rms)
    got0 = y0.cpu().numpy()
    err0, rms0 = max_err_vs_rms(got0, yd)
    assert err0 <= tol_delta(mode) * rms0, (name, "delta only", err0, rms0)
    assert_delta_within_bound(got0, yd, S.host_x(w, 0), osc, p, ids, name)
    assert np.all(got0[ids < 0] == 0)  # tokens without a valid user get no delta at all


def test_decode_without_valid_users_is_the_base_product():
    ids = np.array([-1, -1, -1], np.int32)
    w = custom(50, 640, S.BF16, n_users=2, T=3, b=5e-3, cid=1790)
    p = B.params("matrix")
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(2))
    y = B.apply(x_dev, wb_dev, signs, scales, p, torch.from_numpy(ids).to(DEV), check=True)
    wb = S.host_wbase(w, 0)
    words, osc = oracle_bank(w, 0, wb, p, range(2))
    yr, yb, yd = O.apply(S.host_x(w, 0), wb, words, osc, p.mode, ids)
    assert np.all(yd == 0)
    err, rms = max_err_vs_rms(y.cpu().numpy(), yb)
    assert err <= TOL_BF16 * rms, (err, rms)


def test_decode_matches_the_phased_path_and_is_deterministic():
    """The one-pass kernel and the three-phase calls (prepare, base GEMM, delta)
    implement the same product; both are checked against the oracle elsewhere,
    here they must agree with each other within the bf16 tolerance, and the
    one-pass result must repeat bit for bit."""
    ids = _shuffled([(0, 3), (1, 1), (2, 6), (4, 2)], n_invalid=1, seed=7)
    T, U, d_out, d_in = len(ids), 5, 144, 1536
    w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=1795)
    p = B.params("row", 128, 0.0, B.BD_F16)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(U))
    ids_dev = torch.from_numpy(ids).to(DEV)
    y1 = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, check=True)
    y2 = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev)
    assert torch.equal(y1, y2)
    batch = B.workspace(B.bd_batch_workspace_bytes(T, U, d_in, B.BD_BF16), DEV)
    assert B.bd_batch_prepare(x_dev, ids_dev, U, batch) == B.BD_OK
    yp = torch.empty((T, d_out), dtype=torch.float32, device=DEV)
    assert B.bd_base_gemm(x_dev, wb_dev, yp) == B.BD_OK
    assert B.bd_delta_apply(batch, x_dev, U, signs, scales, p, yp) == B.BD_OK
    torch.cuda.synchronize()
    err, rms = max_err_vs_rms(y1.cpu().numpy(), yp.cpu().numpy().astype(np.float64))
    assert err <= TOL_BF16 * rms, (err, rms)


def test_decode_under_graph_capture_replays_match_eager():
    """bd_apply on the one-pass path captured in a HIP graph: three replays, with
    eager applies on other inputs and synchronisations between them, each equal
    bit for bit to the eager result."""
    ids = np.random.default_rng(3).permutation(16).astype(np.int32)
    T, U, d_out, d_in = 16, 16, 272, 1024
    w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=1797)
    p = B.params("matrix")
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(U))
    ids_dev = torch.from_numpy(ids).to(DEV)
    ws = B.workspace(B.bd_apply_workspace_bytes(p, T, U, d_out, d_in, B.BD_BF16, B.BD_F32), DEV)
    y_eager = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, ws=ws, check=True).clone()
    y = torch.empty_like(y_eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, y=y, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, y=y, ws=ws)
    x_other = torch.flip(x_dev, dims=[0]).contiguous()
    ws_other = B.workspace(ws.numel(), DEV)
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {rep} differs from the eager result"
        B.apply(x_other, wb_dev, signs, scales, p, ids_dev, ws=ws_other)  # eager work between
        torch.cuda.synchronize()


@pytest.mark.parametrize("mode,sd", [("matrix", B.BD_F32), ("row", B.BD_F16)])
def test_single_launch_matches_two_launch_path(mode, sd):
    """The single-launch kernel (bd_apply) and the two-launch decode calls
    (bd_decode_prepare + bd_decode_apply) compute the same product with different
    partitions of the sums: both within the bf16 tolerance of each other, and the
    single-launch result repeats bit for bit."""
    ids = _shuffled([(0, 2), (3, 5), (1, 1), (5, 4), (2, 3)], n_invalid=1, seed=11)
    T, U, d_out, d_in = len(ids), 6, 208, 4096
    w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=1799)
    p = B.params(mode, 128, 0.0, sd)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(U))
    ids_dev = torch.from_numpy(ids).to(DEV)
    y1 = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, check=True)
    y2 = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    ws = B.workspace(B.bd_apply_workspace_bytes(p, T, U, d_out, d_in, B.BD_BF16, B.BD_F32), DEV)
    assert B.bd_decode_prepare(x_dev, ids_dev, U, scales, p, ws) == B.BD_OK
    yt = torch.empty((T, d_out), dtype=torch.float32, device=DEV)
    assert B.bd_decode_apply(x_dev, wb_dev, signs, scales, p, U, yt, ws) == B.BD_OK
    torch.cuda.synchronize()
    assert B.bd_device_status(ws) == B.BD_OK
    err, rms = max_err_vs_rms(y1.cpu().numpy(), yt.cpu().numpy().astype(np.float64))
    assert err <= TOL_BF16 * rms, (err, rms)
    # and both against the oracle's delta term alone (W_base = 0)
    z = torch.zeros_like(wb_dev)
    d1 = B.apply(x_dev, z, signs, scales, p, ids_dev, check=True)
    wb = S.host_wbase(w, 0)
    words, osc = oracle_bank(w, 0, wb, p, range(U))
    _, _, yd = O.apply(S.host_x(w, 0), wb, words, osc, p.mode, ids, g=128, sdtype=o_sdtype(p))
    err, rms = max_err_vs_rms(d1.cpu().numpy(), yd)
    assert err <= tol_delta(mode) * rms, ("delta only", err, rms)
    assert_delta_within_bound(d1.cpu().numpy(), yd, S.host_x(w, 0), osc, p, ids)
