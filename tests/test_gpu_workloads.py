"""GPU parity at the five workloads' full sizes, in the launch configuration the
benchmark uses (bd_apply on device-generated inputs), against the CPU oracle:
- compression: for sampled (user, matrix) pairs the oracle compresses the whole
  matrix from host-generated inputs; the packed signs must match bit for bit and the
  scales within 1e-6 relative;
- apply: every token of the batch on sampled output rows (the first, the last and a
  seeded sample), with the oracle's banks of every user in the batch restricted to
  those rows (built from the oracle's own steps; the clip bounds and the MATRIX and
  COL scales still read each user's whole matrix); y must match within
  max|err| <= tol * rms (1e-4 fp32, 2e-2 bf16), and the delta term alone (the same
  banks on a zero base weight) within 5e-3 rms (1e-2 for COL scales)."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (DEV, TOL_BF16, TOL_F32, assert_delta_within_bound, max_err_vs_rms,
                      oracle_rows_bank, rel_err_ok,
                      scales_as_f64, to_np, tol_delta)
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

pytestmark = pytest.mark.gpu


def params_of(w, mat):
    return B.params(mat.mode, w.group_size, w.clip_k, B.BD_F16 if mat.scale_dtype == S.S_F16 else B.BD_F32)


def o_sd(p):
    return O.F16 if p.scale_dtype == B.BD_F16 else O.F32


def compress_all(w, m, wb_dev, p):
    mat = w.matrices[m]
    n_sc = B.bd_scales_count(p, mat.d_out, mat.d_in)
    signs = torch.empty((w.n_users, mat.d_out, mat.d_in // 64), dtype=torch.int64, device=DEV)
    scales = torch.empty((w.n_users, n_sc), dtype=B.scales_dtype(p), device=DEV)
    ws = B.workspace(B.bd_compress_workspace_bytes(p, mat.d_out, mat.d_in), DEV)
    wf = torch.empty_like(wb_dev)
    for u in range(w.n_users):
        S.dev_wfine(w, m, u, wb_dev, out=wf)
        B.compress(wf, wb_dev, p, signs_out=signs[u], scales_out=scales[u], ws=ws)
    assert B.bd_device_status(ws) == B.BD_OK
    return signs, scales


def oracle_user(w, m, u, wb_np, p):
    wf = S.host_wfine(w, m, u, wbase=wb_np)
    words, sc, _, bad = O.compress(wf, wb_np, p.mode, g=p.group_size, clip_k=p.clip_k,
                                   sdtype=o_sd(p), dtype=w.dtype)
    assert bad == 0
    return words, sc


def rows_of_scales(sc, p, mat, rows):
    if p.mode == B.BD_SCALE_GROUP:
        return sc.reshape(mat.d_out, -1)[rows].reshape(-1)
    if p.mode == B.BD_SCALE_ROW:
        return sc[rows]
    return sc  # MATRIX (1 value) and COL (d_in values) do not depend on the row


def check_matrix(w, m, ids, check_users, rows, wb_dev=None, x_dev=None, banks=None):
    """Compress every user on the GPU, apply the whole batch, compare with the oracle:
    whole-matrix compression of `check_users`, and every token on the output rows `rows`."""
    mat = w.matrices[m]
    p = params_of(w, mat)
    if wb_dev is None:
        wb_dev = S.dev_wbase(w, m)
    if x_dev is None:
        x_dev = S.dev_x(w, mat.xgroup)
    signs, scales = banks if banks is not None else compress_all(w, m, wb_dev, p)
    ids_dev = torch.from_numpy(ids).to(DEV)
    y = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, check=True)
    y0 = B.apply(x_dev, torch.zeros_like(wb_dev), signs, scales, p, ids_dev, check=True)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy()[:, rows]
    got0 = y0.cpu().numpy()[:, rows]
    del y, y0

    # compress parity on the sampled users (whole matrices)
    wb_np = S.host_wbase(w, m)
    for u in check_users:
        words, sc = oracle_user(w, m, u, wb_np, p)
        assert np.array_equal(to_np(signs[u]), words), f"signs differ: user {u} matrix {mat.name}"
        assert rel_err_ok(scales_as_f64(to_np(scales[u]), p), scales_as_f64(sc, p)), \
            f"scales differ: user {u} matrix {mat.name}"
    del wb_np
    # apply parity: every token on the sampled rows, banks of every user in the batch
    users = sorted(set(int(u) for u in ids if u >= 0))
    remap = np.full(w.n_users, -1, dtype=np.int32)
    remap[users] = np.arange(len(users), dtype=np.int32)
    sub_ids = np.where(ids >= 0, remap[np.maximum(ids, 0)], -1).astype(np.int32)
    if users:
        words_bank, sc_bank = oracle_rows_bank(w, m, p, users, rows)
    else:
        words_bank = np.zeros((1, len(rows), mat.d_in // 64), dtype=np.uint64)
        sc_bank = np.zeros((1, 1), dtype=np.float32)
    x_np = S.host_x(w, mat.xgroup)
    yr, yb, yd = O.apply(x_np, S.host_wbase(w, m, rows), words_bank, sc_bank,
                         p.mode, sub_ids, g=p.group_size, sdtype=o_sd(p))
    tol = TOL_F32 if w.dtype == S.F32 else TOL_BF16
    err, rms = max_err_vs_rms(got, yr)
    assert err <= tol * rms, (mat.name, err, rms)
    if np.any(yd != 0):
        tol0 = TOL_F32 if w.dtype == S.F32 else tol_delta(p.mode)
        err0, rms0 = max_err_vs_rms(got0, yd)
        print(f"{mat.name}: {len(users)} users, {len(ids)} tokens x {len(rows)} rows, "
              f"delta-only max|err|/rms = {err0 / rms0:.3e}")
        assert err0 <= tol0 * rms0, (mat.name, "delta only", err0, rms0)
        if w.dtype == S.BF16:
            assert_delta_within_bound(got0, yd, x_np, sc_bank, p, sub_ids, mat.name)
    return signs, scales


def pick_tokens(ids, k, seed):
    rng = np.random.default_rng(seed)
    return sorted(rng.choice(len(ids), size=min(k, len(ids)), replace=False).tolist())


def pick_rows(d_out, k, seed):
    rng = np.random.default_rng(seed)
    r = set(rng.choice(d_out, size=min(k, d_out), replace=False).tolist())
    r |= {0, d_out - 1}
    return sorted(r)


@pytest.mark.timeout(300)
def test_workload1_tiny_fp32_full():
    w = S.workload(1)
    ids = S.user_ids(w)
    mat = w.matrices[0]
    check_matrix(w, 0, ids, [0], list(range(mat.d_out)))


@pytest.mark.timeout(600)
def test_workload2_q_proj_16_users():
    w = S.workload(2)
    ids = S.user_ids(w)
    check_matrix(w, 0, ids, [0, 7, 15], pick_rows(4096, 192, 2))


@pytest.mark.timeout(900)
def test_workload3_mlp_clipped_group_scales():
    w = S.workload(3)
    ids = S.user_ids(w)
    user = int(ids[pick_tokens(ids, 1, 3)[0]])
    for m in range(3):
        check_matrix(w, m, ids, [user], pick_rows(w.matrices[m].d_out, 96, 30 + m))
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_workload4_qwen_mlp_per_axis_mixed_batch():
    w = S.workload(4)
    ids = S.user_ids(w)
    # the user of a prefill chunk and the user of a decode token
    users = sorted({int(ids[5]), int(ids[8 * 128 + 3])})
    for m in range(3):
        check_matrix(w, m, ids, users, pick_rows(w.matrices[m].d_out, 64, 40 + m))
        torch.cuda.empty_cache()


@pytest.mark.timeout(1200)
def test_workload5_llama8b_stack_128_users():
    """All 224 matrices' banks resident (about 112 GB), one decode step of 512
    tokens through every matrix; checks on layer 0 q_proj and layer 31 down_proj
    (compress of a sampled token's user, apply of every token on sampled rows)."""
    w = S.workload(5)
    ids = S.user_ids(w)
    ids_dev = torch.from_numpy(ids).to(DEV)
    tokens = pick_tokens(ids, 1, 5)
    checked = {0: None, 223: None}
    banks, bases, xs = [], [], {}
    for m, mat in enumerate(w.matrices):
        p = params_of(w, mat)
        wb = S.dev_wbase(w, m)
        banks.append(compress_all(w, m, wb, p))
        bases.append(wb)
        if mat.xgroup not in xs:
            xs[mat.xgroup] = S.dev_x(w, mat.xgroup)
    # the decode step over the whole stack (each matrix on its own activations)
    ys = []
    for m, mat in enumerate(w.matrices):
        ys.append(B.apply(xs[mat.xgroup], bases[m], banks[m][0], banks[m][1], params_of(w, mat),
                          ids_dev, check=(m == len(w.matrices) - 1)))
    torch.cuda.synchronize()
    for m in checked:
        mat = w.matrices[m]
        rows = pick_rows(mat.d_out, 48, 50 + m)
        check_matrix(w, m, ids, [int(ids[tokens[0]])], rows, wb_dev=bases[m],
                     x_dev=xs[mat.xgroup], banks=banks[m])
        y_again = ys[m].cpu().numpy()
        y_ref = B.apply(xs[mat.xgroup], bases[m], banks[m][0], banks[m][1], params_of(w, mat),
                        ids_dev).cpu().numpy()
        assert np.array_equal(y_again, y_ref)  # the stack step equals the per-matrix check


def check_matrix_q8(w, m, ids, rows):
    """bd_apply_q8 over every user's GPU bank and the GPU-quantized base, every token on
    the rows `rows`, against the oracle's apply on its own INT8 rows and banks."""
    mat = w.matrices[m]
    p = params_of(w, mat)
    wb_dev = S.dev_wbase(w, m)
    x_dev = S.dev_x(w, mat.xgroup)
    signs, scales = compress_all(w, m, wb_dev, p)
    q, s = B.quantize_base(wb_dev)
    del wb_dev
    ids_dev = torch.from_numpy(ids).to(DEV)
    y = B.apply_q8(x_dev, q, s, signs, scales, p, ids_dev, check=True)
    y0 = B.apply_q8(x_dev, torch.zeros_like(q), s, signs, scales, p, ids_dev, check=True)
    torch.cuda.synchronize()
    got, got0 = y.cpu().numpy()[:, rows], y0.cpu().numpy()[:, rows]
    del y, y0, signs, scales, q
    users = sorted(set(int(u) for u in ids if u >= 0))
    remap = np.full(w.n_users, -1, dtype=np.int32)
    remap[users] = np.arange(len(users), dtype=np.int32)
    sub_ids = np.where(ids >= 0, remap[np.maximum(ids, 0)], -1).astype(np.int32)
    words_bank, sc_bank = oracle_rows_bank(w, m, p, users, rows)
    oq, os_ = O.quantize_rows(S.host_wbase(w, m, rows), dtype=O.BF16)
    x_np = S.host_x(w, mat.xgroup)
    yr, yb, yd = O.apply_q8(x_np, oq, os_, words_bank, sc_bank, p.mode, sub_ids, g=p.group_size,
                            sdtype=o_sd(p))
    err, rms = max_err_vs_rms(got, yr)
    assert err <= TOL_BF16 * rms, (mat.name, err, rms)
    err0, rms0 = max_err_vs_rms(got0, yd)
    print(f"INT8 base {mat.name}: {len(users)} users, {len(ids)} tokens x {len(rows)} rows, "
          f"max|err|/rms {err / rms:.3e}, delta-only {err0 / rms0:.3e}")
    assert err0 <= tol_delta(p.mode) * rms0, (mat.name, "delta only", err0, rms0)
    assert_delta_within_bound(got0, yd, x_np, sc_bank, p, sub_ids, mat.name)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid,m", [(3, 2), (4, 2), (5, 4)])
def test_int8_base_at_workload_shapes(cid, m):
    """The INT8 base under the 1-bit deltas at the workloads' sizes: the clipped MLP's
    down_proj (GROUP, 64 users, 256 tokens), Qwen's down_proj (COL, 1144 mixed tokens)
    and the Llama stack's layer 0 gate_proj (MATRIX, 512 Zipf tokens, 128 users)."""
    w = S.workload(cid)
    check_matrix_q8(w, m, S.user_ids(w), pick_rows(w.matrices[m].d_out, 48, 60 + cid))
    torch.cuda.empty_cache()
