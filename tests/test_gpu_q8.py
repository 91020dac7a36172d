"""The INT8 base: bd_quantize_base against the oracle's row quantizer (codes and
scales bit for bit: both divide in binary32, correctly rounded), and bd_apply_q8
against the oracle's apply on the same INT8 rows (bf16 bar, max|err| <= 2e-2 rms, and
the same rule on the delta term alone; the base term is exact products of bf16
tokens and integer codes, accumulated in fp32)."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, TOL_BF16, custom, gpu_bank, max_err_vs_rms, o_sdtype, oracle_bank, to_np
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


CASES = [
    # (mode, scale dtype, d_out, d_in, ids, n_users, y dtype)
    ("matrix", B.BD_F32, 200, 1024, np.random.default_rng(1).permutation(16).astype(np.int32), 16, torch.float32),
    ("row", B.BD_F16, 130, 1088, np.array([2, 0, -1, 2, 1, 2, 0], np.int32), 3, torch.bfloat16),
    ("matrix", B.BD_F32, 64, 4096, np.array([1, 1, 0], np.int32), 2, torch.float32),
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
    words, osc = oracle_bank(w, 0, wb, p, range(U))
    yr, yb, yd = O.apply_q8(S.host_x(w, 0), to_np(q), to_np(s), words, osc, p.mode, ids, g=128,
                            sdtype=o_sdtype(p))
    err, rms = max_err_vs_rms(y.float().cpu().numpy(), yr)
    assert err <= TOL_BF16 * rms, (err, rms)
    err0, rms0 = max_err_vs_rms(y0.cpu().numpy(), yd)
    assert err0 <= TOL_BF16 * rms0, (err0, rms0)
    assert np.all(y0.cpu().numpy()[ids < 0] == 0)


def test_apply_q8_rejects_what_it_does_not_serve():
    p = B.params("group", 128)
    x = torch.zeros((4, 512), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((64, 512), dtype=torch.int8, device=DEV)
    s = torch.ones(64, dtype=torch.float32, device=DEV)
    signs = torch.zeros((1, 64, 8), dtype=torch.int64, device=DEV)
    sc = torch.zeros((1, 64 * 4), dtype=torch.float32, device=DEV)
    ids = torch.zeros(4, dtype=torch.int32, device=DEV)
    y = torch.empty((4, 64), dtype=torch.float32, device=DEV)
    ws = B.workspace(1 << 20, DEV)
    assert B.bd_apply_q8(x, q, s, signs, sc, p, 1, ids, y, ws) == B.BD_ERR_UNSUPPORTED
