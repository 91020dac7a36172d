"""The dense merge path for a hot user: W_u = W_base + scale (.) sign materialised
once in bf16 (bd_reconstruct with the base), then one plain GEMM over that user's
tokens (bd_base_gemm) ([P2] "Systems Mechanics": the merged per-user weight as the
alternative to the fused per-request delta).  Checked against the oracle's apply of
the same tokens, at token counts that take the streaming GEMM (16 < T <= 64) and the
tiled GEMM (T > 64), in every scale mode.

The merged weight is rounded once to bf16 (8 significant bits, round to nearest), so
each output may differ from the exact X W_u^T by at most 2^-8 of every W_u element it
sums (relative to the rounded value, up to a factor 1 + 2^-8):
    |y - y_exact| <= 1.01 * 2^-8 * (|X| |W_u|^T) + (fp32 accumulation, 2^-16 of it),
which the test checks element by element, beside the bf16 bar of the apply
(max|err| <= 2e-2 rms), and, tighter, Hoeffding's bound for the independent rounding
errors e of W_u (|e| <= half an ulp h of each element): |y - y_exact| <= 8 sqrt(X^2
(h^2)^T) + the same accumulation term (exceeded with probability under 3e-14 per
element).  That error is all in the delta term the merge path carries: it scales with
|W_u| (about |W_base|), not with the delta, so against the delta term alone it grows
as rms(W_base) / mean|delta|: measured max|err| / rms of the delta term about 3 % at
the tests' Laplace scale b = 5e-3 and 10 % at the workloads' b = 5e-4 (printed).
The fused path keeps the delta term within 5e-3 of its rms at any b; the merged path
trades that for one dense GEMM per hot user."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (DEV, TOL_BF16, bf16_to_f64, custom, gpu_bank, max_err_vs_rms, o_sdtype,
                      oracle_bank, to_np)
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

pytestmark = pytest.mark.gpu

CASES = [
    # (mode, scale dtype, d_out, d_in, tokens, Laplace scale of the deltas)
    ("matrix", B.BD_F32, 272, 1024, 40, 5e-3),
    ("group", B.BD_F32, 200, 1152, 96, 5e-3),
    ("row", B.BD_F16, 130, 1088, 80, 5e-3),
    ("col", B.BD_F16, 96, 576, 130, 5e-3),
    ("matrix", B.BD_F32, 256, 2048, 100, 5e-4),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[2]}x{c[3]}-T{c[4]}-b{c[5]}")
def test_merge_path_matches_oracle(case):
    mode, sd, d_out, d_in, T, b = case
    w = custom(d_out, d_in, S.BF16, n_users=2, T=T, b=b, cid=1900 + d_out)
    p = B.params(mode, 128, 0.0, sd)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, [0, 1])
    # user 1 is the hot user: every token is its
    wu = B.reconstruct(signs[1], scales[1], p, d_out, d_in, w_base=wb_dev, out_dtype=torch.bfloat16)
    y = torch.empty((T, d_out), dtype=torch.float32, device=DEV)
    assert B.bd_base_gemm(x_dev, wu, y) == B.BD_OK
    torch.cuda.synchronize()

    wb = S.host_wbase(w, 0)
    x = S.host_x(w, 0)
    words, osc = oracle_bank(w, 0, wb, p, [0, 1])
    assert np.array_equal(to_np(signs), words)
    ids = np.full(T, 1, dtype=np.int32)
    yr, ybr, ydr = O.apply(x, wb, words, osc, p.mode, ids, g=128, sdtype=o_sdtype(p))
    got = y.cpu().numpy().astype(np.float64)
    err, rms = max_err_vs_rms(got, yr)
    assert err <= TOL_BF16 * rms, (err, rms)
    wu_np = wu.float().cpu().numpy().astype(np.float64)
    xf = bf16_to_f64(x)  # (x holds bf16 bit patterns)
    mag = np.abs(xf) @ np.abs(wu_np).T
    bound = (1.01 * 2.0 ** -8 + 2.0 ** -16) * mag
    assert np.all(np.abs(got - yr) <= bound + 1e-30), float(np.max(np.abs(got - yr) - bound))
    m, e = np.frexp(np.abs(wu_np))  # |w| = m 2^e, m in [0.5, 1): half an ulp is 2^(e - 9)
    h = np.where(wu_np != 0, 1.01 * np.ldexp(1.0, e - 9), 0.0)  # (1.01: the fp32 sum before)
    hoeff = 8.0 * np.sqrt((xf ** 2) @ (h ** 2).T) + 2.0 ** -16 * mag
    assert np.all(np.abs(got - yr) <= hoeff + 1e-30), float(np.max(np.abs(got - yr) - hoeff))
    derr, drms = max_err_vs_rms(got - ybr, ydr)  # the delta term as the merge path carries it
    print(f"merge {mode} b={b}: delta-term max|err| / rms = {derr / drms:.4f}")


def test_merged_equals_fused_for_a_zero_delta():
    """With every scale zero the merged weight is W_base exactly, so the merge path and
    the base product agree bit for bit (same GEMM on the same bytes)."""
    d_out, d_in, T = 144, 1024, 72
    w = custom(d_out, d_in, S.BF16, n_users=1, T=T, cid=1990)
    p = B.params("matrix")
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    signs, _ = gpu_bank(w, 0, wb_dev, p, [0])
    zero = torch.zeros((1, 1), dtype=torch.float32, device=DEV)
    wu = B.reconstruct(signs[0], zero[0], p, d_out, d_in, w_base=wb_dev, out_dtype=torch.bfloat16)
    assert torch.equal(wu, wb_dev)
    y1 = torch.empty((T, d_out), dtype=torch.float32, device=DEV)
    y2 = torch.empty_like(y1)
    assert B.bd_base_gemm(x_dev, wu, y1) == B.BD_OK
    assert B.bd_base_gemm(x_dev, wb_dev, y2) == B.BD_OK
    assert torch.equal(y1, y2)
