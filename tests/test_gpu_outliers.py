"""Activations with outlier channels: a few input columns of X far larger than the
rest, as in the hidden states of large language models.  The delta products take the
tokens in blocks of 32 columns under one power-of-two scale per block, and every value
keeps an absolute error within 2^-10 of its block's largest |x|, so a block that holds
an outlier column carries its other values on a coarser grid.  These cases check the
delta term alone (zero base weight) element by element against that bound
(delta_error_bound) and against max|err| <= 2e-2 rms: where outlier blocks dominate,
the expected max|err| / rms is about 1e-2 whatever the outliers' size (the error and
the rms both grow with it), against about 4e-3 on Gaussian tokens.  Many-token and
decode paths, each scale mode.  The outlier columns are the ordinary seeded values
times a power of two, so X is the same bf16 bits on both sides."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (DEV, TOL_BF16, assert_delta_within_bound, custom, gpu_bank, max_err_vs_rms,
                      o_sdtype, oracle_bank, tol_delta)
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

pytestmark = pytest.mark.gpu


def bf16_times_pow2(bits: np.ndarray, cols, k: int) -> np.ndarray:
    """bf16 bit patterns with the given columns multiplied by 2^k (exact)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32).copy()
    f[:, cols] *= np.float32(2.0 ** k)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


CASES = [
    # (mode, scale dtype, d_out, d_in, tokens, share of outlier columns, 2^k)
    ("matrix", B.BD_F32, 136, 2048, 40, 0.01, 5),
    ("row", B.BD_F16, 130, 4096, 40, 0.01, 5),
    ("group", B.BD_F32, 96, 2048, 70, 0.005, 7),
    ("col", B.BD_F16, 100, 2048, 40, 0.01, 5),
    ("matrix", B.BD_F32, 80, 4096, 9, 0.01, 5),
    ("row", B.BD_F16, 64, 5120, 7, 0.002, 8),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[3]}-T{c[4]}-{c[5]}x2^{c[6]}")
def test_delta_term_with_outlier_channels(case):
    mode, sd, d_out, d_in, T, share, k = case
    U = 4
    rng = np.random.default_rng(d_in + T)
    ids = rng.integers(0, U, size=T).astype(np.int32)
    w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=2600 + d_out + T)
    p = B.params(mode, 128, 0.0, sd)
    cols = np.sort(rng.choice(d_in, size=max(1, int(share * d_in)), replace=False))
    x_np = bf16_times_pow2(S.host_x(w, 0), cols, k)
    x_dev = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(DEV)
    wb_dev = S.dev_wbase(w, 0)
    signs, scales = gpu_bank(w, 0, wb_dev, p, range(U))
    ids_dev = torch.from_numpy(ids).to(DEV)
    y0 = B.apply(x_dev, torch.zeros_like(wb_dev), signs, scales, p, ids_dev, check=True)
    y = B.apply(x_dev, wb_dev, signs, scales, p, ids_dev, check=True)
    wb = S.host_wbase(w, 0)
    words, osc = oracle_bank(w, 0, wb, p, range(U))
    yr, _, yd = O.apply(x_np, wb, words, osc, p.mode, ids, g=128, sdtype=o_sdtype(p))
    err0, rms0 = max_err_vs_rms(y0.cpu().numpy(), yd)
    print(f"outliers {mode} d_in={d_in} T={T}: delta-only max|err|/rms = {err0 / rms0:.3e}")
    assert_delta_within_bound(y0.cpu().numpy(), yd, x_np, osc, p, ids)
    assert err0 <= TOL_BF16 * rms0, (err0, rms0)
    err, rms = max_err_vs_rms(y.cpu().numpy(), yr)
    assert err <= tol_delta(mode) * rms, (err, rms)
