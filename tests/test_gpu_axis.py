"""GPU parity of the per-layer axis choice (bd_select_axis) with the oracle's
(oracle.select_axis, which sums both reconstruction errors element by element; the
library uses the per-unit closed form in one pass).  Bar: both errors within 1e-9
relative of the oracle's (binary64 sums in different orders) and the same axis, except
where the two errors lie within 1e-9 of each other, where either axis is valid.
Inputs from the seeded generator: bf16 and fp32 weights, with and without clipping
(injected outliers), ragged d_out; plus matrices built so that one axis reconstructs
them exactly."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import DEV, custom, to_np
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

pytestmark = pytest.mark.gpu

CASES = [
    # (dtype, clip_k, d_out, d_in, outlier probability)
    (S.BF16, 0.0, 256, 512, 0.0),
    (S.BF16, 3.0, 130, 1088, 0.002),
    (S.F32, 0.0, 33, 576, 0.0),
    (S.F32, 3.0, 300, 1024, 0.002),
    (S.BF16, 0.0, 1000, 2048, 0.0),
]


def _check(err, axis, want):
    er, ec, wax, _ = want
    assert abs(err[0] - er) <= 1e-9 * abs(er) and abs(err[1] - ec) <= 1e-9 * abs(ec), (err, want)
    if abs(er - ec) > 1e-9 * max(abs(er), abs(ec)):
        assert axis == wax, (axis, want)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-clip{c[1]}-{c[2]}x{c[3]}")
def test_select_axis_matches_oracle(case):
    dtype, clip, d_out, d_in, outp = case
    w = custom(d_out, d_in, dtype, b=1e-3, outlier_p=outp, cid=2100 + d_out)
    wb_dev = S.dev_wbase(w, 0)
    wf_dev = S.dev_wfine(w, 0, 0, wb_dev)
    errs, axis = B.select_axis(wf_dev, wb_dev, clip, check=True)
    torch.cuda.synchronize()
    wb = S.host_wbase(w, 0)
    wf = S.host_wfine(w, 0, 0, wbase=wb)
    want = O.select_axis(wf, wb, clip)
    _check(to_np(errs), int(to_np(axis)[0]), want)
    # repeated calls agree bit for bit (fixed summation order)
    errs2, axis2 = B.select_axis(wf_dev, wb_dev, clip)
    assert torch.equal(errs, errs2) and torch.equal(axis, axis2)


@pytest.mark.parametrize("by", ["rows", "cols"])
def test_select_axis_finds_the_exact_axis(by):
    rng = np.random.default_rng(3)
    d_out, d_in = 96, 256
    sgn = np.where(rng.random((d_out, d_in)) < 0.5, -1.0, 1.0)
    if by == "rows":
        mag = (2.0 ** -(np.arange(d_out) % 7 + 4))[:, None]
    else:
        mag = (2.0 ** -(np.arange(d_in) % 7 + 4))[None, :]
    d = (sgn * mag).astype(np.float32)
    errs, axis = B.select_axis(torch.from_numpy(d).to(DEV), None)
    torch.cuda.synchronize()
    e = to_np(errs)
    want = O.select_axis(d, None)
    _check(e, int(to_np(axis)[0]), want)
    exact = 0 if by == "rows" else 1
    assert abs(e[exact]) <= 1e-12 * abs(e[1 - exact])
    assert int(to_np(axis)[0]) == (B.BD_SCALE_ROW if by == "rows" else B.BD_SCALE_COL)
