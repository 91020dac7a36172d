"""The row-restricted oracle banks the full-size workload checks use equal the rows of
the oracle's whole-matrix compression, bit for bit, in every scale mode, with and
without clipping (CPU only)."""
import numpy as np
import pytest

from gpu_util import custom, oracle_bank, oracle_rows_bank
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S


@pytest.mark.parametrize("clip_k", [0.0, 3.0])
@pytest.mark.parametrize("mode", ["matrix", "group", "row", "col"])
def test_rows_bank_equals_rows_of_whole_compression(mode, clip_k):
    d_out, d_in = 48, 640
    w = custom(d_out, d_in, S.BF16, n_users=3, T=4, b=5e-3, outlier_p=2e-3, cid=2700)
    p = B.params(mode, 128, clip_k, B.BD_F16 if mode in ("row", "col") else B.BD_F32)
    rows = [0, 5, 17, 30, 47]
    words, scs = oracle_bank(w, 0, S.host_wbase(w, 0), p, [2, 0])
    rw, rs = oracle_rows_bank(w, 0, p, [2, 0], rows)
    assert np.array_equal(rw, words[:, rows])
    if p.mode == B.BD_SCALE_GROUP:
        want = scs.reshape(2, d_out, -1)[:, rows].reshape(2, -1)
    elif p.mode == B.BD_SCALE_ROW:
        want = scs[:, rows]
    else:
        want = scs
    assert np.array_equal(rs, want)
