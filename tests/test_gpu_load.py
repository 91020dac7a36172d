"""Loading packed deltas: one user's banks of one module (several matrices) packed
into one pinned host buffer in the module layout (tenant_serving_amd.banks), moved to
the device in one copy, and applied from views into that copy.  The bytes are the
bd_compress output, so the apply must reproduce, bit for bit, the apply from the
banks as bd_compress wrote them; the views are checked against the oracle's signs."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, custom, gpu_bank, oracle_bank, to_np
from tenant_serving_amd import banks
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

pytestmark = pytest.mark.gpu


def test_module_packed_load_applies_bit_for_bit():
    shapes = [(96, 576), (40, 576), (130, 576)]  # one module's matrices, one input width
    T, d_in = 8, 576
    p = B.params("row", 128, 0.0, B.BD_F16)
    mats = []
    for k, (d_out, _) in enumerate(shapes):
        w = custom(d_out, d_in, S.BF16, n_users=1, T=T, b=5e-3, cid=2200 + k)
        wb_dev = S.dev_wbase(w, 0)
        signs, scales = gpu_bank(w, 0, wb_dev, p, [0])
        mats.append((w, wb_dev, signs, scales))
    offs, total = banks.module_layout(shapes, [m[3].shape[1] for m in mats], 2)
    host = torch.zeros(total, dtype=torch.uint8, pin_memory=True)
    banks.pack_module(host, shapes, [m[2][0] for m in mats], [m[3][0] for m in mats])
    dev_buf = torch.empty(total, dtype=torch.uint8, device=DEV)
    dev_buf.copy_(host, non_blocking=True)  # the module in one transfer
    views = banks.module_views(dev_buf, shapes, [m[3].shape[1] for m in mats], torch.float16)
    ids = torch.zeros(T, dtype=torch.int32, device=DEV)
    for (w, wb_dev, signs, scales), (sv, cv), (d_out, _) in zip(mats, views, shapes):
        x = S.dev_x(w, 0)
        y_ref = B.apply(x, wb_dev, signs, scales, p, ids, check=True)
        y = B.apply(x, wb_dev, sv.view(1, d_out, d_in // 64), cv.view(1, -1), p, ids, check=True)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref)
        words, _ = oracle_bank(w, 0, S.host_wbase(w, 0), p, [0])
        assert np.array_equal(to_np(sv), words[0])
    assert all(o[0] % 256 == 0 and o[1] % 256 == 0 for o in offs)
