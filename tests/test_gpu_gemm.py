"""GPU parity of the shared base product for batches above the decode range
(the tiled matrix-core GEMM): bd_base_gemm against a binary64 product of the
same bf16 inputs, over shapes with ragged token counts, row counts that are not
multiples of the 256-row tile, K from one 64-column stage up, and a batch past
one token tile, and every tile shape (the dispatch takes the largest of 256 x 256
(8 waves), 128 x 256, 128 x 128, 64 x 128 and 64 x 64 that yields about 200 blocks).  Accumulation is fp32
over exact bf16 products, so the bound is the fp32 one (max |err| <= 1e-4 * rms)."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, TOL_F32, custom, max_err_vs_rms
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

pytestmark = pytest.mark.gpu

SHAPES = [  # (T, d_out, d_in)
    (65, 300, 64),
    (128, 256, 640),
    (200, 1000, 1024),
    (257, 520, 2048),
    (1144, 384, 5120),
    (512, 1024, 512),    # 64 x 64 tiles
    (512, 4096, 256),    # 64 x 128
    (256, 14336, 128),   # 128 x 128
    (2048, 4096, 128),   # 128 x 256
    (512, 25600, 128),   # 256 x 256, 8 waves
    (700, 25700, 192),   # 256 x 256 with ragged tokens and rows
    (40, 10240, 256),    # 17..64 tokens on a wide matrix: 64 x 64 tiles
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"T{s[0]}-{s[1]}x{s[2]}")
def test_base_gemm_matches_binary64_product(shape):
    T, d_out, d_in = shape
    w = custom(d_out, d_in, S.BF16, n_users=1, T=T, cid=1900 + T + d_out)
    wb_dev = S.dev_wbase(w, 0)
    x_dev = S.dev_x(w, 0)
    y = torch.empty((T, d_out), dtype=torch.float32, device=DEV)
    assert B.bd_base_gemm(x_dev, wb_dev, y) == B.BD_OK
    torch.cuda.synchronize()
    ref = S.as_f32(S.host_x(w, 0), S.BF16).astype(np.float64) @ \
        S.as_f32(S.host_wbase(w, 0), S.BF16).astype(np.float64).T
    err, rms = max_err_vs_rms(y.cpu().numpy(), ref)
    assert err <= TOL_F32 * rms, (shape, err, rms)
