"""bd_apply_noalloc (no workspace, no allocation: the library's per-device scratch)
against bd_apply on a fresh workspace: two calls in a row, the second with a smaller
input, give bit for bit the same y and the same status word; a call whose workspace
would exceed the scratch is refused and enqueues nothing."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, custom, gpu_bank
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 8 << 20  # BD_NOALLOC_SCRATCH_BYTES


def _case(T, U, d_out, d_in, mode, cid, bad_id=False):
    p = B.params(mode)
    w = custom(d_out, d_in, S.BF16, n_users=U, T=T, b=5e-3, cid=cid)
    wb = S.dev_wbase(w, 0)
    signs, scales = gpu_bank(w, 0, wb, p, list(range(U)))
    ids = np.array([(5 * t) % (U + 1) - 1 for t in range(T)], dtype=np.int32)
    if bad_id:
        ids[T // 2] = U + 3  # outside [0, n_users): base term only, status bit 1
    return p, S.dev_x(w, 0), wb, signs, scales, torch.from_numpy(ids).to(DEV)


def _reference(p, x, wb, signs, scales, ids, U, y_dtype):
    T, d_in = x.shape
    d_out = wb.shape[0]
    y = torch.empty((T, d_out), dtype=y_dtype, device=DEV)
    yd = B.BD_F32 if y_dtype == torch.float32 else B.BD_BF16
    ws = B.workspace(B.bd_apply_workspace_bytes(p, T, U, d_out, d_in, B.BD_BF16, yd), DEV)
    assert B.bd_apply(x, wb, signs, scales, p, U, ids, y, ws) == B.BD_OK
    return y, B.bd_device_status(ws)


def _status_code(word: int) -> int:  # the word as bd_device_status reads it
    return B.BD_ERR_NONFINITE if word & 1 else B.BD_ERR_USER_ID if word & 2 else \
        B.BD_ERR_BATCH if word & 4 else B.BD_OK


def test_noalloc_equals_bd_apply_on_two_calls_in_a_row():
    U = 5
    # a prepared-batch call (40 tokens, bf16 y), then a smaller decode call (9 tokens)
    cases = [(40, 300, 1152, "matrix", torch.bfloat16, False, 3100),
             (9, 200, 1024, "row", torch.float32, True, 3101)]
    for T, d_out, d_in, mode, y_dtype, bad, cid in cases:
        p, x, wb, signs, scales, ids = _case(T, U, d_out, d_in, mode, cid, bad)
        y_ref, st_ref = _reference(p, x, wb, signs, scales, ids, U, y_dtype)
        y = torch.full((T, d_out), float("nan"), dtype=y_dtype, device=DEV)
        status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        assert B.bd_apply_noalloc(x, wb, signs, scales, p, U, ids, y, status) == B.BD_OK
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16) if y_dtype == torch.bfloat16 else y,
                           y_ref.view(torch.int16) if y_dtype == torch.bfloat16 else y_ref)
        assert _status_code(int(status.item())) == st_ref
        assert st_ref == (B.BD_ERR_USER_ID if bad else B.BD_OK)


def test_noalloc_refuses_a_call_beyond_the_scratch():
    U, T, d_out, d_in = 4, 2048, 512, 4096
    p = B.params("matrix")
    need = B.bd_apply_workspace_bytes(p, T, U, d_out, d_in, B.BD_BF16, B.BD_F32)
    assert need > SCRATCH_BYTES
    x = torch.zeros((T, d_in), dtype=torch.bfloat16, device=DEV)
    wb = torch.zeros((d_out, d_in), dtype=torch.bfloat16, device=DEV)
    signs = torch.zeros((U, d_out, d_in // 64), dtype=torch.int64, device=DEV)
    scales = torch.ones((U, 1), dtype=torch.float32, device=DEV)
    ids = torch.zeros(T, dtype=torch.int32, device=DEV)
    y = torch.full((T, d_out), 7.0, device=DEV)
    assert B.bd_apply_noalloc(x, wb, signs, scales, p, U, ids, y) == B.BD_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
