"""GPU checks of the paged banks: a module of two matrices for five users, three device
slots fed from the pinned host store, requests that evict and reload users.  For each
request and matrix, bd_apply_paged (through the pager) must equal
- bit for bit, bd_apply on dense banks copied out of the pool's slots with the tokens'
  slot ids (the strided slot addressing reads the same bytes);
- bit for bit, bd_apply on the never-evicted dense banks of all five users (GROUP:
  within one rounding, see below);
- the oracle: each slot's signs equal the oracle's words of the user it holds, and y
  and the delta term alone are within the bf16 bars.
Many-token and decode batches, every scale mode.  A token whose user is not resident
gets the base product only and sets BD_ERR_USER_ID."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (DEV, TOL_BF16, custom, gpu_bank, max_err_vs_rms, o_sdtype, oracle_bank,
                      to_np, tol_delta)
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S
from tenant_serving_amd.pager import BankPager

pytestmark = pytest.mark.gpu

SHAPES = [(136, 1024), (200, 1152)]


def _setup(mode, sd, T, U=5):
    p = B.params(mode, 128, 0.0, sd)
    ws_ = [custom(o, i, S.BF16, n_users=U, T=T, b=5e-3, cid=2800 + o) for o, i in SHAPES]
    bases = [S.dev_wbase(w, 0) for w in ws_]
    dense = [gpu_bank(w, 0, wb, p, range(U)) for w, wb in zip(ws_, bases)]
    counts = [B.bd_scales_count(p, o, i) for o, i in SHAPES]
    pager = BankPager(SHAPES, counts, B.scales_dtype(p), n_slots=3, n_users=U, device=DEV)
    for u in range(U):
        pager.pack(u, [d[0][u] for d in dense], [d[1][u] for d in dense])
    return p, ws_, bases, dense, pager


def _slot_banks(pager, j, p):
    """Dense [n_slots] banks copied out of the pool's slots of matrix j."""
    d_out, d_in = SHAPES[j]
    s_off, c_off = pager.offs[j]
    n_sc = pager.scale_counts[j]
    esz = 2 if p.scale_dtype == B.BD_F16 else 4
    sg, sc = [], []
    for k in range(pager.n_slots):
        a = k * pager.slot_bytes
        sg.append(pager.pool[a + s_off:a + s_off + d_out * d_in // 8].view(torch.int64)
                  .view(d_out, d_in // 64))
        sc.append(pager.pool[a + c_off:a + c_off + n_sc * esz].view(B.scales_dtype(p)))
    return torch.stack(sg).contiguous(), torch.stack(sc).contiguous()


REQUESTS = [[0, 1, 2], [3, 4, 0], [1, 2], [4, 2, 3]]


@pytest.mark.parametrize("T", [40, 9])
@pytest.mark.parametrize("mode,sd", [("matrix", B.BD_F32), ("row", B.BD_F16),
                                     ("group", B.BD_F32), ("col", B.BD_F16)])
def test_paged_apply_through_evictions(mode, sd, T):
    if mode == "group" and T == 9:
        pytest.skip("GROUP batches take the many-token path at any size")
    p, ws_, bases, dense, pager = _setup(mode, sd, T)
    rng = np.random.default_rng(T + len(mode))
    oracle_banks = [oracle_bank(w, 0, S.host_wbase(w, 0), p, range(5)) for w in ws_]
    loads = []
    for r, users in enumerate(REQUESTS):
        ids = np.concatenate([users, rng.choice(users, size=T - len(users) - 1), [-1]])
        ids = rng.permutation(ids).astype(np.int32)  # every user of the request, one -1
        loads.append(pager.ensure(ids))
        ids_dev = torch.from_numpy(ids).to(DEV)
        slot_ids = np.array([pager.slot_of(int(u)) if u >= 0 else -1 for u in ids], np.int32)
        assert np.all(slot_ids[ids >= 0] >= 0)
        for j, w in enumerate(ws_):
            x_dev = S.dev_x(w, 0)
            y = pager.apply(j, x_dev, bases[j], p, ids_dev, check=True)
            sgs, scs = _slot_banks(pager, j, p)
            y_slots = B.apply(x_dev, bases[j], sgs, scs, p, torch.from_numpy(slot_ids).to(DEV))
            y_dense = B.apply(x_dev, bases[j], dense[j][0], dense[j][1], p, ids_dev)
            torch.cuda.synchronize()
            assert torch.equal(y, y_slots), (r, j, "slot addressing")
            if mode != "group":
                assert torch.equal(y, y_dense), (r, j, "never-evicted banks")
            else:
                # GROUP scales every product of a 16-token tile by the row's group scale,
                # including the 2^-127-scaled products of the tile's other users' tokens;
                # which users share a tile follows the order of the ids (slot ids here,
                # user ids there), and such a tiny term can decide the rounding tie of a
                # token's first scaled sum: one rounding, carried through the sums
                d = (y - y_dense).abs().max().item()
                assert d <= 2.0 ** -20 * y.abs().max().item(), (r, j, d)
            # the slots' contents against the oracle, and y against the oracle
            words, osc = oracle_banks[j]
            for u in set(int(v) for v in ids if v >= 0):
                k = pager.slot_of(u)
                assert np.array_equal(to_np(sgs[k]), words[u]), (r, j, u)
            yr, _, yd = O.apply(S.host_x(w, 0), S.host_wbase(w, 0), words, osc, p.mode, ids,
                                g=128, sdtype=o_sdtype(p))
            err, rms = max_err_vs_rms(y.cpu().numpy(), yr)
            assert err <= TOL_BF16 * rms, (r, j, err, rms)
            y0 = pager.apply(j, x_dev, torch.zeros_like(bases[j]), p, ids_dev, check=True)
            err0, rms0 = max_err_vs_rms(y0.cpu().numpy(), yd)
            assert err0 <= tol_delta(mode) * rms0, (r, j, err0, rms0)
    # [3, 4, 0]: 0 hits, 3 and 4 take 1's and 2's slots; [1, 2] take 0's and 3's;
    # [4, 2, 3]: 4 and 2 hit, 3 takes 1's
    assert loads == [3, 2, 2, 1]
    assert pager.loads == 8


def test_token_of_a_user_without_a_slot_gets_the_base_product():
    p, ws_, bases, dense, pager = _setup("matrix", B.BD_F32, 7)
    pager.ensure([0, 1, 2])
    ids = np.array([0, 3, 1, 2, -1, 3, 0], np.int32)  # user 3 has no slot
    ids_dev = torch.from_numpy(ids).to(DEV)
    x_dev = S.dev_x(ws_[0], 0)
    ws = B.workspace(B.bd_apply_paged_workspace_bytes(p, len(ids), 3, *SHAPES[0], B.BD_BF16,
                                                      B.BD_F32), DEV)
    y = pager.apply(0, x_dev, bases[0], p, ids_dev, ws=ws)
    assert B.bd_device_status(ws) == B.BD_ERR_USER_ID
    y_ref = B.apply(x_dev, bases[0], dense[0][0], dense[0][1], p,
                    torch.from_numpy(np.where(ids == 3, -1, ids).astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
