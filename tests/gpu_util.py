"""Helpers shared by the GPU parity tests (inputs, copies, tolerances)."""
import numpy as np
import torch

import oracle as O
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

DEV = "cuda:0"
TOL_F32 = 1e-4   # max |err| <= TOL * rms(ref) for fp32 activations and weights
TOL_BF16 = 2e-2  # ... for bf16 activations and weights


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int64:
        return t.numpy().view(np.uint64)
    return t.numpy()


def custom(d_out, d_in, dtype=S.BF16, n_users=1, T=4, b=5e-4, outlier_p=0.0, cid=1000, seed=0):
    return S.Workload(cid, "custom", dtype, n_users, T, 128, 0.0, b, outlier_p, "custom",
                      [S.Matrix("m", d_out, d_in, S.MATRIX, S.S_F32, 0)], [d_in], seed)


def o_sdtype(p):
    return O.F16 if p.scale_dtype == B.BD_F16 else O.F32


def rel_err_ok(got: np.ndarray, want: np.ndarray, rel: float = 1e-6) -> bool:
    got = got.astype(np.float64)
    want = want.astype(np.float64)
    return bool(np.all(np.abs(got - want) <= rel * np.abs(want)))


def scales_as_f64(a: np.ndarray, p) -> np.ndarray:
    if p.scale_dtype == B.BD_F16:
        return a.view(np.float16).astype(np.float64)
    return a.astype(np.float64)


def max_err_vs_rms(got: np.ndarray, ref: np.ndarray):
    err = np.abs(got.astype(np.float64) - ref).max()
    rms = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2)))
    return float(err), rms


def gpu_bank(w: S.Workload, m: int, wbase_dev, p, users):
    """Compress each listed user's fine-tuned weight on the GPU into a bank."""
    mat = w.matrices[m]
    n_sc = B.bd_scales_count(p, mat.d_out, mat.d_in)
    signs = torch.empty((len(users), mat.d_out, mat.d_in // 64), dtype=torch.int64, device=DEV)
    scales = torch.empty((len(users), n_sc), dtype=B.scales_dtype(p), device=DEV)
    ws = B.workspace(B.bd_compress_workspace_bytes(p, mat.d_out, mat.d_in), DEV)
    wf = torch.empty_like(wbase_dev)
    for j, u in enumerate(users):
        S.dev_wfine(w, m, u, wbase_dev, out=wf)
        B.compress(wf, wbase_dev, p, signs_out=signs[j], scales_out=scales[j], ws=ws, check=True)
    return signs, scales


def oracle_bank(w: S.Workload, m: int, wbase_np, p, users):
    mat = w.matrices[m]
    words, scs = [], []
    for u in users:
        wf = S.host_wfine(w, m, u, wbase=wbase_np)
        ww, ss, _, bad = O.compress(wf, wbase_np, p.mode, g=p.group_size, clip_k=p.clip_k,
                                    sdtype=o_sdtype(p), dtype=w.dtype)
        assert bad == 0
        words.append(ww)
        scs.append(ss)
    return np.stack(words), np.stack(scs)
