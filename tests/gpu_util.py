"""Helpers shared by the GPU parity tests (inputs, copies, tolerances)."""
import numpy as np
import torch

import oracle as O
from tenant_serving_amd import bitdelta as B
from tenant_serving_amd import synth as S

DEV = "cuda:0"
TOL_F32 = 1e-4   # max |err| <= TOL * rms(ref) for fp32 activations and weights
TOL_BF16 = 2e-2  # ... for bf16 activations and weights
# The delta term alone (bf16 activations): the tokens enter the products as an fp6 hi part
# plus an fp6 lo residual under one power-of-two scale per 32 columns, which hold each
# value within 2^(E-10), 2^E <= the block's largest |x| (see delta_error_bound); on
# Gaussian tokens the seeded cases measure max|err| / rms <= 4.2e-3.  COL scales are
# multiplied into the tokens first and rounded to bf16 (one more rounding, 2^-8
# relative): measured <= 6.8e-3.
TOL_DELTA = 5e-3
TOL_DELTA_COL = 1e-2


def tol_delta(mode) -> float:
    """The delta-only bar of a scale mode (B.BD_SCALE_* or its name)."""
    return TOL_DELTA_COL if mode in (3, "col") else TOL_DELTA


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


def oracle_rows_bank(w: S.Workload, m: int, p, users, rows):
    """The oracle's banks of `users`, restricted to the output rows `rows`, composed
    from the oracle's compression steps (delta, clip statistics, clamp, sign packing,
    absmean) so that each step reads only what its definition needs: the signs and the
    ROW and GROUP scales of a row read that row alone, the clip bounds and the MATRIX
    and COL scales read the whole matrix.  Equal to the rows of O.compress (a CPU test
    checks that in every mode, with and without clipping); returns
    (words [len(users)][len(rows)][wpr], scales [len(users)][scales of those rows])."""
    mat = w.matrices[m]
    clip = p.clip_k > 0.0
    whole = clip or p.mode in (B.BD_SCALE_MATRIX, B.BD_SCALE_COL)
    wb_rows = S.host_wbase(w, m, rows)
    wb_all = S.host_wbase(w, m) if whole else None
    words, scs = [], []
    for u in users:
        d_rows = O.delta(S.host_wfine(w, m, u, rows=rows, wbase=wb_rows), wb_rows, dtype=w.dtype)
        lo = hi = 0.0
        d_all = None
        if whole:
            d_all = O.delta(S.host_wfine(w, m, u, wbase=wb_all), wb_all, dtype=w.dtype)
            assert np.all(np.isfinite(d_all))
            if clip:
                _, _, lo, hi = O.clip_stats(d_all, p.clip_k)
        dc_rows = O.clamp(d_rows, clip, lo, hi)
        words.append(O.pack_signs(dc_rows))
        if p.mode in (B.BD_SCALE_ROW, B.BD_SCALE_GROUP):
            scs.append(O.absmean_scales(dc_rows, p.mode, p.group_size, o_sdtype(p)))
        else:
            scs.append(O.absmean_scales(O.clamp(d_all, clip, lo, hi), p.mode, p.group_size,
                                        o_sdtype(p)))
        del d_all
    return np.stack(words), np.stack(scs)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def delta_error_bound(x_bits: np.ndarray, scales_bank: np.ndarray, p, ids: np.ndarray,
                      n_rows: int, hoeffding_k: float = 0.0) -> np.ndarray:
    """Element-wise bound [T][n_rows] on |delta term (GPU) - delta term (oracle)| for bf16
    tokens x_bits [T][d_in] (bf16 bit patterns) and the oracle's scales of the same rows.

    The delta products take each token in blocks of 32 columns: with 2^E <= the block's
    largest |x| < 2^(E+1) and s = 2^(E-1), hi = fp6 e2m3(x / s) and lo = fp6 e2m3((x -
    hi) / (s / 32)), both rounded to nearest.  A bf16 value |x| >= s has at most 4
    significant bits left after hi, which lo holds exactly; below s the residual is under
    2 lo units, where the lo grid is 1/8 unit, so |x - hi - lo| <= a = s / 512 = 2^(E-10).
    COL scales are multiplied into the tokens before the encoding and rounded to bf16
    (2^-8 relative): x' = bf16(c x), |x'| <= (1 + 2^-8) |c x|, a = 2^-8 |c x| + 2^-10
    (1 + 2^-8) max_block |c x|.  The bound is sum_i |f_u(r, i)| a_i (f the scale of
    element (r, i) of the token's user u; 1 for COL), or with hoeffding_k > 0
    k sqrt(sum_i f^2 a^2): Hoeffding's inequality for independent zero-mean rounding
    errors |e_i| <= a_i, exceeded with probability at most 2 exp(-k^2 / 2) per element;
    either plus 2^-15 sum_i |f x| for the fp32 sums of the products and their scaling."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    T, d_in = x_bits.shape
    nb = (d_in + 31) // 32
    pad = nb * 32 - d_in
    xa = np.abs(bf16_to_f64(x_bits))
    sq = hoeffding_k > 0
    bound = np.zeros((T, n_rows), dtype=np.float64)
    for u in sorted(set(int(v) for v in ids if v >= 0)):
        tk = np.nonzero(ids == u)[0]
        sc = np.abs(scales_as_f64(np.asarray(scales_bank[u]), p))
        if p.mode == B.BD_SCALE_COL:
            v = xa[tk] * sc[None, :]
            vmax = np.pad(v, ((0, 0), (0, pad))).reshape(len(tk), nb, 32).max(axis=2)
            a = 2.0 ** -8 * v + 2.0 ** -10 * (1 + 2.0 ** -8) * np.repeat(vmax, 32, axis=1)[:, :d_in]
            e = hoeffding_k * np.sqrt((a * a).sum(axis=1)) if sq else a.sum(axis=1)
            bound[tk] = (e + 2.0 ** -15 * v.sum(axis=1))[:, None]
            continue
        if p.mode == B.BD_SCALE_MATRIX:
            F = np.full((n_rows, d_in), sc[0])
        elif p.mode == B.BD_SCALE_ROW:
            F = np.repeat(sc[:n_rows, None], d_in, axis=1)
        else:
            F = np.repeat(sc.reshape(n_rows, d_in // p.group_size), p.group_size, axis=1)
        eb = np.pad(x_bits[tk] & 0x7FFF, ((0, 0), (0, pad))).reshape(len(tk), nb, 32).max(axis=2)
        eb = eb.astype(np.int64) >> 7
        # blocks of zeros and tiny values (below 2^-120) take s = 1 and encode to 0
        P = np.where(eb >= 7, np.ldexp(1.0, eb - 137), np.ldexp(1.0, eb - 126))
        Fp = np.pad(F, ((0, 0), (0, pad))).reshape(n_rows, nb, 32)
        if sq:
            e = hoeffding_k * np.sqrt((P * P) @ (Fp * Fp).sum(axis=2).T)
        else:
            e = P @ Fp.sum(axis=2).T
        bound[tk] = e + 2.0 ** -15 * (xa[tk] @ F.T)
    return bound


def assert_delta_within_bound(got0: np.ndarray, yd: np.ndarray, x_bits: np.ndarray,
                              scales_bank: np.ndarray, p, ids: np.ndarray, what=""):
    """The delta term within the encoding's worst-case bound and within its Hoeffding
    bound at k = 8 (2.5e-14 per element)."""
    err = np.abs(got0.astype(np.float64) - yd)
    for k in (0.0, 8.0):
        excess = err - delta_error_bound(x_bits, scales_bank, p, ids, yd.shape[1], k)
        assert np.all(excess <= 0), (what, k, float(excess.max()),
                                     np.unravel_index(excess.argmax(), excess.shape))
