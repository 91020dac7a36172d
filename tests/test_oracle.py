"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check is a printed worked
example, a library routine (numpy packbits / mean / std / clip / float16 /
matmul), a brute-force argmin, or a closed special case.  A dropped term, a
wrong sign, a wrong axis or a wrong ddof fails at least one of them.
"""
import numpy as np
import pytest

import oracle as O


def rel(a, b):
    return abs(a - b) / abs(b)


# ------------------------------------------------------------ worked examples

def test_worked_delta(golden):
    g = golden["delta"]
    wb = np.array([g["base_weight"]], dtype=np.float32)
    wf = np.array([g["fine_tuned_weight"]], dtype=np.float32)
    d = O.delta(wf, wb)
    for got, want in zip(d[0], g["delta"]):
        assert rel(float(got), want) <= 1e-6


def test_worked_group_scale_g4(golden):
    g = golden["group_scale"]
    dc = np.array([g["delta_group"]], dtype=np.float64)
    s = O.absmean_scales(dc, O.GROUP, g=4)
    assert rel(float(s[0]), g["scale"]) <= 1e-6


def test_worked_group_scale_tiled_g128(golden):
    # the printed group tiled 32x fills one 128-element group: same absmean
    g = golden["group_scale"]
    dc = np.tile(np.array(g["delta_group"], dtype=np.float32), 32)[None, :].astype(np.float64)
    s = O.absmean_scales(dc, O.GROUP, g=128)
    assert s.shape == (1,)
    assert rel(float(s[0]), g["scale"]) <= 1e-6
    s2 = golden["second_group_derived"]
    dc2 = np.tile(np.array(s2["delta_group"], dtype=np.float32), 32)[None, :].astype(np.float64)
    assert rel(float(O.absmean_scales(dc2, O.GROUP, g=128)[0]), s2["scale"]) <= 1e-6


def test_worked_signs_and_packing(golden):
    for case in golden["signs"]["cases"]:
        grp = np.array(case["delta_group"], dtype=np.float64)
        words = O.pack_signs(np.tile(grp, 16)[None, :])
        # bit k of the word is column k, 1 <-> +1; the 4-pattern repeats 16x
        expect = 0
        for k in range(64):
            if case["signs"][k % 4] > 0:
                expect |= 1 << k
        assert int(words[0, 0]) == expect
    # the two printed cases as words
    all_pos = O.pack_signs(np.tile([0.2, 0.2, 0.1, 0.3], 16)[None, :])
    alt = O.pack_signs(np.tile([0.2, -0.1, 0.1, -0.3], 16)[None, :])
    assert int(all_pos[0, 0]) == 0xFFFFFFFFFFFFFFFF
    assert int(alt[0, 0]) == 0x5555555555555555


def test_worked_reconstruction(golden):
    r = golden["reconstruction"]
    grp = np.tile(np.array([0.2, 0.2, 0.1, 0.3], dtype=np.float32), 32)[None, :]
    words, scales, _, _ = O.compress(grp, None, O.GROUP, g=128)
    rec = O.reconstruct(words, scales, O.GROUP, 1, 128, g=128)
    assert np.allclose(rec[0, :4], r["reconstructed"], rtol=1e-6, atol=0)
    s2 = golden["second_group_derived"]
    grp2 = np.tile(np.array(s2["delta_group"], dtype=np.float32), 32)[None, :]
    words2, scales2, _, _ = O.compress(grp2, None, O.GROUP, g=128)
    rec2 = O.reconstruct(words2, scales2, O.GROUP, 1, 128, g=128)
    assert np.allclose(rec2[0, :4], s2["reconstructed"], rtol=1e-6, atol=0)


# ------------------------------------------------------- library cross-checks

def test_pack_matches_numpy_packbits():
    rng = np.random.default_rng(1)
    d = rng.standard_normal((7, 320))
    d[rng.random(d.shape) < 0.1] = 0.0
    d[0, :5] = -0.0
    words = O.pack_signs(d)
    bits = ~(d < 0)
    ref = np.packbits(bits, axis=1, bitorder="little").view("<u8")
    assert np.array_equal(words, ref)


def test_sign_of_zero_is_plus_one():
    d = np.zeros((1, 64))
    d[0, 1] = -0.0
    d[0, 2] = -1e-300
    d[0, 3] = 1e-300
    w = int(O.pack_signs(d)[0, 0])
    assert w & 1 and (w >> 1) & 1, "+0 and -0 must map to +1"
    assert not (w >> 2) & 1
    assert (w >> 3) & 1


def test_clip_stats_match_numpy_sample_std():
    rng = np.random.default_rng(2)
    d = (rng.laplace(0, 5e-4, 20000)).astype(np.float32)
    d[rng.choice(d.size, 20, replace=False)] = 0.035
    mu, sigma, lo, hi = O.clip_stats(d, 3.0)
    d64 = d.astype(np.float64)
    assert rel(mu, d64.mean()) <= 1e-9
    assert rel(sigma, d64.std(ddof=1)) <= 1e-12
    assert rel(lo, d64.mean() - 3 * d64.std(ddof=1)) <= 1e-12
    assert rel(hi, d64.mean() + 3 * d64.std(ddof=1)) <= 1e-12
    dc = O.clamp(d, True, lo, hi)
    assert np.allclose(dc, np.clip(d64, lo, hi), rtol=0, atol=1e-18)
    assert (np.abs(dc - mu) <= 3 * sigma * (1 + 1e-12)).all()


def test_clip_is_sensitive_to_ddof():
    # few elements and k=1 clip many values: an (n) instead of (n-1) std moves
    # every clipped value by sqrt(19/20) of sigma
    d = np.array([0.3, -1.2, 0.8, 2.5, -0.4, 0.0, 1.1, -2.2, 0.6, -0.9,
                  1.7, -0.1, 0.2, -1.6, 0.9, 3.1, -0.7, 0.4, -2.9, 1.3], dtype=np.float32)
    words, scales, st, _ = O.compress(np.tile(d, 4)[None, :64], None, O.MATRIX, clip_k=1.0)
    x = np.tile(d, 4)[:64].astype(np.float64)
    lo, hi = x.mean() - x.std(ddof=1), x.mean() + x.std(ddof=1)
    assert rel(st[2], lo) <= 1e-12 and rel(st[3], hi) <= 1e-12
    assert rel(float(scales[0]), float(np.float32(np.abs(np.clip(x, lo, hi)).mean()))) <= 1e-6


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(3)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-9, 5, 3000))
    # ties at every binade, subnormal grid, limits
    vals += [1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -24 * 0.5, 2 ** -24 * 1.5, 2 ** -14 * (1 - 2 ** -12),
             65504.0, 65519.99, 65520.0, 1e-30, 0.0, -0.0, 5.96e-8, 6.1e-5, 1.0, -3.0e-4]
    for v in vals:
        assert O.f64_to_f16(v) == int(np.array(v, dtype=np.float64).astype(np.float16).view(np.uint16)), v
    for h in [0, 1, 0x3C00, 0x7BFF, 0x0400, 0x8001, 0xBC00, 0x03FF]:
        assert O.f16_to_f64(h) == float(np.array(h, dtype=np.uint16).view(np.float16))


# ----------------------------------------------------- closed form / argmin

@pytest.mark.parametrize("mode", [O.MATRIX, O.GROUP, O.ROW, O.COL])
def test_absmean_is_the_l2_argmin(mode):
    # the pages derive alpha = mean|delta| as the minimiser of
    # ||delta - alpha Sign(delta)||_F^2; check it by brute force per unit
    rng = np.random.default_rng(10 + mode)
    d_out, d_in, g = 3, 128, 64
    d = rng.laplace(0, 1.0, (d_out, d_in))
    d[0, :7] = 0.0
    d[:, 5] *= 4.0  # a heavy column, so row and column units differ
    s = O.absmean_scales(d, mode, g=g).astype(np.float64)
    sg = np.where(d < 0, -1.0, 1.0)
    if mode == O.MATRIX:
        units = [(np.s_[:, :], 0)]
    elif mode == O.GROUP:
        units = [(np.s_[o, j * g:(j + 1) * g], o * (d_in // g) + j) for o in range(d_out)
                 for j in range(d_in // g)]
    elif mode == O.ROW:
        units = [(np.s_[o, :], o) for o in range(d_out)]
    else:
        units = [(np.s_[:, i], i) for i in range(d_in)]
    assert len(s) == len(units)
    for sl, idx in units:
        a, b = d[sl], sg[sl]
        grid = np.linspace(0.0, 2.0 * np.abs(a).max() + 1e-12, 20001)
        f = ((a[None, ...] - grid.reshape((-1,) + (1,) * a.ndim) * b[None, ...]) ** 2)
        f = f.reshape(len(grid), -1).sum(1)
        best = grid[int(np.argmin(f))]
        step = grid[1] - grid[0]
        assert abs(best - s[idx]) <= step * 1.01 + 1e-7 * s[idx]


# ------------------------------------------------------------ special cases

def test_all_zero_delta():
    wb = np.random.default_rng(4).standard_normal((4, 128)).astype(np.float32)
    words, scales, _, _ = O.compress(wb.copy(), wb, O.GROUP, g=64)
    assert (words == np.uint64(0xFFFFFFFFFFFFFFFF)).all()
    assert (scales == 0).all()
    x = np.random.default_rng(5).standard_normal((3, 128)).astype(np.float32)
    y, yb, yd = O.apply(x, wb, words[None], scales[None], O.GROUP, np.zeros(3, np.int32), g=64)
    assert np.allclose(y, x.astype(np.float64) @ wb.astype(np.float64).T, rtol=1e-12, atol=1e-12)
    assert (yd == 0).all()


def _exact_case(mode, d_out=6, d_in=128, g=64, seed=7):
    """W_fine = W_base + s*S with power-of-two s and coarse W_base values, so
    delta and scales are exact and the apply reduces to numpy matmul."""
    rng = np.random.default_rng(seed)
    wb = (rng.integers(-512, 512, (d_out, d_in)) / 1024.0).astype(np.float32)
    S = np.where(rng.random((d_out, d_in)) < 0.5, -1.0, 1.0)
    if mode == O.MATRIX:
        s_full = np.full((d_out, d_in), 2.0 ** -6)
    elif mode == O.GROUP:
        sg = 2.0 ** -rng.integers(4, 9, (d_out, d_in // g))
        s_full = np.repeat(sg, g, axis=1)
    elif mode == O.ROW:
        s_full = np.repeat(2.0 ** -rng.integers(4, 9, (d_out, 1)), d_in, axis=1)
    else:
        s_full = np.repeat(2.0 ** -rng.integers(4, 9, (1, d_in)), d_out, axis=0)
    wf = (wb + s_full * S).astype(np.float32)
    assert np.array_equal(wf.astype(np.float64) - wb, s_full * S)  # exact by construction
    return wb, wf, S, s_full


@pytest.mark.parametrize("mode", [O.MATRIX, O.GROUP, O.ROW, O.COL])
def test_apply_reduces_to_numpy_matmul(mode):
    wb, wf, S, s_full = _exact_case(mode)
    sd = O.F16 if mode in (O.ROW, O.COL) else O.F32
    words, scales, _, _ = O.compress(wf, wb, mode, g=64, sdtype=sd)
    assert np.array_equal(O.reconstruct(words, scales, mode, *wb.shape, g=64, sdtype=sd), s_full * S)
    x = np.random.default_rng(8).standard_normal((5, wb.shape[1])).astype(np.float32)
    y, yb, yd = O.apply(x, wb, words[None], scales[None], mode, np.zeros(5, np.int32), g=64, sdtype=sd)
    x64 = x.astype(np.float64)
    ref = x64 @ (wb.astype(np.float64) + s_full * S).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(yb, x64 @ wb.astype(np.float64).T, rtol=1e-12, atol=1e-12)
    assert np.allclose(yd, x64 @ (s_full * S).T, rtol=1e-12, atol=1e-12)


def test_apply_routes_each_token_to_its_user():
    d_out, d_in = 4, 128
    cases = [_exact_case(O.MATRIX, d_out, d_in, seed=20 + u) for u in range(3)]
    wb = cases[0][0]
    banks, scs = [], []
    for u in range(3):
        _, wf_u, S_u, s_u = cases[u]
        wf = (wb + s_u * S_u).astype(np.float32)
        w, s, _, _ = O.compress(wf, wb, O.MATRIX)
        banks.append(w)
        scs.append(s)
    ids = np.array([2, -1, 0, 1, 7, 0], dtype=np.int32)  # 7 is out of range: base only
    x = np.random.default_rng(9).standard_normal((len(ids), d_in)).astype(np.float32)
    y, yb, yd = O.apply(x, wb, np.stack(banks), np.stack(scs), O.MATRIX, ids)
    for t, u in enumerate(ids):
        w_eff = wb.astype(np.float64)
        if 0 <= u < 3:
            w_eff = w_eff + cases[u][3] * cases[u][2]
        assert np.allclose(y[t], x[t].astype(np.float64) @ w_eff.T, rtol=1e-12, atol=1e-12)


def test_delta_only_when_base_is_zero():
    wb, wf, S, s_full = _exact_case(O.GROUP)
    z = np.zeros_like(wb)
    words, scales, _, _ = O.compress((s_full * S).astype(np.float32), z, O.GROUP, g=64)
    x = np.random.default_rng(11).standard_normal((2, wb.shape[1])).astype(np.float32)
    y, yb, yd = O.apply(x, z, words[None], scales[None], O.GROUP, np.zeros(2, np.int32), g=64)
    assert (yb == 0).all()
    assert np.allclose(y, x.astype(np.float64) @ (s_full * S).T, rtol=1e-12, atol=1e-12)


def test_bf16_inputs_widen_exactly():
    rng = np.random.default_rng(12)
    f = rng.standard_normal((2, 64)).astype(np.float32)
    bf = (f.view(np.uint32) >> 16).astype(np.uint16)
    wide = (bf.astype(np.uint32) << 16).view(np.float32)
    d = O.delta(bf, np.zeros_like(bf))
    assert np.array_equal(d, wide)


def test_nonfinite_deltas_are_counted():
    wf = np.zeros((1, 64), dtype=np.float32)
    wf[0, 3] = np.inf
    wf[0, 9] = np.nan
    _, _, _, bad = O.compress(wf, np.zeros_like(wf), O.MATRIX)
    assert bad == 2


def test_llama8b_scalar_artifact_size(golden):
    # 1 bit per weight of the linear stack, packed in 64-bit words
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096),
              (14336, 4096), (4096, 14336)]
    bits = 32 * sum(o * O.lib().orc_words_per_row(i) * 8 for o, i in shapes)
    assert bits == 872_415_232
    g = golden["llama8b_scalar_artifact"]
    total_mb = (bits + 2 * g["vocab"] * g["hidden"] * 2) / 1e6
    assert round(total_mb) == g["printed_mb"]


# ------------------------------------------------- per-layer axis selection

def _closed_form_axis_errors(wf, wb, clip_k):
    """The errors from per-unit sums only: a unit of n deltas with absmean s has
    sum (|d| - s)^2 = sum d^2 - (sum |d|)^2 / n.  Delta and clipping with numpy."""
    d = wf.astype(np.float32) - wb.astype(np.float32)
    dc = d.astype(np.float64)
    if clip_k > 0:
        mu, sd = dc.mean(), dc.std(ddof=1)
        dc = np.clip(dc, mu - clip_k * sd, mu + clip_k * sd)
    ss = np.sum(dc * dc)
    a = np.abs(dc)
    er = ss - np.sum(a.sum(axis=1) ** 2) / dc.shape[1]
    ec = ss - np.sum(a.sum(axis=0) ** 2) / dc.shape[0]
    return er, ec


@pytest.mark.parametrize("clip_k", [0.0, 3.0])
@pytest.mark.parametrize("shape", [(7, 64), (64, 192), (130, 128)])
def test_axis_errors_match_the_closed_form(shape, clip_k):
    rng = np.random.default_rng(31 + shape[0] + int(clip_k))
    wb = rng.normal(0, 0.02, shape).astype(np.float32)
    d = rng.laplace(0, 1e-3, shape)
    d[rng.random(shape) < 0.01] *= 50  # outliers, so that clipping bites
    wf = (wb + d).astype(np.float32)
    er, ec, axis, bad = O.select_axis(wf, wb, clip_k)
    cer, cec = _closed_form_axis_errors(wf, wb, clip_k)
    assert bad == 0
    assert rel(er, cer) <= 1e-9 and rel(ec, cec) <= 1e-9
    assert axis == (O.ROW if cer <= cec else O.COL)


def test_axis_choice_on_rows_or_columns_of_one_magnitude():
    rng = np.random.default_rng(5)
    sgn = np.where(rng.random((8, 64)) < 0.5, -1.0, 1.0)
    # every row of one magnitude: the row scales reconstruct it exactly
    rows = (sgn * (2.0 ** -np.arange(1, 9))[:, None]).astype(np.float32)
    er, ec, axis, _ = O.select_axis(rows, None)
    assert er == 0.0 and ec > 0.0 and axis == O.ROW
    # every column of one magnitude: the column scales do
    cols = (sgn * (2.0 ** -(np.arange(64) % 9 + 1))[None, :]).astype(np.float32)
    er, ec, axis, _ = O.select_axis(cols, None)
    assert ec == 0.0 and er > 0.0 and axis == O.COL


def test_axis_errors_swap_under_transposition_and_scale_quadratically():
    rng = np.random.default_rng(9)
    d = rng.laplace(0, 1e-3, (24, 128)).astype(np.float32)
    er, ec, _, _ = O.select_axis(d, None)
    er_t, ec_t, _, _ = O.select_axis(np.ascontiguousarray(d.T), None)
    assert rel(er_t, ec) <= 1e-12 and rel(ec_t, er) <= 1e-12
    er2, ec2, _, _ = O.select_axis(d * np.float32(4.0), None)  # exact power-of-two scaling
    assert rel(er2, 16 * er) <= 1e-12 and rel(ec2, 16 * ec) <= 1e-12


# ------------------------------------------------------ INT8 base weights

def test_row_quantizer_matches_numpy_and_its_bounds():
    rng = np.random.default_rng(17)
    w = rng.normal(0, 0.02, (12, 192)).astype(np.float32)
    w[3] = 0.0  # a zero row
    w[5, 7] = -0.5  # a row whose maximum is negative
    q, s = O.quantize_rows(w)
    m = np.abs(w).max(axis=1)
    ns = (m / np.float32(127.0)).astype(np.float32)  # binary32 division, as the reading states
    assert np.array_equal(s, ns)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(ns[:, None] > 0, w / ns[:, None], 0).astype(np.float32)
    assert np.array_equal(q, np.clip(np.rint(v), -127, 127).astype(np.int8))
    assert np.all(q[3] == 0) and s[3] == 0.0 and q[5, 7] == -127
    err = np.abs(w.astype(np.float64) - q * s[:, None].astype(np.float64))
    assert np.all(err <= 0.5 * s[:, None] * (1 + 1e-6) + 1e-30)  # half a step per element


def test_row_quantizer_marks_rows_with_non_finite_weights():
    """A row holding a NaN or an Inf has no INT8 codes: scale NaN, codes 0 (so its base
    outputs are NaN); the other rows are quantized as without it."""
    rng = np.random.default_rng(23)
    w = rng.normal(0, 0.02, (6, 128)).astype(np.float32)
    clean_q, clean_s = O.quantize_rows(w)
    w[1, 5] = np.nan
    w[4, 100] = -np.inf
    q, s = O.quantize_rows(w)
    assert np.isnan(s[1]) and np.isnan(s[4]) and np.all(q[[1, 4]] == 0)
    keep = [0, 2, 3, 5]
    assert np.array_equal(q[keep], clean_q[keep]) and np.array_equal(s[keep], clean_s[keep])
    words = np.zeros((1, 6, 2), np.uint64)
    _, yb, _ = O.apply_q8(np.ones((1, 128), np.float32), q, s, words, np.zeros((1, 1), np.float32),
                          O.MATRIX, np.array([-1], np.int32))
    assert np.all(np.isnan(yb[0, [1, 4]])) and np.all(np.isfinite(yb[0, keep]))


def test_apply_on_int8_base_reduces_to_numpy_matmul():
    rng = np.random.default_rng(19)
    T, d_out, d_in, U = 5, 24, 128, 3
    x = rng.normal(0, 1, (T, d_in)).astype(np.float32)
    wb = rng.normal(0, 0.02, (d_out, d_in)).astype(np.float32)
    q, s = O.quantize_rows(wb)
    d = rng.laplace(0, 1e-3, (U, d_out, d_in))
    words = np.stack([O.pack_signs(d[u]) for u in range(U)])
    scales = np.stack([O.absmean_scales(d[u], O.ROW) for u in range(U)])
    ids = np.array([2, 0, -1, 1, 2], dtype=np.int32)
    y, yb, yd = O.apply_q8(x, q, s, words, scales, O.ROW, ids)
    deq = q.astype(np.float64) * s[:, None].astype(np.float64)
    assert np.allclose(yb, x.astype(np.float64) @ deq.T, rtol=1e-12, atol=1e-15)
    _, _, yd_ref = O.apply(x, np.zeros((d_out, d_in), np.float32), words, scales, O.ROW, ids)
    assert np.allclose(yd, yd_ref, rtol=1e-12, atol=1e-15)
    assert np.allclose(y, yb + yd, rtol=1e-15, atol=0)
